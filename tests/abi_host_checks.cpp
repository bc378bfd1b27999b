// Host-side argument checks of the C ABI, driven from C++ (no GPU: every call below fails
// validation before any launch, or is a documented no-op).  Built with the host address and
// undefined-behaviour sanitizers by tests/test_abi_sanitizers.py, so a bad read, overflow or
// undefined operation in the validation code stops the run.
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "dsv4.h"

static int failures = 0;
#define EXPECT(cond)                                                              \
    do {                                                                          \
        if (!(cond)) {                                                            \
            std::fprintf(stderr, "FAILED %s:%d: %s\n", __FILE__, __LINE__, #cond); \
            ++failures;                                                           \
        }                                                                         \
    } while (0)

int main() {
    void* fake = reinterpret_cast<void*>(uintptr_t(0x1000));   // never dereferenced
    int64_t zero[4] = {0, 0, 0, 0};
    // compressor
    dsv4_comp_cfg cc{4, 1, 64, 16, 1e-6f, DSV4_BF16, 0};
    EXPECT(dsv4_compress_prefill(nullptr, fake, fake, fake, 1, 4, zero, fake, fake, nullptr, fake, 100, nullptr) == DSV4_EINVAL);
    EXPECT(dsv4_compress_prefill(&cc, fake, fake, fake, 1, -1, zero, fake, fake, nullptr, fake, 100, nullptr) == DSV4_EINVAL);
    EXPECT(dsv4_compress_prefill(&cc, fake, fake, fake, 0, 4, zero, fake, fake, nullptr, fake, 100, nullptr) == DSV4_OK);
    int64_t lb_big[1] = {int64_t(1) << 40};
    EXPECT(dsv4_compress_prefill(&cc, fake, fake, fake, 1, 4, lb_big, fake, fake, reinterpret_cast<float*>(fake), fake, 100, nullptr) == DSV4_ECAPACITY);
    EXPECT(dsv4_compress_prefill(&cc, fake, fake, fake, 1, 4000, zero, fake, fake, reinterpret_cast<float*>(fake), fake, 100, nullptr) == DSV4_ECAPACITY);
    dsv4_comp_cfg bad = cc;
    bad.ratio = 0;
    EXPECT(dsv4_comp_state_bytes(&bad, 1) == 0);
    bad = cc;
    bad.rope_dim = 65;
    EXPECT(dsv4_compress_step(&bad, fake, fake, fake, 1, zero, fake, fake, nullptr, fake, 100, nullptr) == DSV4_EINVAL);
    EXPECT(std::strlen(dsv4_last_error()) > 0);
    // indexer
    dsv4_index_cfg ic{64, 128, 512, 4, DSV4_BF16};
    int64_t nr[1] = {1000}, p0[1] = {3999}, nr_small[1] = {10};
    EXPECT(dsv4_index_topk(&ic, fake, reinterpret_cast<float*>(fake), fake, 1000, nr, p0, 1, 1, reinterpret_cast<int32_t*>(fake), fake, 16, nullptr) == DSV4_EWORKSPACE);
    EXPECT(dsv4_index_topk(&ic, fake, reinterpret_cast<float*>(fake), fake, 1000, nr_small, p0, 1, 1, reinterpret_cast<int32_t*>(fake), fake, size_t(1) << 30, nullptr) == DSV4_EINVAL);
    EXPECT(dsv4_index_topk(&ic, fake, reinterpret_cast<float*>(fake), fake, 5, nr, p0, 1, 1, reinterpret_cast<int32_t*>(fake), fake, size_t(1) << 30, nullptr) == DSV4_ECAPACITY);
    dsv4_index_cfg icbad{300, 128, 512, 4, DSV4_BF16};
    EXPECT(dsv4_index_topk(&icbad, fake, reinterpret_cast<float*>(fake), fake, 1000, nr, p0, 1, 1, reinterpret_cast<int32_t*>(fake), fake, size_t(1) << 30, nullptr) == DSV4_EUNSUPPORTED);
    EXPECT(dsv4_index_workspace_bytes(&ic, 4, 1, 65536) > size_t(4) * 65536 * 4);
    // attention
    dsv4_attn_cfg ac{64, 512, 128, 4, 512, 0.044f, DSV4_BF16, 0};
    int64_t pos[1] = {4000}, rows_n[1] = {2000};
    EXPECT(dsv4_csa_attn_decode(&ac, fake, fake, fake, fake, 100, nullptr, rows_n, pos, reinterpret_cast<float*>(fake), fake, 1, fake, size_t(1) << 30, nullptr) == DSV4_ECAPACITY);
    EXPECT(dsv4_csa_attn_decode(&ac, fake, fake, fake, nullptr, 100, nullptr, rows_n, pos, reinterpret_cast<float*>(fake), fake, 1, fake, size_t(1) << 30, nullptr) == DSV4_EINVAL);
    dsv4_attn_cfg acbad = ac;
    acbad.window = 0;
    EXPECT(dsv4_csa_attn_prefill(&acbad, fake, fake, fake, fake, 100, nullptr, rows_n, pos, reinterpret_cast<float*>(fake), fake, 1, 3, fake, 0, nullptr) == DSV4_EINVAL);
    EXPECT(dsv4_csa_attn_prefill(&ac, fake, fake, fake, fake, 100, nullptr, rows_n, pos, reinterpret_cast<float*>(fake), fake, 1, 70000, fake, 0, nullptr) == DSV4_EUNSUPPORTED);
    dsv4_frontier_store st[3] = {};
    EXPECT(dsv4_csa_attn_decode_store(&ac, fake, fake, fake, fake, 3000, nullptr, rows_n, pos, reinterpret_cast<float*>(fake), fake, 1, fake, size_t(1) << 30, st, 3, nullptr) == DSV4_EINVAL);
    // RoPE and the grouped projection
    dsv4_rope_cfg rc{64, 512, 64, 0, DSV4_BF16};
    int64_t neg[1] = {-1};
    EXPECT(dsv4_rope(&rc, fake, neg, 1, 1, reinterpret_cast<float*>(fake), nullptr) == DSV4_EINVAL);
    dsv4_gproj_cfg gc{0, 4096, 1024, DSV4_BF16};
    EXPECT(dsv4_grouped_proj(&gc, fake, fake, fake, 8, nullptr) == DSV4_EINVAL);
    dsv4_gproj_cfg lc{2, 4096, 1024, DSV4_BF16};                       // lanes take one group
    EXPECT(dsv4_lane_proj(&lc, fake, fake, fake, fake, fake, 8, nullptr) == DSV4_EINVAL);
    lc.groups = 1;
    EXPECT(dsv4_lane_proj(&lc, fake, fake, nullptr, fake, fake, 8, nullptr) == DSV4_EINVAL);
    EXPECT(dsv4_lane_proj(&lc, nullptr, nullptr, nullptr, nullptr, nullptr, 0, nullptr) == DSV4_OK);
    // trace bookkeeping
    int64_t n = -1;
    double ms = -1.0;
    EXPECT(dsv4_trace_reset() == DSV4_OK);
    EXPECT(dsv4_trace_read("", &n, &ms) == DSV4_OK && n == 0 && ms == 0.0);
    EXPECT(dsv4_trace_read(nullptr, nullptr, nullptr) == DSV4_EINVAL);
    EXPECT(dsv4_trace_kernel_name(-1) == nullptr);
    if (failures == 0) std::printf("abi host checks: all passed\n");
    return failures == 0 ? 0 : 1;
}
