// C ABI of libdsv4.so: host-side validation, then the launchers in kernels.hpp.
//
// Every entry point checks all of its arguments before enqueuing anything, so a failed
// call leaves every buffer as it was (pages: MTPLX PR #216 "Stage 4" and the 0731 PR: fail
// before generation, no silent fallback; mlx-lm PR #1189: fail loudly on mismatched cache
// state; MTPLX PR #216 speculative-decode comment: raise rather than clamp).
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/dsv4.h"
#include "common.hpp"
#include "kernels.hpp"
#include "proj.hpp"

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

int ok() {
    g_err.clear();
    return DSV4_OK;
}

int hip_status(hipError_t e, const char* what) {
    if (e == hipSuccess) return ok();
    return fail(DSV4_EHIP, "%s: HIP error %d (%s)", what, int(e), hipGetErrorString(e));
}

constexpr int64_t kPosLimit = (int64_t(1) << 31) - 2;   // positions travel as int32

bool dtype_ok(int32_t d) { return d == DSV4_BF16 || d == DSV4_F32; }
size_t dtype_size(int32_t d) { return d == DSV4_BF16 ? 2 : 4; }

// Windows of the frontier state: the coff pooled ones plus those a trim of `retain` tokens
// back can reach.
int64_t state_windows(const dsv4_comp_cfg* c) {
    return (c->overlap ? 2 : 1) + (int64_t(c->retain) + c->ratio - 1) / c->ratio;
}

int check_comp_cfg(const dsv4_comp_cfg* c) {
    if (!c) return fail(DSV4_EINVAL, "cfg is NULL");
    if (c->ratio < 1) return fail(DSV4_EINVAL, "ratio %d < 1", c->ratio);
    if (c->overlap != 0 && c->overlap != 1) return fail(DSV4_EINVAL, "overlap must be 0 or 1");
    if (c->dim < 1 || c->dim > 4096) return fail(DSV4_EINVAL, "dim %d outside 1..4096", c->dim);
    if (c->rope_dim < 0 || c->rope_dim > c->dim || (c->rope_dim & 1))
        return fail(DSV4_EINVAL, "rope_dim %d must be even and within 0..dim", c->rope_dim);
    if (!(c->eps >= 0.f) || !std::isfinite(c->eps)) return fail(DSV4_EINVAL, "eps must be >= 0");
    if (!dtype_ok(c->dtype)) return fail(DSV4_EINVAL, "unknown dtype %d", c->dtype);
    if (c->retain < 0 || c->retain > (1 << 20)) return fail(DSV4_EINVAL, "retain %d outside 0..2^20", c->retain);
    if (int64_t(c->ratio) * state_windows(c) * (c->overlap ? 2 : 1) * 2 * c->dim > (int64_t(1) << 30))
        return fail(DSV4_EUNSUPPORTED, "state per sequence too large");
    return DSV4_OK;
}

int check_index_cfg(const dsv4_index_cfg* c) {
    if (!c) return fail(DSV4_EINVAL, "cfg is NULL");
    if (c->heads < 1 || c->heads > 256) return fail(DSV4_EUNSUPPORTED, "heads %d outside 1..256", c->heads);
    if (c->dim < 1 || c->dim > 1024) return fail(DSV4_EUNSUPPORTED, "dim %d outside 1..1024", c->dim);
    if (int64_t(c->heads) * c->dim > 15360)
        return fail(DSV4_EUNSUPPORTED, "heads*dim %d above 15360", c->heads * c->dim);
    if (c->topk < 1) return fail(DSV4_EINVAL, "topk %d < 1", c->topk);
    if (c->ratio < 1) return fail(DSV4_EINVAL, "ratio %d < 1", c->ratio);
    if (!dtype_ok(c->dtype)) return fail(DSV4_EINVAL, "unknown dtype %d", c->dtype);
    return DSV4_OK;
}

int check_attn_cfg(const dsv4_attn_cfg* c) {
    if (!c) return fail(DSV4_EINVAL, "cfg is NULL");
    if (c->heads < 1 || c->heads > 65535) return fail(DSV4_EINVAL, "heads %d outside 1..65535", c->heads);
    if (c->dim < 1 || c->dim > 4096) return fail(DSV4_EINVAL, "dim %d outside 1..4096", c->dim);
    if (c->window < 1) return fail(DSV4_EINVAL, "window %d < 1", c->window);
    if (c->ratio < 0) return fail(DSV4_EINVAL, "ratio %d < 0", c->ratio);
    if (c->topk < 0) return fail(DSV4_EINVAL, "topk %d < 0", c->topk);
    if (!std::isfinite(c->scale)) return fail(DSV4_EINVAL, "scale is not finite");
    if (!dtype_ok(c->dtype)) return fail(DSV4_EINVAL, "unknown dtype %d", c->dtype);
    if (c->retain < 0 || c->retain > (1 << 20)) return fail(DSV4_EINVAL, "retain %d outside 0..2^20", c->retain);
    return DSV4_OK;
}

// ------------------------------------------------------------------ kernel trace
struct TraceRec {
    const char* name;
    hipEvent_t start, stop;
};
std::atomic<bool> g_trace_on{false};
std::mutex g_trace_mu;
std::vector<TraceRec> g_recs;
std::vector<hipEvent_t> g_event_pool;
std::vector<std::string> g_trace_names;

hipEvent_t take_event() {
    if (!g_event_pool.empty()) {
        hipEvent_t e = g_event_pool.back();
        g_event_pool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}

}  // namespace

namespace dsv4 {

bool trace_events(const char* name, hipEvent_t* start, hipEvent_t* stop) {
    if (!g_trace_on.load(std::memory_order_relaxed)) return false;
    std::lock_guard<std::mutex> lk(g_trace_mu);
    TraceRec r{name, take_event(), take_event()};
    if (!r.start || !r.stop) {                 // no events: launch untraced, keep the pool
        if (r.start) g_event_pool.push_back(r.start);
        if (r.stop) g_event_pool.push_back(r.stop);
        return false;
    }
    g_recs.push_back(r);
    bool known = false;
    for (auto& n : g_trace_names) known |= (n == name);
    if (!known) g_trace_names.emplace_back(name);
    *start = r.start;
    *stop = r.stop;
    return true;
}

}  // namespace dsv4

extern "C" {

const char* dsv4_version(void) { return "dsv4-csa 0.1 (gfx950)"; }

const char* dsv4_last_error(void) { return g_err.c_str(); }

size_t dsv4_comp_state_bytes(const dsv4_comp_cfg* cfg, int32_t batch) {
    if (check_comp_cfg(cfg) != DSV4_OK || batch < 0) return 0;
    const int coff = cfg->overlap ? 2 : 1;
    return size_t(batch) * 2 * size_t(state_windows(cfg)) * size_t(cfg->ratio) * coff * cfg->dim *
           dtype_size(cfg->dtype);
}

size_t dsv4_index_workspace_bytes(const dsv4_index_cfg* cfg, int32_t batch, int64_t s,
                                  int64_t n_max) {
    if (check_index_cfg(cfg) != DSV4_OK || batch < 0 || s < 0 || n_max < 0) return 0;
    return dsv4::index_workspace_bytes(cfg->heads, cfg->dim, cfg->topk, batch, s, n_max);
}

size_t dsv4_attn_workspace_bytes(const dsv4_attn_cfg* cfg, int32_t batch, int64_t s) {
    if (check_attn_cfg(cfg) != DSV4_OK || batch < 0 || s < 0) return 0;
    return dsv4::attn_workspace_bytes(cfg->dtype == DSV4_BF16, cfg->heads, cfg->dim, cfg->window,
                                      cfg->ratio, cfg->topk, batch, s);
}

int dsv4_compress_prefill(const dsv4_comp_cfg* cfg, void* state, const void* kv_lane,
                          const void* gate_lane, int32_t batch, int64_t n_new,
                          const int64_t* len_before, const void* ape, const void* norm_w,
                          const float* inv_freq, void* rows, int64_t row_cap, void* stream) {
    int st = check_comp_cfg(cfg);
    if (st) return st;
    if (batch < 0) return fail(DSV4_EINVAL, "batch %d < 0", batch);
    if (n_new < 0) return fail(DSV4_EINVAL, "n_new %lld < 0", (long long)n_new);
    if (row_cap < 0) return fail(DSV4_EINVAL, "row_cap < 0");
    if (batch == 0 || n_new == 0) return ok();
    if (!state || !kv_lane || !gate_lane || !len_before || !ape || !norm_w || !rows)
        return fail(DSV4_EINVAL, "NULL buffer pointer");
    if (cfg->rope_dim > 0 && !inv_freq) return fail(DSV4_EINVAL, "inv_freq is NULL");
    for (int b = 0; b < batch; ++b) {
        const int64_t lb = len_before[b];
        if (lb < 0) return fail(DSV4_EINVAL, "len_before[%d] = %lld < 0", b, (long long)lb);
        if (lb + n_new > kPosLimit) return fail(DSV4_ECAPACITY, "sequence %d passes 2^31 tokens", b);
        if ((lb + n_new) / cfg->ratio > row_cap)
            return fail(DSV4_ECAPACITY, "sequence %d needs %lld rows, row_cap %lld", b,
                        (long long)((lb + n_new) / cfg->ratio), (long long)row_cap);
    }
    dsv4::CompressJob j;
    j.r = cfg->ratio; j.coff = cfg->overlap ? 2 : 1; j.nw = int(state_windows(cfg));
    j.D = cfg->dim; j.rd = cfg->rope_dim;
    j.eps = cfg->eps; j.bf16 = cfg->dtype == DSV4_BF16;
    j.state = state; j.lane_a = kv_lane; j.lane_g = gate_lane; j.ape = ape; j.gamma = norm_w;
    j.inv_freq = inv_freq; j.rows = rows; j.row_cap = row_cap; j.n_new = n_new;
    j.batch = batch; j.len_before = len_before;
    return hip_status(dsv4::launch_compress(j, static_cast<hipStream_t>(stream)), "compress");
}

int dsv4_compress_step(const dsv4_comp_cfg* cfg, void* state, const void* kv_lane,
                       const void* gate_lane, int32_t batch, const int64_t* len_before,
                       const void* ape, const void* norm_w, const float* inv_freq,
                       void* rows, int64_t row_cap, void* stream) {
    return dsv4_compress_prefill(cfg, state, kv_lane, gate_lane, batch, 1, len_before, ape,
                                 norm_w, inv_freq, rows, row_cap, stream);
}

}  // extern "C"

namespace {

// The checks and the launch of dsv4_index_topk; `ws_what` names the workspace in errors.
int index_topk_impl(const dsv4_index_cfg* cfg, const void* qi, const float* w,
                    const void* idx_rows, int64_t row_cap, const int64_t* n_rows,
                    const int64_t* pos0, int32_t batch, int64_t s, int32_t* sel, void* ws,
                    size_t ws_bytes, void* stream, const char* ws_what) {
    int st = check_index_cfg(cfg);
    if (st) return st;
    if (batch < 0) return fail(DSV4_EINVAL, "batch %d < 0", batch);
    if (s < 0) return fail(DSV4_EINVAL, "s < 0");
    if (s > 65535) return fail(DSV4_EUNSUPPORTED, "s %lld above 65535 queries per call", (long long)s);
    if (row_cap < 0) return fail(DSV4_EINVAL, "row_cap < 0");
    if (batch == 0 || s == 0) return ok();
    if (!qi || !w || !idx_rows || !n_rows || !pos0 || !sel)
        return fail(DSV4_EINVAL, "NULL buffer pointer");
    int64_t n_max = 0;
    for (int b = 0; b < batch; ++b) {
        if (pos0[b] < 0) return fail(DSV4_EINVAL, "pos0[%d] < 0", b);
        if (pos0[b] + s > kPosLimit) return fail(DSV4_ECAPACITY, "sequence %d passes 2^31 tokens", b);
        if (n_rows[b] > row_cap) return fail(DSV4_ECAPACITY, "n_rows[%d] > row_cap", b);
        const int64_t need = (pos0[b] + s) / cfg->ratio;
        if (n_rows[b] < need)
            return fail(DSV4_EINVAL, "n_rows[%d] = %lld but the last query sees %lld rows", b,
                        (long long)n_rows[b], (long long)need);
        n_max = std::max(n_max, n_rows[b]);
    }
    const size_t need_ws = dsv4::index_workspace_bytes(cfg->heads, cfg->dim, cfg->topk, batch, s, n_max);
    if (!ws || ws_bytes < need_ws)
        return fail(DSV4_EWORKSPACE, "%s of %zu bytes, this call needs %zu", ws_what, ws_bytes,
                    need_ws);
    if (reinterpret_cast<uintptr_t>(ws) % 16 != 0)
        return fail(DSV4_EINVAL, "workspace must be 16-byte aligned");
    dsv4::IndexJob j;
    j.Hi = cfg->heads; j.di = cfg->dim; j.k = cfg->topk; j.r = cfg->ratio;
    j.bf16 = cfg->dtype == DSV4_BF16;
    j.qi = qi; j.w = w; j.rows = idx_rows; j.row_cap = row_cap; j.S = s;
    j.n_stride = dsv4::index_key_stride(n_max);
    j.n_max = n_max;
    j.batch = batch; j.n_rows = n_rows; j.pos0 = pos0; j.sel = sel;
    j.keys = static_cast<uint32_t*>(ws);
    return hip_status(dsv4::launch_index_topk(j, static_cast<hipStream_t>(stream)), "index_topk");
}

// ------------------------------------------------------------------ allocation-free top-k
// The scratch of dsv4_index_topk_noalloc: one array per GPU, in the library's device code
// object, alive until the process ends.  In host code `scratch` is only a stand-in for the
// symbol; its device address (per device) comes from hipGetSymbolAddress.
constexpr size_t kNoallocScratchBytes = size_t(16) << 20;
static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's address of `scratch`, looked up on the first call on that device.
int scratch_address(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return fail(DSV4_EUNSUPPORTED, "device %d above %d", dev, kMaxDevices - 1);
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(scratch)");
        if (!p) return fail(DSV4_EHIP, "hipGetSymbolAddress(scratch) returned NULL");
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return DSV4_OK;
}

}  // namespace

extern "C" {

int dsv4_index_topk(const dsv4_index_cfg* cfg, const void* qi, const float* w,
                    const void* idx_rows, int64_t row_cap, const int64_t* n_rows,
                    const int64_t* pos0, int32_t batch, int64_t s, int32_t* sel, void* ws,
                    size_t ws_bytes, void* stream) {
    return index_topk_impl(cfg, qi, w, idx_rows, row_cap, n_rows, pos0, batch, s, sel, ws,
                           ws_bytes, stream, "workspace");
}

size_t dsv4_index_topk_noalloc_scratch_bytes(void) { return kNoallocScratchBytes; }

int dsv4_index_topk_noalloc(const dsv4_index_cfg* cfg, const void* qi, const float* w,
                            const void* idx_rows, int64_t row_cap, const int64_t* n_rows,
                            const int64_t* pos0, int32_t batch, int64_t s, int32_t* sel,
                            void* stream) {
    void* ws = nullptr;
    int st = scratch_address(&ws);
    if (st) return st;
    return index_topk_impl(cfg, qi, w, idx_rows, row_cap, n_rows, pos0, batch, s, sel, ws,
                           kNoallocScratchBytes, stream, "the library's fixed scratch");
}

static int attn_common(const dsv4_attn_cfg* cfg, const void* q, const void* kv_new,
                       void* win_ring, const void* rows, int64_t row_cap, const int32_t* sel,
                       const int64_t* n_rows, const int64_t* pos0, const float* sinks,
                       void* out, int32_t batch, int64_t s, void* ws, size_t ws_bytes,
                       void* stream, const dsv4_frontier_store* stores = nullptr,
                       int32_t n_stores = 0) {
    int st = check_attn_cfg(cfg);
    if (st) return st;
    if (batch < 0) return fail(DSV4_EINVAL, "batch %d < 0", batch);
    if (s < 0) return fail(DSV4_EINVAL, "s < 0");
    if (s > 65535) return fail(DSV4_EUNSUPPORTED, "s %lld above 65535 queries per call", (long long)s);
    if (batch == 0 || s == 0) return ok();
    if (!q || !kv_new || !win_ring || !sinks || !out || !pos0)
        return fail(DSV4_EINVAL, "NULL buffer pointer");
    const bool has_rows = cfg->ratio > 0;
    if (has_rows && (!rows || !n_rows))
        return fail(DSV4_EINVAL, "ratio > 0 needs rows and n_rows");
    if (has_rows && row_cap < 0) return fail(DSV4_EINVAL, "row_cap < 0");
    if (sel && !has_rows) return fail(DSV4_EINVAL, "sel given for a layer without rows");
    if (sel && cfg->topk < 1) return fail(DSV4_EINVAL, "sel given with topk < 1");
    const int64_t key_cap = dsv4::attn_max_keys(cfg->dtype == DSV4_BF16, cfg->heads, cfg->dim,
                                                cfg->topk, sel != nullptr);
    for (int b = 0; b < batch; ++b) {
        if (pos0[b] < 0) return fail(DSV4_EINVAL, "pos[%d] < 0", b);
        if (pos0[b] + s > kPosLimit) return fail(DSV4_ECAPACITY, "sequence %d passes 2^31 tokens", b);
        int64_t nkeys = cfg->window;
        if (has_rows) {
            if (n_rows[b] > row_cap) return fail(DSV4_ECAPACITY, "n_rows[%d] > row_cap", b);
            const int64_t need = (pos0[b] + s) / cfg->ratio;
            if (n_rows[b] < need)
                return fail(DSV4_EINVAL, "n_rows[%d] = %lld but the last query sees %lld rows", b,
                            (long long)n_rows[b], (long long)need);
            nkeys += sel ? std::min<int64_t>(need, cfg->topk) : need;
        }
        if (nkeys > key_cap)
            return fail(DSV4_EUNSUPPORTED, "a query of sequence %d has %lld keys, above %lld", b,
                        (long long)nkeys, (long long)key_cap);
    }
    const size_t need_ws = dsv4::attn_workspace_bytes(cfg->dtype == DSV4_BF16, cfg->heads, cfg->dim,
                                                      cfg->window, cfg->ratio, cfg->topk, batch, s);
    if (need_ws > 0 && (!ws || ws_bytes < need_ws))
        return fail(DSV4_EWORKSPACE, "workspace %zu bytes, need %zu", ws_bytes, need_ws);
    if (n_stores < 0 || n_stores > 2) return fail(DSV4_EINVAL, "n_stores %d outside 0..2", n_stores);
    if (n_stores > 0 && !stores) return fail(DSV4_EINVAL, "stores is NULL");
    dsv4::FrontierJob fronts[2];
    for (int f = 0; f < n_stores; ++f) {
        const dsv4_frontier_store& fs = stores[f];
        if (!fs.cfg) return fail(DSV4_EINVAL, "stores[%d].cfg is NULL", f);
        st = check_comp_cfg(fs.cfg);
        if (st) return st;
        if (fs.cfg->ratio != cfg->ratio || fs.cfg->dtype != cfg->dtype)
            return fail(DSV4_EINVAL, "stores[%d]: ratio or dtype differs from the attention's", f);
        if (!fs.state || !fs.kv_lane || !fs.gate_lane)
            return fail(DSV4_EINVAL, "stores[%d]: NULL buffer pointer", f);
        for (int b = 0; b < batch; ++b)
            if ((pos0[b] + 1) % cfg->ratio == 0)
                return fail(DSV4_EINVAL, "sequence %d completes row %lld at this step: call "
                            "dsv4_compress_step, then dsv4_csa_attn_decode", b,
                            (long long)((pos0[b] + 1) / cfg->ratio - 1));
        const int coff = fs.cfg->overlap ? 2 : 1;
        fronts[f].state = fs.state; fronts[f].lane_a = fs.kv_lane; fronts[f].lane_g = fs.gate_lane;
        fronts[f].r = fs.cfg->ratio; fronts[f].nw = int(state_windows(fs.cfg));
        fronts[f].W = coff * fs.cfg->dim;
    }
    dsv4::AttnJob j;
    j.H = cfg->heads; j.D = cfg->dim; j.W = cfg->window; j.Wr = cfg->window + cfg->retain;
    j.r = cfg->ratio; j.k = cfg->topk;
    j.scale = cfg->scale; j.bf16 = cfg->dtype == DSV4_BF16;
    j.q = q; j.kv_new = kv_new; j.ring = win_ring; j.rows = has_rows ? rows : nullptr;
    j.row_cap = row_cap; j.sel = sel; j.sinks = sinks; j.out = out; j.S = s; j.batch = batch;
    j.n_rows = has_rows ? n_rows : nullptr; j.pos0 = pos0; j.ws = ws; j.ws_bytes = ws_bytes;
    j.n_fronts = n_stores;
    for (int f = 0; f < n_stores; ++f) j.fronts[f] = fronts[f];
    return hip_status(dsv4::launch_attention(j, static_cast<hipStream_t>(stream)), "attention");
}

int dsv4_csa_attn_decode(const dsv4_attn_cfg* cfg, const void* q, const void* kv_new,
                         void* win_ring, const void* rows, int64_t row_cap,
                         const int32_t* sel, const int64_t* n_rows, const int64_t* pos,
                         const float* sinks, void* out, int32_t batch, void* ws,
                         size_t ws_bytes, void* stream) {
    return attn_common(cfg, q, kv_new, win_ring, rows, row_cap, sel, n_rows, pos, sinks, out,
                       batch, 1, ws, ws_bytes, stream);
}

int dsv4_csa_attn_decode_store(const dsv4_attn_cfg* cfg, const void* q, const void* kv_new,
                               void* win_ring, const void* rows, int64_t row_cap,
                               const int32_t* sel, const int64_t* n_rows, const int64_t* pos,
                               const float* sinks, void* out, int32_t batch, void* ws,
                               size_t ws_bytes, const dsv4_frontier_store* stores,
                               int32_t n_stores, void* stream) {
    if (cfg && cfg->ratio <= 0 && n_stores > 0)
        return fail(DSV4_EINVAL, "frontier stores given for a layer without a compressed lane");
    return attn_common(cfg, q, kv_new, win_ring, rows, row_cap, sel, n_rows, pos, sinks, out,
                       batch, 1, ws, ws_bytes, stream, stores, n_stores);
}

int dsv4_csa_attn_prefill(const dsv4_attn_cfg* cfg, const void* q, const void* kv_new,
                          void* win_ring, const void* rows, int64_t row_cap,
                          const int32_t* sel, const int64_t* n_rows, const int64_t* pos0,
                          const float* sinks, void* out, int32_t batch, int64_t s, void* ws,
                          size_t ws_bytes, void* stream) {
    return attn_common(cfg, q, kv_new, win_ring, rows, row_cap, sel, n_rows, pos0, sinks, out,
                       batch, s, ws, ws_bytes, stream);
}

int dsv4_rope(const dsv4_rope_cfg* cfg, void* x, const int64_t* pos0, int32_t batch, int64_t s,
              const float* inv_freq, void* stream) {
    if (!cfg) return fail(DSV4_EINVAL, "cfg is NULL");
    if (cfg->heads < 1 || cfg->heads > 65535) return fail(DSV4_EINVAL, "heads %d outside 1..65535", cfg->heads);
    if (cfg->dim < 1 || cfg->dim > 4096) return fail(DSV4_EINVAL, "dim %d outside 1..4096", cfg->dim);
    if (cfg->rope_dim < 0 || cfg->rope_dim > cfg->dim || (cfg->rope_dim & 1))
        return fail(DSV4_EINVAL, "rope_dim %d must be even and within 0..dim", cfg->rope_dim);
    if (cfg->inverse != 0 && cfg->inverse != 1) return fail(DSV4_EINVAL, "inverse must be 0 or 1");
    if (!dtype_ok(cfg->dtype)) return fail(DSV4_EINVAL, "unknown dtype %d", cfg->dtype);
    if (batch < 0) return fail(DSV4_EINVAL, "batch %d < 0", batch);
    if (s < 0) return fail(DSV4_EINVAL, "s < 0");
    if (s > 65535) return fail(DSV4_EUNSUPPORTED, "s %lld above 65535 tokens per call", (long long)s);
    if (batch == 0 || s == 0 || cfg->rope_dim == 0) return ok();
    if (!x || !pos0 || !inv_freq) return fail(DSV4_EINVAL, "NULL buffer pointer");
    for (int b = 0; b < batch; ++b) {
        if (pos0[b] < 0) return fail(DSV4_EINVAL, "pos0[%d] < 0", b);
        if (pos0[b] + s > kPosLimit) return fail(DSV4_ECAPACITY, "sequence %d passes 2^31 tokens", b);
    }
    dsv4::RopeJob j;
    j.H = cfg->heads; j.D = cfg->dim; j.rd = cfg->rope_dim; j.inverse = cfg->inverse != 0;
    j.bf16 = cfg->dtype == DSV4_BF16; j.x = x; j.inv_freq = inv_freq; j.S = s; j.batch = batch;
    j.pos0 = pos0;
    return hip_status(dsv4::launch_rope(j, static_cast<hipStream_t>(stream)), "rope");
}

int dsv4_grouped_proj(const dsv4_gproj_cfg* cfg, const void* x, const void* w, void* y,
                      int64_t tokens, void* stream) {
    if (!cfg) return fail(DSV4_EINVAL, "cfg is NULL");
    if (cfg->groups < 1) return fail(DSV4_EINVAL, "groups %d < 1", cfg->groups);
    if (cfg->in_dim < 1 || cfg->in_dim > 65536) return fail(DSV4_EINVAL, "in_dim %d outside 1..65536", cfg->in_dim);
    if (cfg->out_dim < 1 || cfg->out_dim > 65536) return fail(DSV4_EINVAL, "out_dim %d outside 1..65536", cfg->out_dim);
    if (!dtype_ok(cfg->dtype)) return fail(DSV4_EINVAL, "unknown dtype %d", cfg->dtype);
    if (tokens < 0) return fail(DSV4_EINVAL, "tokens < 0");
    if (tokens == 0) return ok();
    if (!x || !w || !y) return fail(DSV4_EINVAL, "NULL buffer pointer");
    if (tokens * cfg->groups * int64_t(cfg->out_dim) > (int64_t(1) << 39) || tokens > (int64_t(1) << 31))
        return fail(DSV4_EUNSUPPORTED, "tokens x groups x out_dim too large");
    dsv4::GprojJob j;
    j.G = cfg->groups; j.K = cfg->in_dim; j.R = cfg->out_dim; j.bf16 = cfg->dtype == DSV4_BF16;
    j.x = x; j.w = w; j.y = y; j.T = tokens;
    return hip_status(dsv4::launch_grouped_proj(j, static_cast<hipStream_t>(stream)), "grouped_proj");
}

int dsv4_lane_proj(const dsv4_gproj_cfg* cfg, const void* x, const void* w_kv, const void* w_gate, void* a,
                   void* g, int64_t tokens, void* stream) {
    if (!cfg) return fail(DSV4_EINVAL, "cfg is NULL");
    if (cfg->groups != 1) return fail(DSV4_EINVAL, "groups %d: the lane projection takes one group", cfg->groups);
    if (cfg->in_dim < 1 || cfg->in_dim > 65536) return fail(DSV4_EINVAL, "in_dim %d outside 1..65536", cfg->in_dim);
    if (cfg->out_dim < 1 || cfg->out_dim > 65536) return fail(DSV4_EINVAL, "out_dim %d outside 1..65536", cfg->out_dim);
    if (!dtype_ok(cfg->dtype)) return fail(DSV4_EINVAL, "unknown dtype %d", cfg->dtype);
    if (tokens < 0) return fail(DSV4_EINVAL, "tokens < 0");
    if (tokens == 0) return ok();
    if (!x || !w_kv || !w_gate || !a || !g) return fail(DSV4_EINVAL, "NULL buffer pointer");
    if (tokens * int64_t(cfg->out_dim) > (int64_t(1) << 39) || tokens > (int64_t(1) << 31))
        return fail(DSV4_EUNSUPPORTED, "tokens x out_dim too large");
    dsv4::GprojJob j;
    j.G = 1; j.K = cfg->in_dim; j.R = cfg->out_dim; j.bf16 = cfg->dtype == DSV4_BF16;
    j.x = x; j.w = w_kv; j.y = a; j.T = tokens; j.w2 = w_gate; j.y2 = g;
    return hip_status(dsv4::launch_grouped_proj(j, static_cast<hipStream_t>(stream)), "lane_proj");
}

int dsv4_trace_enable(int32_t on) {
    g_trace_on.store(on != 0);
    return ok();
}

int dsv4_trace_reset(void) {
    std::lock_guard<std::mutex> lk(g_trace_mu);
    for (auto& r : g_recs) {
        if (r.start) g_event_pool.push_back(r.start);
        if (r.stop) g_event_pool.push_back(r.stop);
    }
    g_recs.clear();
    return ok();
}

int dsv4_trace_read(const char* name_substr, int64_t* launches, double* total_ms) {
    if (!launches || !total_ms) return fail(DSV4_EINVAL, "NULL output pointer");
    std::lock_guard<std::mutex> lk(g_trace_mu);
    int64_t n = 0;
    double ms = 0.0;
    for (auto& r : g_recs) {
        if (name_substr && name_substr[0] == '=') {          // "=name": that kernel only
            if (std::strcmp(r.name, name_substr + 1) != 0) continue;
        } else if (name_substr && *name_substr && !std::strstr(r.name, name_substr)) {
            continue;
        }
        if (!r.start || !r.stop) return fail(DSV4_EHIP, "trace record without events");
        hipError_t e = hipEventSynchronize(r.stop);
        if (e != hipSuccess) return hip_status(e, "trace sync");
        float t = 0.f;
        e = hipEventElapsedTime(&t, r.start, r.stop);
        if (e != hipSuccess) return hip_status(e, "trace elapsed");
        ms += t;
        ++n;
    }
    *launches = n;
    *total_ms = ms;
    return ok();
}

const char* dsv4_trace_kernel_name(int32_t i) {
    std::lock_guard<std::mutex> lk(g_trace_mu);
    if (i < 0 || size_t(i) >= g_trace_names.size()) return nullptr;
    return g_trace_names[size_t(i)].c_str();
}

}  // extern "C"
