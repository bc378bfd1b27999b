// Sparse MQA attention with sinks over a sliding window plus selected compressed rows.
//
// Pages: MTPLX PR #216 opening and "What V4 adds" (H query heads over one shared latent
// that serves as key and value, a 128-token sliding window beside the compressed lane, per-
// head sink logits); "Decode dispatch reduction" (A) (the sink acts as an extra key column
// with an all-zero value, so it appears in the softmax denominator only; softmax max and
// sums in fp32); "Decode path" (q/kv/o stored bf16 with fp32 accumulation); mlx-lm PR
// #1189 stepnoy's patch (selected rows attended beside the window; row j visible to the
// query at p iff (j+1)*r <= p+1) and aidiffuser's mask diagnosis (window of W tokens
// ending at the query).
//
// generic kernel: one workgroup per (query, head).  Phase 1 computes every key's logit
// into LDS (one wave per key), phase 2 takes the max (with the sink) and the exponentials,
// phase 3 forms the weighted sum of the key rows with threads over the latent dims.
//
// The ring update runs after the attention kernel on the stream: writing token t evicts
// token t - W, which an earlier query of the same call may still need.
#include "common.hpp"
#include "kernels.hpp"

namespace dsv4 {

namespace {

constexpr int kAttnThreads = 256;
constexpr size_t kAttnLdsMax = 65536 - 1024;   // dynamic LDS: 4 B per latent dim + 8 per key

template <typename T>
struct AttnArgs {
    int H, D, W, r, k;
    float scale;
    const T* q;
    const T* kv_new;
    T* ring;
    const T* rows;
    int64_t row_cap;
    const int32_t* sel;
    const float* sinks;
    T* out;
    int64_t S;
    int nk_cap;        // keys one query may have (sizes the LDS arrays)
};

// Key source code: >= 0 compressed row j; < 0 window token t encoded as -(t + 1).
template <typename T>
__device__ __forceinline__ const T* key_row(const AttnArgs<T>& a, int b, int32_t code,
                                            int64_t pos0) {
    if (code >= 0) return a.rows + (size_t(b) * a.row_cap + size_t(code)) * a.D;
    const int64_t t = -int64_t(code) - 1;
    if (t >= pos0) return a.kv_new + (size_t(b) * a.S + size_t(t - pos0)) * a.D;
    return a.ring + (size_t(b) * a.W + size_t(t % a.W)) * a.D;
}

template <typename T>
__global__ void __launch_bounds__(kAttnThreads)
attn_generic_kernel(AttnArgs<T> a, SeqInts pos0v, SeqInts n_rows) {
    extern __shared__ unsigned char smem[];
    __shared__ float red[16];
    __shared__ int nk_sh;
    const int b = blockIdx.z;
    const int h = blockIdx.y;
    const int64_t s = blockIdx.x;
    const int64_t pos0 = pos0v.v[b];
    const int64_t p = pos0 + s;
    const int tid = threadIdx.x;
    float* qs = reinterpret_cast<float*>(smem);                 // [D]
    float* lg = qs + a.D;                                       // [nk_cap]
    int32_t* code = reinterpret_cast<int32_t*>(lg + a.nk_cap);  // [nk_cap]

    const T* qh = a.q + ((size_t(b) * a.S + size_t(s)) * a.H + h) * a.D;
    for (int d = tid; d < a.D; d += blockDim.x) qs[d] = to_f32(qh[d]);

    // key list: compressed rows first, then the window
    int64_t nrow = 0;
    if (a.r > 0 && a.rows != nullptr) {
        int64_t nv = (p + 1) / a.r;
        if (nv > n_rows.v[b]) nv = n_rows.v[b];
        if (a.sel == nullptr) {
            for (int64_t i = tid; i < nv; i += blockDim.x) code[i] = int32_t(i);
            nrow = nv;
        } else {
            const int32_t* sr = a.sel + (size_t(b) * a.S + size_t(s)) * a.k;
            if (tid == 0) {
                int64_t c = 0;
                const int64_t cap = a.nk_cap - a.W;    // bounds the LDS list even for duplicates
                for (int i = 0; i < a.k && c < cap; ++i) {
                    const int32_t jj = sr[i];
                    if (jj >= 0 && jj < nv) code[c++] = jj;
                }
                nk_sh = int(c);
            }
            __syncthreads();
            nrow = nk_sh;
        }
    }
    const int64_t t0 = p - a.W + 1 > 0 ? p - a.W + 1 : 0;
    const int64_t nwin = p - t0 + 1;
    for (int64_t i = tid; i < nwin; i += blockDim.x) code[nrow + i] = int32_t(-(t0 + i + 1));
    const int64_t nk = nrow + nwin;
    __syncthreads();

    // phase 1: logits, one wave per key (coalesced row reads, wave reduction)
    const int lane = tid & 63, wave = tid >> 6, nwave = blockDim.x >> 6;
    float mx = -INFINITY;
    for (int64_t i = wave; i < nk; i += nwave) {
        const T* x = key_row(a, b, code[i], pos0);
        float dot = 0.f;
        for (int d = lane; d < a.D; d += 64) dot = fmaf(qs[d], to_f32(x[d]), dot);
        dot = wave_sum(dot);
        const float l = dot * a.scale;
        if (lane == 0) lg[i] = l;
        mx = fmaxf(mx, l);
    }
    __syncthreads();
    const float z = a.sinks[h];
    const float m = fmaxf(block_max(mx, red), z);
    // phase 2: exponentials and the denominator
    float sum = 0.f;
    for (int64_t i = tid; i < nk; i += blockDim.x) {
        const float e = expf(lg[i] - m);
        lg[i] = e;
        sum += e;
    }
    const float den = block_sum(sum, red) + expf(z - m);
    __syncthreads();
    // phase 3: weighted sum of the key rows
    T* o = a.out + ((size_t(b) * a.S + size_t(s)) * a.H + h) * a.D;
    for (int d = tid; d < a.D; d += blockDim.x) {
        float acc = 0.f;
        for (int64_t i = 0; i < nk; ++i) acc = fmaf(lg[i], to_f32(key_row(a, b, code[i], pos0)[d]), acc);
        o[d] = from_f32<T>(acc / den);
    }
}

template <typename T>
__global__ void __launch_bounds__(kAttnThreads)
ring_update_kernel(AttnArgs<T> a, SeqInts pos0v) {
    const int b = blockIdx.y;
    const int64_t pos0 = pos0v.v[b];
    const int64_t first = a.S > a.W ? pos0 + a.S - a.W : pos0;
    const int64_t t = first + blockIdx.x;
    if (t >= pos0 + a.S) return;
    const T* src = a.kv_new + (size_t(b) * a.S + size_t(t - pos0)) * a.D;
    T* dst = a.ring + (size_t(b) * a.W + size_t(t % a.W)) * a.D;
    for (int d = threadIdx.x; d < a.D; d += blockDim.x) dst[d] = src[d];
}

template <typename T>
hipError_t run(const AttnJob& j, hipStream_t st) {
    for (int b0 = 0; b0 < j.batch; b0 += kSeqSlice) {
        const int nb = std::min(kSeqSlice, j.batch - b0);
        SeqInts pos{}, nr{};
        int64_t nrow_max = 0;
        for (int i = 0; i < nb; ++i) {
            pos.v[i] = int32_t(j.pos0[b0 + i]);
            nr.v[i] = j.n_rows ? int32_t(j.n_rows[b0 + i]) : 0;
            if (j.r > 0 && j.rows) {
                const int64_t nv = std::min<int64_t>((j.pos0[b0 + i] + j.S) / j.r, j.n_rows[b0 + i]);
                nrow_max = std::max<int64_t>(nrow_max, j.sel ? std::min<int64_t>(nv, j.k) : nv);
            }
        }
        const size_t qoff = size_t(b0) * j.S;
        AttnArgs<T> a;
        a.H = j.H; a.D = j.D; a.W = j.W; a.r = j.r; a.k = j.k; a.scale = j.scale;
        a.q = static_cast<const T*>(j.q) + qoff * j.H * j.D;
        a.kv_new = static_cast<const T*>(j.kv_new) + qoff * j.D;
        a.ring = static_cast<T*>(j.ring) + size_t(b0) * j.W * j.D;
        a.rows = j.rows ? static_cast<const T*>(j.rows) + size_t(b0) * j.row_cap * j.D : nullptr;
        a.row_cap = j.row_cap;
        a.sel = j.sel ? j.sel + qoff * j.k : nullptr;
        a.sinks = j.sinks;
        a.out = static_cast<T*>(j.out) + qoff * j.H * j.D;
        a.S = j.S;
        a.nk_cap = int(nrow_max + j.W);
        const size_t lds = size_t(j.D) * 4 + size_t(a.nk_cap) * 8;
        trace_begin("attn_generic", st);
        hipLaunchKernelGGL(attn_generic_kernel<T>, dim3(unsigned(j.S), unsigned(j.H), nb),
                           dim3(kAttnThreads), lds, st, a, pos, nr);
        trace_end("attn_generic", st);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        const int64_t nupd = std::min<int64_t>(j.S, j.W);
        trace_begin("ring_update", st);
        hipLaunchKernelGGL(ring_update_kernel<T>, dim3(unsigned(nupd), nb), dim3(kAttnThreads), 0,
                           st, a, pos);
        trace_end("ring_update", st);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace

int64_t attn_max_keys(int H, int D) {
    (void)H;
    return int64_t((kAttnLdsMax - size_t(D) * 4) / 8);
}

size_t attn_workspace_bytes(int H, int D, int W, int r, int k, int batch, int64_t S) {
    (void)H; (void)D; (void)W; (void)r; (void)k; (void)batch; (void)S;
    return 0;
}

hipError_t launch_attention(const AttnJob& j, hipStream_t s) {
    return j.bf16 ? run<bf16>(j, s) : run<float>(j, s);
}

}  // namespace dsv4
