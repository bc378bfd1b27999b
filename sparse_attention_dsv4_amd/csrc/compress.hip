// Gated-pooling compressor (one lane): rows for completed windows + frontier state update.
//
// Pages: MTPLX PR #216 "What V4 adds" (learned gated pooling, overlapping ratio-4 windows,
// plain ratio-128 windows, compressed lanes maintained incrementally in prefill and decode);
// mlx-lm PR #1189 Thump604's fix list (ratio-4 lanes are 2*D wide), aidiffuser's indexer
// path (the overlap transform folds the previous window in; the tail and previous window
// are carried across calls; absolute positions set the APE origin), stepnoy's index-space
// fix (tail buffered and replayed, absolute position accumulates), OmarB97 note 2 (rows
// RoPE'd at birth at j*r); MTPLX PR #216 "Decode path" (pool in fp32, cast to the storage
// dtype before the norm).
//
// Layout of the frontier state of one sequence: [lane (kv, gate)][nw][r][coff*D].  Token t
// lives in window slot (t / r) % nw at position t % r.  nw = coff + ceil(retain / r): with
// coff = 2 the state holds the previous complete window and the current partial one, with
// coff = 1 only the current one, and `retain` tokens of rollback add older windows that a
// trim back across a window boundary needs again.
//
// Two kernels per call:
//   compress_rows_kernel  one workgroup per emitted row: reads every slot of the row from
//                         the state (tokens before the call) or the new lanes, pools per
//                         channel with an online softmax, then norm and RoPE in LDS;
//   compress_state_kernel copies the new tokens of the last nw windows into the state.
// The second runs after the first on the stream, because a row of this call may read a
// state slot that the update overwrites.  With one new token per sequence (decode) the two
// fuse into compress_step_kernel.
#include "common.hpp"
#include "kernels.hpp"

namespace dsv4 {

namespace {

constexpr int kCompThreads = 256;
constexpr int kStepThreads = 512;     // decode step: one latent channel per thread at D = 512

template <typename T>
struct CompArgs {
    int r, coff, nw, D, rd;
    float eps;
    T* state;
    const T* lane_a;
    const T* lane_g;
    const T* ape;
    const T* gamma;
    const float* inv_freq;
    T* rows;
    int64_t row_cap;
    int64_t n_new;
};

// One slot of the per-channel online softmax.  Branch-free form of the usual update: when
// the logit does not raise the running max, f = exp(0) = 1 and e = exp(logit - m); when it
// does, f = exp(m - logit) and e = exp(0) = 1 -- the same values as the branching update.
__device__ __forceinline__ void pool_slot(float logit, float v, float& m, float& l, float& acc) {
    const float mn = fmaxf(m, logit);
    const float f = expf(m - mn);             // 0 when m = -inf
    const float e = expf(logit - mn);
    acc = acc * f + e * v;
    l = l * f + e;
    m = mn;
}

// Row j of sequence b: pooled per channel with an online softmax over its slots, rounded,
// RMS-normalised, rounded, RoPE'd on the last rd dims at position j*r, rounded.  Slot s of
// window w is token w*r + s: tokens before the call (t < lb) sit in state window (w % nw)
// at position s, later ones in the new lanes at t - lb.  All positions fit in 32 bits.
template <typename T>
__device__ __forceinline__ void emit_row(const CompArgs<T>& a, int b, int j, int lb,
                                         float* zrow, float* red) {
    const int D = a.D, W = a.coff * a.D, r = a.r;
    const size_t st = size_t(2) * a.nw * r * W;
    const T* sa0 = a.state + size_t(b) * st;                 // kv lane of this sequence
    const T* sg0 = sa0 + size_t(a.nw) * r * W;               // gate lane
    float ss = 0.f;
    for (int c = threadIdx.x; c < D; c += blockDim.x) {
        float m = -INFINITY, l = 0.f, acc = 0.f;
        for (int half = 0; half < a.coff; ++half) {
            // overlap: half 0 <- window j-1, half 1 <- window j; plain: half 0 <- window j
            const int win = (a.coff == 2 && half == 0) ? j - 1 : j;
            if (win < 0) continue;
            const int col = half * D + c;
            const int t0 = win * r;
            int n_state = lb - t0;                             // slots taken from the state
            n_state = n_state < 0 ? 0 : (n_state > r ? r : n_state);
            const size_t wo = size_t(win % a.nw) * r * W + col;
            const T* sa = sa0 + wo;
            const T* sg = sg0 + wo;
            const T* ap = a.ape + col;
#pragma unroll 8
            for (int s = 0; s < n_state; ++s)
                pool_slot(to_f32(sg[size_t(s) * W]) + to_f32(ap[size_t(s) * W]),
                          to_f32(sa[size_t(s) * W]), m, l, acc);
            if (n_state < r) {                                 // first new token: t0 + n_state
                const size_t first = size_t(b) * a.n_new + size_t(t0 + n_state - lb);
                const T* la = a.lane_a + first * W + col;
                const T* lg = a.lane_g + first * W + col;
#pragma unroll 8
                for (int s = n_state; s < r; ++s) {
                    const size_t o = size_t(s - n_state) * W;
                    pool_slot(to_f32(lg[o]) + to_f32(ap[size_t(s) * W]), to_f32(la[o]), m, l, acc);
                }
            }
        }
    const float y = round_to<T>(acc / l);
        zrow[c] = y;
        ss += y * y;
    }
    const float tot = block_sum(ss, red);
    const float den = sqrtf(tot / float(D) + a.eps);
    for (int c = threadIdx.x; c < D; c += blockDim.x)
        zrow[c] = round_to<T>(zrow[c] / den * to_f32(a.gamma[c]));
    __syncthreads();
    const int r0 = D - a.rd;
    const float pos = float(int64_t(j) * a.r);
    T* out = a.rows + (size_t(b) * a.row_cap + size_t(j)) * D;
    for (int c = threadIdx.x; c < D; c += blockDim.x) {
        float v = zrow[c];
        if (c >= r0) {
            const int i = (c - r0) >> 1;
            const float x0 = zrow[r0 + 2 * i], x1 = zrow[r0 + 2 * i + 1];
            float sn, cs;
            sincosf(pos * a.inv_freq[i], &sn, &cs);
            v = ((c - r0) & 1) ? (x0 * sn + x1 * cs) : (x0 * cs - x1 * sn);
        }
        out[c] = from_f32<T>(v);
    }
}

template <typename T>
__global__ void __launch_bounds__(kCompThreads)
compress_rows_kernel(CompArgs<T> a, SeqInts len_before) {
    extern __shared__ float zrow[];           // [D]
    __shared__ float red[16];
    const int b = blockIdx.y;
    const int lb = len_before.v[b];
    const int j = lb / a.r + int(blockIdx.x);  // row index
    if (int64_t(j + 1) * a.r > lb + a.n_new) return;
    emit_row(a, b, j, lb, zrow, red);
}

// One new token per sequence (decode): store it in the frontier and, when it completes a
// window, emit that row -- one launch.  The row reads the state only at positions of
// earlier tokens and takes the new token from the lane, so the store cannot race it.
template <typename T>
__global__ void __launch_bounds__(kStepThreads)
compress_step_kernel(CompArgs<T> a, SeqInts len_before) {
    extern __shared__ float zrow[];
    __shared__ float red[16];
    const int b = blockIdx.x;
    const int64_t lb = len_before.v[b];
    const int W = a.coff * a.D;
    const size_t st = size_t(2) * a.nw * a.r * W;
    T* sa = a.state + size_t(b) * st + frontier_slot(lb, a.r, a.nw, W);
    T* sg = sa + size_t(a.nw) * a.r * W;
    for (int c = threadIdx.x; c < W; c += blockDim.x) {
        sa[c] = a.lane_a[size_t(b) * W + c];
        sg[c] = a.lane_g[size_t(b) * W + c];
    }
    if ((lb + 1) % a.r == 0) emit_row(a, b, int(lb / a.r), int(lb), zrow, red);
}

template <typename T>
__global__ void __launch_bounds__(kCompThreads)
compress_state_kernel(CompArgs<T> a, SeqInts len_before) {
    const int b = blockIdx.y;
    const int64_t lb = len_before.v[b];
    const int64_t la = lb + a.n_new;
    int64_t keep_from = (la / a.r - (a.nw - 1)) * a.r;     // first token of the kept windows
    if (keep_from < lb) keep_from = lb;
    const int64_t t = keep_from + blockIdx.x;
    if (t >= la) return;
    const int W = a.coff * a.D;
    const size_t st = size_t(2) * a.nw * a.r * W;
    const size_t src = (size_t(b) * a.n_new + size_t(t - lb)) * W;
    T* sa = a.state + size_t(b) * st + frontier_slot(t, a.r, a.nw, W);
    T* sg = sa + size_t(a.nw) * a.r * W;
    for (int c = threadIdx.x; c < W; c += blockDim.x) {
        sa[c] = a.lane_a[src + c];
        sg[c] = a.lane_g[src + c];
    }
}

// The frontier store of a decode step alone (no row completes): one workgroup per sequence.
template <typename T>
__global__ void __launch_bounds__(kCompThreads)
frontier_store_kernel(FrontierJob f, SeqInts pos) {
    const int b = blockIdx.x;
    const size_t st = size_t(2) * f.nw * f.r * f.W;
    T* sa = static_cast<T*>(f.state) + size_t(b) * st + frontier_slot(pos.v[b], f.r, f.nw, f.W);
    T* sg = sa + size_t(f.nw) * f.r * f.W;
    const T* la = static_cast<const T*>(f.lane_a) + size_t(b) * f.W;
    const T* lg = static_cast<const T*>(f.lane_g) + size_t(b) * f.W;
    for (int c = threadIdx.x; c < f.W; c += blockDim.x) {
        sa[c] = la[c];
        sg[c] = lg[c];
    }
}

template <typename T>
hipError_t run(const CompressJob& j, hipStream_t s) {
    const int W = j.coff * j.D;
    const size_t st_elems = size_t(2) * j.nw * j.r * W;
    for (int b0 = 0; b0 < j.batch; b0 += kSeqSlice) {
        const int nb = std::min(kSeqSlice, j.batch - b0);
        SeqInts lb{};
        if (j.n_new == 1) {
            CompArgs<T> a;
            a.r = j.r; a.coff = j.coff; a.nw = j.nw; a.D = j.D; a.rd = j.rd; a.eps = j.eps;
            a.state = static_cast<T*>(j.state) + size_t(b0) * st_elems;
            a.lane_a = static_cast<const T*>(j.lane_a) + size_t(b0) * W;
            a.lane_g = static_cast<const T*>(j.lane_g) + size_t(b0) * W;
            a.ape = static_cast<const T*>(j.ape);
            a.gamma = static_cast<const T*>(j.gamma);
            a.inv_freq = j.inv_freq;
            a.rows = static_cast<T*>(j.rows) + size_t(b0) * j.row_cap * j.D;
            a.row_cap = j.row_cap;
            a.n_new = 1;
            for (int i = 0; i < nb; ++i) lb.v[i] = int32_t(j.len_before[b0 + i]);
            DSV4_LAUNCH("compress_step", compress_step_kernel<T>, dim3(nb), dim3(kStepThreads),
                               j.D * sizeof(float), s, a, lb);
            hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
            continue;
        }
        int64_t max_rows = 0, max_keep = 0;
        for (int i = 0; i < nb; ++i) {
            const int64_t l0 = j.len_before[b0 + i];
            lb.v[i] = int32_t(l0);
            const int64_t la = l0 + j.n_new;
            max_rows = std::max(max_rows, la / j.r - l0 / j.r);
            int64_t keep_from = std::max<int64_t>(l0, (la / j.r - (j.nw - 1)) * j.r);
            max_keep = std::max(max_keep, la - keep_from);
        }
        CompArgs<T> a;
        a.r = j.r; a.coff = j.coff; a.nw = j.nw; a.D = j.D; a.rd = j.rd; a.eps = j.eps;
        a.state = static_cast<T*>(j.state) + size_t(b0) * st_elems;
        a.lane_a = static_cast<const T*>(j.lane_a) + size_t(b0) * j.n_new * W;
        a.lane_g = static_cast<const T*>(j.lane_g) + size_t(b0) * j.n_new * W;
        a.ape = static_cast<const T*>(j.ape);
        a.gamma = static_cast<const T*>(j.gamma);
        a.inv_freq = j.inv_freq;
        a.rows = static_cast<T*>(j.rows) + size_t(b0) * j.row_cap * j.D;
        a.row_cap = j.row_cap;
        a.n_new = j.n_new;
        if (max_rows > 0) {
            DSV4_LAUNCH("compress_rows", compress_rows_kernel<T>, dim3(unsigned(max_rows), nb),
                               dim3(kCompThreads), j.D * sizeof(float), s, a, lb);
            hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
        if (max_keep > 0) {
            DSV4_LAUNCH("compress_state", compress_state_kernel<T>, dim3(unsigned(max_keep), nb),
                               dim3(kCompThreads), 0, s, a, lb);
            hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
    }
    return hipSuccess;
}

}  // namespace

hipError_t launch_compress(const CompressJob& j, hipStream_t s) {
    return j.bf16 ? run<bf16>(j, s) : run<float>(j, s);
}

hipError_t launch_frontier_store(const FrontierJob& f, bool bf16_, int batch, const int64_t* pos,
                                 hipStream_t s) {
    const size_t es = bf16_ ? sizeof(bf16) : sizeof(float);
    const size_t st = size_t(2) * f.nw * f.r * f.W;
    for (int b0 = 0; b0 < batch; b0 += kSeqSlice) {
        const int nb = std::min(kSeqSlice, batch - b0);
        SeqInts p{};
        for (int i = 0; i < nb; ++i) p.v[i] = int32_t(pos[b0 + i]);
        FrontierJob g = f;
        g.state = static_cast<char*>(f.state) + size_t(b0) * st * es;
        g.lane_a = static_cast<const char*>(f.lane_a) + size_t(b0) * f.W * es;
        g.lane_g = static_cast<const char*>(f.lane_g) + size_t(b0) * f.W * es;
        if (bf16_)
            DSV4_LAUNCH("frontier_store", frontier_store_kernel<bf16>, dim3(nb), dim3(kCompThreads), 0, s, g, p);
        else
            DSV4_LAUNCH("frontier_store", frontier_store_kernel<float>, dim3(nb), dim3(kCompThreads), 0, s, g, p);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace dsv4
