// Indexer: fp32 scores of the visible compressed rows, then an exact per-query top-k.
//
// Pages: mlx-lm PR #1189 stepnoy's patch ("Reference scoring": raw weights_proj output, no
// sigmoid, scale d_i^-1/2 * H_i^-1/2 folded into the weights, ReLU on the logits, summed
// over heads, fp32; causality applied before ranking) and aidiffuser's indexer path (per-
// query top-k over the indexer's own cache-backed lane, same ratio as the attention lane,
// so both index spaces coincide); MTPLX PR #216 "What V4 adds" (the filter engages once the
// lane holds more than index_topk rows) and "Verification" (tie-break is part of the
// contract).
//
// Scores are written as order-preserving u32 keys (larger score -> larger key, -0 == +0)
// into a workspace [B][S][n_stride].  Selection finds the k-th largest key T of the query's
// visible prefix by a 4-pass, 8-bit radix select, then compacts in row order: every row
// with key > T, plus the lowest-indexed rows with key == T until k rows are taken.  Row
// order compaction makes the output ascending without a sort.
#include "common.hpp"
#include "kernels.hpp"

namespace dsv4 {

namespace {

constexpr int kScoreRows = 64;      // rows per workgroup of the scoring kernel
constexpr int kScoreThreads = 256;
constexpr int kSelThreads = 256;

template <typename T>
struct ScoreArgs {
    int Hi, di, r;
    float scale;
    const T* qi;
    const float* w;
    const T* rows;
    int64_t row_cap;
    int64_t S;
    int64_t n_stride;
    uint32_t* keys;
};

// One workgroup scores kScoreRows rows for one query, one wave per row at a time: each
// lane holds a strided slice of the row, and every head's dot product is a wave reduction.
// LDS holds the query's heads in fp32 and the folded head weights.
template <typename T>
__global__ void __launch_bounds__(kScoreThreads)
index_score_kernel(ScoreArgs<T> a, SeqInts pos0, SeqInts n_rows) {
    extern __shared__ float sh[];                 // [Hi*di] q, then [Hi] weights
    float* qs = sh;
    float* ws = sh + a.Hi * a.di;
    const int b = blockIdx.z;
    const int64_t s = blockIdx.y;
    const int64_t p = int64_t(pos0.v[b]) + s;
    int64_t nv = (p + 1) / a.r;
    if (nv > n_rows.v[b]) nv = n_rows.v[b];
    const int64_t j0 = int64_t(blockIdx.x) * kScoreRows;
    if (j0 >= nv) return;
    const T* q = a.qi + (size_t(b) * a.S + size_t(s)) * a.Hi * a.di;
    for (int i = threadIdx.x; i < a.Hi * a.di; i += blockDim.x) qs[i] = to_f32(q[i]);
    for (int h = threadIdx.x; h < a.Hi; h += blockDim.x)
        ws[h] = a.w[(size_t(b) * a.S + size_t(s)) * a.Hi + h] * a.scale;
    __syncthreads();
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwave = blockDim.x >> 6;
    const int64_t j1 = j0 + kScoreRows < nv ? j0 + kScoreRows : nv;
    uint32_t* out = a.keys + (size_t(b) * a.S + size_t(s)) * a.n_stride;
    for (int64_t j = j0 + wave; j < j1; j += nwave) {
        const T* kr = a.rows + (size_t(b) * a.row_cap + size_t(j)) * a.di;
        float score = 0.f;
        for (int h = 0; h < a.Hi; ++h) {
            const float* qh = qs + h * a.di;
            float dot = 0.f;
            for (int d = lane; d < a.di; d += 64) dot = fmaf(qh[d], to_f32(kr[d]), dot);
            dot = wave_sum(dot);
            score = fmaf(ws[h], fmaxf(dot, 0.f), score);
        }
        if (lane == 0) out[j] = score_key(score);
    }
}

struct SelArgs {
    int k, r;
    int64_t S;
    int64_t n_stride;
    const uint32_t* keys;
    int32_t* sel;
};

// One workgroup selects for one query.
__global__ void __launch_bounds__(kSelThreads)
topk_select_kernel(SelArgs a, SeqInts pos0, SeqInts n_rows) {
    __shared__ uint32_t hist[256];
    __shared__ int32_t cnt_gt[kSelThreads], cnt_eq[kSelThreads];
    __shared__ uint32_t sh_digit;
    __shared__ int32_t sh_rem;
    const int b = blockIdx.y;
    const int64_t s = blockIdx.x;
    const int64_t p = int64_t(pos0.v[b]) + s;
    int64_t nv = (p + 1) / a.r;
    if (nv > n_rows.v[b]) nv = n_rows.v[b];
    int32_t* out = a.sel + (size_t(b) * a.S + size_t(s)) * a.k;
    const int tid = threadIdx.x;
    if (nv <= a.k) {                                  // dense regime: every visible row
        for (int i = tid; i < a.k; i += blockDim.x) out[i] = i < nv ? i : -1;
        return;
    }
    const uint32_t* key = a.keys + (size_t(b) * a.S + size_t(s)) * a.n_stride;

    // radix select of the k-th largest key
    uint32_t prefix = 0, mask = 0;
    int32_t rem = a.k;
    for (int shift = 24; shift >= 0; shift -= 8) {
        for (int i = tid; i < 256; i += blockDim.x) hist[i] = 0;
        __syncthreads();
        for (int64_t j = tid; j < nv; j += blockDim.x) {
            const uint32_t kk = key[j];
            if ((kk & mask) == prefix) atomicAdd(&hist[(kk >> shift) & 255u], 1u);
        }
        __syncthreads();
        if (tid == 0) {
            int32_t cum = 0;
            int d = 255;
            for (; d > 0; --d) {
                if (cum + int32_t(hist[d]) >= rem) break;
                cum += int32_t(hist[d]);
            }
            sh_digit = uint32_t(d);
            sh_rem = rem - cum;
        }
        __syncthreads();
        prefix |= sh_digit << shift;
        mask |= 255u << shift;
        rem = sh_rem;
        __syncthreads();
    }
    const uint32_t thr = prefix;     // the k-th largest key; take `rem` rows equal to it

    // compaction in row order: each thread owns a contiguous segment of rows
    const int64_t seg = (nv + blockDim.x - 1) / blockDim.x;
    const int64_t lo = int64_t(tid) * seg;
    const int64_t hi = lo + seg < nv ? lo + seg : nv;
    int32_t ngt = 0, neq = 0;
    for (int64_t j = lo; j < hi; ++j) {
        const uint32_t kk = key[j];
        ngt += kk > thr;
        neq += kk == thr;
    }
    cnt_gt[tid] = ngt;
    cnt_eq[tid] = neq;
    __syncthreads();
    if (tid == 0) {                                   // exclusive scan over the segments
        int32_t g = 0, e = 0;
        for (int i = 0; i < int(blockDim.x); ++i) {
            const int32_t tg = cnt_gt[i], te = cnt_eq[i];
            cnt_gt[i] = g;
            cnt_eq[i] = e;
            g += tg;
            e += te;
        }
    }
    __syncthreads();
    int32_t eq_rank = cnt_eq[tid];
    int32_t o = cnt_gt[tid] + (eq_rank < rem ? eq_rank : rem);
    for (int64_t j = lo; j < hi; ++j) {
        const uint32_t kk = key[j];
        if (kk > thr) {
            out[o++] = int32_t(j);
        } else if (kk == thr) {
            if (eq_rank < rem) out[o++] = int32_t(j);
            ++eq_rank;
        }
    }
}

template <typename T>
hipError_t run(const IndexJob& j, hipStream_t st) {
    for (int b0 = 0; b0 < j.batch; b0 += kSeqSlice) {
        const int nb = std::min(kSeqSlice, j.batch - b0);
        SeqInts pos{}, nr{};
        int64_t nv_max = 0;
        for (int i = 0; i < nb; ++i) {
            pos.v[i] = int32_t(j.pos0[b0 + i]);
            nr.v[i] = int32_t(j.n_rows[b0 + i]);
            const int64_t nv = std::min<int64_t>((j.pos0[b0 + i] + j.S) / j.r, j.n_rows[b0 + i]);
            nv_max = std::max(nv_max, nv);
        }
        const size_t qoff = size_t(b0) * j.S;
        if (nv_max > j.k) {
            ScoreArgs<T> a;
            a.Hi = j.Hi; a.di = j.di; a.r = j.r;
            a.scale = 1.0f / sqrtf(float(j.di)) / sqrtf(float(j.Hi));
            a.qi = static_cast<const T*>(j.qi) + qoff * j.Hi * j.di;
            a.w = j.w + qoff * j.Hi;
            a.rows = static_cast<const T*>(j.rows) + size_t(b0) * j.row_cap * j.di;
            a.row_cap = j.row_cap;
            a.S = j.S;
            a.n_stride = j.n_stride;
            a.keys = j.keys + qoff * j.n_stride;
            const unsigned gx = unsigned((nv_max + kScoreRows - 1) / kScoreRows);
            const size_t lds = size_t(j.Hi) * j.di * sizeof(float) + j.Hi * sizeof(float);
            trace_begin("index_score", st);
            hipLaunchKernelGGL(index_score_kernel<T>, dim3(gx, unsigned(j.S), nb),
                               dim3(kScoreThreads), lds, st, a, pos, nr);
            trace_end("index_score", st);
            hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
        SelArgs sa;
        sa.k = j.k; sa.r = j.r; sa.S = j.S; sa.n_stride = j.n_stride;
        sa.keys = j.keys + qoff * j.n_stride;
        sa.sel = j.sel + qoff * j.k;
        trace_begin("topk_select", st);
        hipLaunchKernelGGL(topk_select_kernel, dim3(unsigned(j.S), nb), dim3(kSelThreads), 0,
                           st, sa, pos, nr);
        trace_end("topk_select", st);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace

size_t index_workspace_bytes(int Hi, int di, int k, int batch, int64_t S, int64_t n_max) {
    (void)Hi; (void)di; (void)k;
    return size_t(batch) * size_t(S) * size_t(n_max < 1 ? 1 : n_max) * sizeof(uint32_t);
}

hipError_t launch_index_topk(const IndexJob& j, hipStream_t s) {
    return j.bf16 ? run<bf16>(j, s) : run<float>(j, s);
}

}  // namespace dsv4
