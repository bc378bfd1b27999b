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
// mfma kernel (bf16, 64 heads, 512 latent): one workgroup per (query, key split) with all
// 64 heads sharing every 64-key tile staged in LDS.  Q*K^T and P*V run on
// v_mfma_f32_32x32x16_bf16; the softmax is online in base 2 with fp32 running max and sum;
// P is rounded to bf16 before P*V (the pages' reference kernel does the same, MTPLX PR #216
// "Decode path").  A query whose key list is split over several workgroups (decode) writes
// fp32 partials (max, sum, unnormalised output) that attn_combine_kernel merges with the
// sink; a query handled by one workgroup (prefill) normalises and writes its output.
//
// The ring update runs after the attention kernel on the stream: writing token t evicts
// token t - W, which an earlier query of the same call may still need.
#include "common.hpp"
#include "kernels.hpp"
#include "mfma.hpp"

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


// ------------------------------------------------------------------ mfma path
constexpr int MH = 64;                    // heads
constexpr int MD = 512;                   // latent dims
constexpr int MKT = 64;                   // keys per tile
constexpr int KPITCH = MD * 2 + 16;       // LDS bytes per key row (padded against bank conflicts)
constexpr int PPITCH = MKT * 2 + 16;      // LDS bytes per head row of P
constexpr int MAX_CODES = 1024;           // selected rows one workgroup may list
constexpr int MAX_SPLITS = 32;
constexpr float kLog2e = 1.4426950408889634f;

struct AttnMfmaArgs {
    const bf16* q;
    const bf16* kv_new;
    const bf16* ring;
    const bf16* rows;
    int64_t row_cap;
    const int32_t* sel;
    int k;
    const float* sinks;
    bf16* out;
    int64_t S;
    int W, r;
    float scale_log2;                     // logit scale * log2(e)
    int keys_per_split, n_splits;
    float* part_ml;                       // [B][S][n_splits][H][2]  running max, sum
    float* part_o;                        // [B][S][n_splits][H][D]  unnormalised output
};

// Source row of key `i` of the query's list: selected/visible rows first, then the window.
__device__ __forceinline__ const bf16* mfma_key(const AttnMfmaArgs& a, int b, int64_t i,
                                                int64_t nrow, const int32_t* codes, int64_t kb,
                                                int64_t t0, int64_t pos0) {
    if (i < nrow) {
        const int64_t j = a.sel ? codes[i - kb] : i;
        return a.rows + (size_t(b) * a.row_cap + size_t(j)) * MD;
    }
    const int64_t t = t0 + (i - nrow);
    if (t >= pos0) return a.kv_new + (size_t(b) * a.S + size_t(t - pos0)) * MD;
    return a.ring + (size_t(b) * a.W + size_t(t % a.W)) * MD;
}

__global__ void __launch_bounds__(256)
attn_mfma_kernel(AttnMfmaArgs a, SeqInts pos0v, SeqInts n_rows) {
    __shared__ __attribute__((aligned(16))) unsigned char ktile[MKT * KPITCH];
    __shared__ __attribute__((aligned(16))) unsigned char ptile[MH * PPITCH];
    __shared__ float xch[2][2][MH];       // [max | sum][key half][head]
    __shared__ int32_t codes[MAX_CODES];
    __shared__ int32_t scan[256];

    const int b = blockIdx.z;
    const int64_t s = blockIdx.y;
    const int split = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int mt = w >> 1, nt = w & 1;    // head half; key half (QK) and dim half (PV)
    const int l32 = lane & 31, hi = lane >> 5;
    const int64_t pos0 = pos0v.v[b];
    const int64_t p = pos0 + s;

    int64_t nv = 0;
    if (a.r > 0 && a.rows != nullptr) {
        nv = (p + 1) / a.r;
        if (nv > n_rows.v[b]) nv = n_rows.v[b];
    }
    const int64_t t0 = p - a.W + 1 > 0 ? p - a.W + 1 : 0;
    const int64_t nwin = p - t0 + 1;
    const int64_t kb = int64_t(split) * a.keys_per_split;
    int64_t nrow = nv;
    if (a.sel != nullptr) {
        // compact the valid entries of the selection row, in order; keep those in this split
        const int32_t* sr = a.sel + (size_t(b) * a.S + size_t(s)) * a.k;
        const int per = (a.k + 255) / 256;
        const int e0 = tid * per, e1 = e0 + per < a.k ? e0 + per : a.k;
        int cnt = 0;
        for (int e = e0; e < e1; ++e) {
            const int32_t j = sr[e];
            cnt += (j >= 0 && j < nv);
        }
        scan[tid] = cnt;
        __syncthreads();
        for (int off = 1; off < 256; off <<= 1) {      // inclusive scan (Hillis-Steele)
            const int v = tid >= off ? scan[tid - off] : 0;
            __syncthreads();
            scan[tid] += v;
            __syncthreads();
        }
        nrow = scan[255];
        int64_t pos = scan[tid] - cnt;
        for (int e = e0; e < e1; ++e) {
            const int32_t j = sr[e];
            if (j >= 0 && j < nv) {
                if (pos >= kb && pos < kb + a.keys_per_split) codes[pos - kb] = j;
                ++pos;
            }
        }
        __syncthreads();
    }
    const int64_t nk = nrow + nwin;
    const size_t pbase = ((size_t(b) * a.S + size_t(s)) * a.n_splits + split) * MH;
    if (kb >= nk) {                                   // nothing in this split
        if (tid < MH) {
            a.part_ml[(pbase + tid) * 2 + 0] = -INFINITY;
            a.part_ml[(pbase + tid) * 2 + 1] = 0.f;
        }
        return;
    }
    const int64_t ke = kb + a.keys_per_split < nk ? kb + a.keys_per_split : nk;

    // this wave's 32 heads of q, as MFMA A fragments over all 512 dims
    bf16x8 qa[MD / 16];
    {
        const bf16* qh = a.q + ((size_t(b) * a.S + size_t(s)) * MH + 32 * mt + l32) * MD + 8 * hi;
#pragma unroll
        for (int ks = 0; ks < MD / 16; ++ks) qa[ks] = load_bf16x8(qh + ks * 16);
    }
    floatx16 o[8];
#pragma unroll
    for (int n8 = 0; n8 < 8; ++n8)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[n8][i] = 0.f;
    float m_run[16], l_run[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        m_run[i] = -INFINITY;
        l_run[i] = 0.f;
    }

    for (int64_t tb = kb; tb < ke; tb += MKT) {
        const int nkt = ke - tb < MKT ? int(ke - tb) : MKT;
        // stage the tile: each wave copies whole 1 KB rows (16 B per lane)
#pragma unroll 4
        for (int i = 0; i < MKT / 4; ++i) {
            const int kk = w + 4 * i;
            uint4 v = make_uint4(0, 0, 0, 0);
            if (kk < nkt) {
                const bf16* src = mfma_key(a, b, tb + kk, nrow, codes, kb, t0, pos0);
                v = *reinterpret_cast<const uint4*>(src + lane * 8);
            }
            store16(ktile + kk * KPITCH + lane * 16, v);
        }
        __syncthreads();

        // S = Q K^T for (heads 32mt.., keys 32nt..)
        floatx16 sacc;
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[i] = 0.f;
        const unsigned char* kr = ktile + (32 * nt + l32) * KPITCH + 16 * hi;
#pragma unroll
        for (int ks = 0; ks < MD / 16; ++ks) sacc = mfma32x32x16(qa[ks], load_bf16x8(kr + ks * 32), sacc);
        const bool kvalid = 32 * nt + l32 < nkt;
        float sv[16], red[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            sv[i] = kvalid ? sacc[i] * a.scale_log2 : -INFINITY;
            red[i] = sv[i];
        }
#pragma unroll
        for (int off = 1; off < 32; off <<= 1)
#pragma unroll
            for (int i = 0; i < 16; ++i) red[i] = fmaxf(red[i], __shfl_xor(red[i], off, 64));
        if (l32 == 0)
#pragma unroll
            for (int i = 0; i < 16; ++i) xch[0][nt][32 * mt + c_row(i, lane)] = red[i];
        __syncthreads();
        float alpha[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const float tmax = fmaxf(red[i], xch[0][nt ^ 1][32 * mt + c_row(i, lane)]);
            const float mnew = fmaxf(m_run[i], tmax);
            alpha[i] = exp2f(m_run[i] - mnew);
            m_run[i] = mnew;
            const float pv = exp2f(sv[i] - mnew);
            red[i] = pv;
            *reinterpret_cast<uint16_t*>(ptile + (32 * mt + c_row(i, lane)) * PPITCH +
                                         (32 * nt + l32) * 2) = bf16_bits(pv);
        }
#pragma unroll
        for (int off = 1; off < 32; off <<= 1)
#pragma unroll
            for (int i = 0; i < 16; ++i) red[i] += __shfl_xor(red[i], off, 64);
        if (l32 == 0)
#pragma unroll
            for (int i = 0; i < 16; ++i) xch[1][nt][32 * mt + c_row(i, lane)] = red[i];
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 16; ++i)
            l_run[i] = l_run[i] * alpha[i] + red[i] + xch[1][nt ^ 1][32 * mt + c_row(i, lane)];

        // O += P V for (heads 32mt.., dims 256nt..)
#pragma unroll
        for (int n8 = 0; n8 < 8; ++n8)
#pragma unroll
            for (int i = 0; i < 16; ++i) o[n8][i] *= alpha[i];
        const unsigned char* pr = ptile + (32 * mt + l32) * PPITCH + 16 * hi;
#pragma unroll
        for (int ks = 0; ks < MKT / 16; ++ks) {
            const bf16x8 pa = load_bf16x8(pr + ks * 32);
            const unsigned char* vr = ktile + (16 * ks + 8 * hi) * KPITCH + (256 * nt + l32) * 2;
#pragma unroll
            for (int n8 = 0; n8 < 8; ++n8) {
                bf16x8 vb;
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    vb[e] = *reinterpret_cast<const __bf16*>(vr + e * KPITCH + n8 * 64);
                o[n8] = mfma32x32x16(pa, vb, o[n8]);
            }
        }
        __syncthreads();
    }

    if (a.n_splits == 1) {
        float f[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const float z = a.sinks[32 * mt + c_row(i, lane)] * kLog2e;
            const float mf = fmaxf(m_run[i], z);
            const float sc = exp2f(m_run[i] - mf);
            f[i] = sc / (l_run[i] * sc + exp2f(z - mf));
        }
        bf16* ob = a.out + (size_t(b) * a.S + size_t(s)) * MH * MD + 256 * nt + l32;
#pragma unroll
        for (int n8 = 0; n8 < 8; ++n8)
#pragma unroll
            for (int i = 0; i < 16; ++i)
                ob[(32 * mt + c_row(i, lane)) * MD + 32 * n8] = from_f32<bf16>(o[n8][i] * f[i]);
    } else {
        if (nt == 0 && l32 == 0)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const size_t h = pbase + 32 * mt + c_row(i, lane);
                a.part_ml[h * 2 + 0] = m_run[i];
                a.part_ml[h * 2 + 1] = l_run[i];
            }
        float* po = a.part_o + pbase * MD + 256 * nt + l32;
#pragma unroll
        for (int n8 = 0; n8 < 8; ++n8)
#pragma unroll
            for (int i = 0; i < 16; ++i) po[(32 * mt + c_row(i, lane)) * MD + 32 * n8] = o[n8][i];
    }
}

// Merge the split partials of one query with the sink: weights 2^(m_i - M) / den.
__global__ void __launch_bounds__(256)
attn_combine_kernel(AttnMfmaArgs a) {
    __shared__ float wgt[MAX_SPLITS][MH];
    const int b = blockIdx.y;
    const int64_t s = blockIdx.x;
    const size_t base = (size_t(b) * a.S + size_t(s)) * a.n_splits;
    const int tid = threadIdx.x;
    if (tid < MH) {
        const float z = a.sinks[tid] * kLog2e;
        float M = z;
        for (int sp = 0; sp < a.n_splits; ++sp) M = fmaxf(M, a.part_ml[((base + sp) * MH + tid) * 2]);
        float den = exp2f(z - M);
        for (int sp = 0; sp < a.n_splits; ++sp) {
            const float m = a.part_ml[((base + sp) * MH + tid) * 2];
            const float e = m == -INFINITY ? 0.f : exp2f(m - M);
            den += a.part_ml[((base + sp) * MH + tid) * 2 + 1] * e;
            wgt[sp][tid] = e;
        }
        const float inv = 1.f / den;
        for (int sp = 0; sp < a.n_splits; ++sp) wgt[sp][tid] *= inv;
    }
    __syncthreads();
    bf16* ob = a.out + (size_t(b) * a.S + size_t(s)) * MH * MD;
    for (int idx = tid; idx < MH * MD; idx += blockDim.x) {
        const int h = idx / MD;
        float acc = 0.f;
        for (int sp = 0; sp < a.n_splits; ++sp) {
            const float wv = wgt[sp][h];
            if (wv != 0.f) acc += wv * a.part_o[(base + sp) * MH * MD + idx];
        }
        ob[idx] = from_f32<bf16>(acc);
    }
}

// Splits per query: enough workgroups to cover the chip when there are few queries.
int mfma_splits(int64_t queries, int64_t nk_max, int* keys_per_split) {
    const int64_t tiles = (nk_max + MKT - 1) / MKT;
    int64_t want = queries >= 512 ? 1 : (512 + queries - 1) / queries;
    if (want > MAX_SPLITS) want = MAX_SPLITS;
    if (want > tiles) want = tiles;
    if (want < 1) want = 1;
    const int64_t tiles_per = (tiles + want - 1) / want;
    *keys_per_split = int(tiles_per * MKT);
    return int((tiles + tiles_per - 1) / tiles_per);
}

bool use_mfma(bool bf16_, int H, int D) { return bf16_ && H == MH && D == MD; }

hipError_t run_mfma(const AttnJob& j, hipStream_t st) {
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
        AttnMfmaArgs a;
        a.q = static_cast<const bf16*>(j.q) + qoff * MH * MD;
        a.kv_new = static_cast<const bf16*>(j.kv_new) + qoff * MD;
        a.ring = static_cast<const bf16*>(j.ring) + size_t(b0) * j.W * MD;
        a.rows = j.rows ? static_cast<const bf16*>(j.rows) + size_t(b0) * j.row_cap * MD : nullptr;
        a.row_cap = j.row_cap;
        a.sel = j.sel ? j.sel + qoff * j.k : nullptr;
        a.k = j.k;
        a.sinks = j.sinks;
        a.out = static_cast<bf16*>(j.out) + qoff * MH * MD;
        a.S = j.S;
        a.W = j.W;
        a.r = j.r;
        a.scale_log2 = j.scale * kLog2e;
        a.n_splits = mfma_splits(int64_t(nb) * j.S, nrow_max + j.W, &a.keys_per_split);
        float* ws = static_cast<float*>(j.ws);
        a.part_ml = ws;
        a.part_o = ws + size_t(nb) * j.S * a.n_splits * MH * 2;
        trace_begin("attn_mfma", st);
        hipLaunchKernelGGL(attn_mfma_kernel, dim3(unsigned(a.n_splits), unsigned(j.S), nb), dim3(256),
                           0, st, a, pos, nr);
        trace_end("attn_mfma", st);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        if (a.n_splits > 1) {
            trace_begin("attn_combine", st);
            hipLaunchKernelGGL(attn_combine_kernel, dim3(unsigned(j.S), nb), dim3(256), 0, st, a);
            trace_end("attn_combine", st);
            e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
        AttnArgs<bf16> ra;
        ra.D = MD; ra.W = j.W; ra.S = j.S;
        ra.kv_new = a.kv_new;
        ra.ring = static_cast<bf16*>(j.ring) + size_t(b0) * j.W * MD;
        const int64_t nupd = std::min<int64_t>(j.S, j.W);
        trace_begin("ring_update", st);
        hipLaunchKernelGGL(ring_update_kernel<bf16>, dim3(unsigned(nupd), nb), dim3(256), 0, st, ra, pos);
        trace_end("ring_update", st);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace

int64_t attn_max_keys(bool bf16_, int H, int D, int k, bool has_sel) {
    if (use_mfma(bf16_, H, D)) return has_sel && k > MAX_CODES ? 0 : (int64_t(1) << 31) - 1;
    return int64_t((kAttnLdsMax - size_t(D) * 4) / 8);
}

// Partials of the split-key path: for every query, up to the split count mfma_splits picks
// for B*S queries, H (max, sum) pairs and an H x D fp32 output.
size_t attn_workspace_bytes(bool bf16_, int H, int D, int W, int r, int k, int batch, int64_t S) {
    (void)W; (void)r; (void)k;
    if (!use_mfma(bf16_, H, D)) return 0;
    size_t total = 0;
    for (int b0 = 0; b0 < batch; b0 += kSeqSlice) {
        const int64_t q = int64_t(std::min(kSeqSlice, batch - b0)) * S;
        if (q >= 512) continue;
        const int64_t splits = std::min<int64_t>(MAX_SPLITS, (512 + q - 1) / q);
        total = std::max(total, size_t(q) * splits * MH * (2 + MD) * sizeof(float));
    }
    return total;
}

hipError_t launch_attention(const AttnJob& j, hipStream_t s) {
    if (use_mfma(j.bf16, j.H, j.D)) return run_mfma(j, s);
    return j.bf16 ? run<bf16>(j, s) : run<float>(j, s);
}

}  // namespace dsv4
