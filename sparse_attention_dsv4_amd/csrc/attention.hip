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
// LDS bytes per key row: 1024 + 48 makes both the Q.K^T operand reads (16 rows x 16 B) and
// the transposed P.V operand reads (4 rows x 32 B per 16-lane group) bank-conflict free.
constexpr int KPITCH = MD * 2 + 48;
constexpr int KBUF = MKT * KPITCH;        // one key tile
constexpr int PPITCH = MKT * 2 + 16;      // LDS bytes per head row of P
constexpr int OPITCH = MD * 4 + 16;       // LDS bytes per head row of staged fp32 output
constexpr int MAX_CODES = 1024;           // selected rows one workgroup may list
constexpr int MAX_SPLITS = 32;
constexpr float kLog2e = 1.4426950408889634f;

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef __attribute__((address_space(3))) unsigned char lds_u8;

// Direct global -> LDS copy of 16 bytes per lane: lane l's bytes land at lds_row + 16 l
// (global_load_lds_dwordx4; the LDS base goes through m0 and must be wave-uniform).  Issued
// as inline asm so the compiler does not order later LDS reads of the *other* key buffer
// behind it; the caller waits with vmcnt(0) before the barrier that publishes the tile.
__device__ __forceinline__ void dma16(const void* gptr, const unsigned char* lds_row) {
    const uint32_t la = __builtin_amdgcn_readfirstlane(uint32_t(size_t((const lds_u8*)lds_row)));
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
                 :: "s"(la), "v"(gptr) : "memory", "m0");
}
__device__ __forceinline__ void wait_vm() { __builtin_amdgcn_s_waitcnt(0x0F70); }   // vmcnt(0)

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

// Barrier for LDS exchanges inside a tile: waits for this wave's LDS operations only, so
// the next tile's direct-to-LDS loads stay in flight.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0); vmcnt and expcnt unconstrained
    __builtin_amdgcn_s_barrier();
}

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

struct TileCtx {
    int b, w, lane, mt, nt, l32, hi;
    int64_t nrow, kb, t0, pos0;
};

// Enqueue the direct-to-LDS copy of keys [tb, tb + nkt) (one 1 KB row per wave instruction)
// and zero the unused rows of a partial tile.
__device__ __forceinline__ void load_tile(const AttnMfmaArgs& a, const TileCtx& c,
                                          const int32_t* codes, unsigned char* buf, int64_t tb,
                                          int nkt) {
#pragma unroll 4
    for (int i = 0; i < MKT / 4; ++i) {
        const int kk = c.w + 4 * i;
        if (kk < nkt) {
            const bf16* src = mfma_key(a, c.b, tb + kk, c.nrow, codes, c.kb, c.t0, c.pos0);
            dma16(src + c.lane * 8, buf + kk * KPITCH);
        } else {
            store16(buf + kk * KPITCH + c.lane * 16, make_uint4(0, 0, 0, 0));
        }
    }
}

// Lazy rescaling: the running reference max of a head moves only when a tile's max exceeds
// it by more than kLazy (log2 units), so most tiles skip rescaling the output accumulators.
// Every exponent stays <= 2^kLazy, far inside fp32 and bf16 range, and the final division
// uses the same reference, so the result is unchanged.
constexpr float kLazy = 8.0f;

__device__ __forceinline__ uint2 pack4_bf16(float a, float b, float c, float d) {
    return make_uint2(uint32_t(bf16_bits(a)) | (uint32_t(bf16_bits(b)) << 16),
                      uint32_t(bf16_bits(c)) | (uint32_t(bf16_bits(d)) << 16));
}

// One key tile.  Wave (mt, nt): S^T = K Q^T for keys 32nt.. x heads 32mt.., so lane l owns
// head 32mt + l%32 and 16 keys; O^T += V^T P^T for dims 256nt.. x the same heads.
__device__ __forceinline__ void attend_tile(const AttnMfmaArgs& a, const TileCtx& c,
                                            const unsigned char* buf, unsigned char* ptile,
                                            float (*xch)[2][MH], const bf16x8* qa, floatx16* o,
                                            float& m_run, float& l_run, int nkt) {
    const int mt = c.mt, nt = c.nt, lane = c.lane, l32 = c.l32, hi = c.hi;
    const int head = 32 * mt + l32;
    floatx16 st;
#pragma unroll
    for (int i = 0; i < 16; ++i) st[i] = 0.f;
    const unsigned char* kr = buf + (32 * nt + l32) * KPITCH + 16 * hi;
#pragma unroll
    for (int ks = 0; ks < MD / 16; ++ks) st = mfma32x32x16(load_bf16x8(kr + ks * 32), qa[ks], st);
    float sv[16];
    float lmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const bool kvalid = 32 * nt + c_row(i, lane) < nkt;
        sv[i] = kvalid ? st[i] * a.scale_log2 : -INFINITY;
        lmax = fmaxf(lmax, sv[i]);
    }
    lmax = fmaxf(lmax, __shfl_xor(lmax, 32, 64));      // this key half, this head
    if (hi == 0) xch[0][nt][head] = lmax;
    lds_barrier();
    const float tmax = fmaxf(lmax, xch[0][nt ^ 1][head]);
    // the decision depends only on (m_run, tmax), equal in both waves of this head half
    if (tmax > m_run + kLazy) {
        const float alpha = exp2f(m_run - tmax);        // 0 on the first tile
        m_run = tmax;
        l_run *= alpha;
#pragma unroll
        for (int n8 = 0; n8 < 8; ++n8)
#pragma unroll
            for (int i = 0; i < 16; ++i) o[n8][i] *= alpha;
    }
    float psum = 0.f;
    unsigned char* prow = ptile + head * PPITCH + (32 * nt + 4 * hi) * 2;
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {                    // registers 4 q4 .. 4 q4 + 3: 4 consecutive keys
        float p4[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            p4[r] = exp2f(sv[4 * q4 + r] - m_run);
            psum += p4[r];
        }
        *reinterpret_cast<uint2*>(prow + 16 * q4) = pack4_bf16(p4[0], p4[1], p4[2], p4[3]);
    }
    l_run += psum + __shfl_xor(psum, 32, 64);          // this wave's key half only
    lds_barrier();
    // O^T += V^T P^T: A = 32 dims x 16 keys of V (two transposed reads), B = P^T fragment
    const unsigned char* pr = ptile + head * PPITCH + 16 * hi;
    const int j16 = lane & 15;
    const unsigned char* vb0 = buf + (8 * hi + (j16 >> 2)) * KPITCH +
                               (256 * nt + 16 * ((lane >> 4) & 1) + 4 * (j16 & 3)) * 2;
#pragma unroll
    for (int ks = 0; ks < MKT / 16; ++ks) {
        const bf16x8 pb = load_bf16x8(pr + ks * 32);
#pragma unroll
        for (int n8 = 0; n8 < 8; ++n8) {
            const unsigned char* vp = vb0 + 16 * ks * KPITCH + n8 * 64;
            const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(vp));
            const v4i16 up = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(vp + 4 * KPITCH));
            bf16x8 va;
            __builtin_memcpy(&va, &lo, 8);
            __builtin_memcpy(reinterpret_cast<char*>(&va) + 8, &up, 8);
            o[n8] = mfma32x32x16(va, pb, o[n8]);
        }
    }
}

__global__ void __launch_bounds__(256)
attn_mfma_kernel(AttnMfmaArgs a, SeqInts pos0v, SeqInts n_rows) {
    __shared__ __attribute__((aligned(16))) unsigned char kbuf[2][KBUF];
    __shared__ __attribute__((aligned(16))) unsigned char ptile[MH * PPITCH];
    __shared__ float xch[2][2][MH];       // [max | sum][key half][head]
    __shared__ int32_t codes[MAX_CODES];
    __shared__ int32_t scan[256];

    TileCtx c;
    c.b = blockIdx.z;
    const int64_t s = blockIdx.y;
    const int split = blockIdx.x;
    const int tid = threadIdx.x;
    c.lane = tid & 63;
    c.w = tid >> 6;
    c.mt = c.w >> 1;                      // head half
    c.nt = c.w & 1;                       // key half in Q.K^T, dim half in P.V
    c.l32 = c.lane & 31;
    c.hi = c.lane >> 5;
    const int b = c.b;
    c.pos0 = pos0v.v[b];
    const int64_t p = c.pos0 + s;

    int64_t nv = 0;
    if (a.r > 0 && a.rows != nullptr) {
        nv = (p + 1) / a.r;
        if (nv > n_rows.v[b]) nv = n_rows.v[b];
    }
    c.t0 = p - a.W + 1 > 0 ? p - a.W + 1 : 0;
    const int64_t nwin = p - c.t0 + 1;
    c.kb = int64_t(split) * a.keys_per_split;
    c.nrow = nv;
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
        c.nrow = scan[255];
        int64_t pos = scan[tid] - cnt;
        for (int e = e0; e < e1; ++e) {
            const int32_t j = sr[e];
            if (j >= 0 && j < nv) {
                if (pos >= c.kb && pos < c.kb + a.keys_per_split) codes[pos - c.kb] = j;
                ++pos;
            }
        }
        __syncthreads();
    }
    const int64_t nk = c.nrow + nwin;
    const size_t pbase = ((size_t(b) * a.S + size_t(s)) * a.n_splits + split) * MH;
    if (a.S == 1 && split == 0) {
        // decode: store the new latent in its ring slot here.  Slot p % W holds token p - W,
        // which no query of this launch reads (its window is p-W+1 .. p, with p itself
        // taken from kv_new), so the store cannot race the key loads.
        const uint4* src = reinterpret_cast<const uint4*>(a.kv_new + size_t(b) * MD);
        uint4* dst = reinterpret_cast<uint4*>(const_cast<bf16*>(a.ring) + (size_t(b) * a.W + size_t(p % a.W)) * MD);
        if (tid < MD / 8) dst[tid] = src[tid];
    }
    if (c.kb >= nk) {                                 // nothing in this split
        if (tid < MH) {
            a.part_ml[(pbase + tid) * 2 + 0] = -INFINITY;
            a.part_ml[(pbase + tid) * 2 + 1] = 0.f;
        }
        return;
    }
    const int64_t ke = c.kb + a.keys_per_split < nk ? c.kb + a.keys_per_split : nk;
    const int ntiles = int((ke - c.kb + MKT - 1) / MKT);
    auto tile_keys = [&](int t) -> int {
        const int64_t left = ke - (c.kb + int64_t(t) * MKT);
        return left < MKT ? int(left) : MKT;
    };

    load_tile(a, c, codes, kbuf[0], c.kb, tile_keys(0));
    // this wave's 32 heads of q, as MFMA A fragments over all 512 dims
    bf16x8 qa[MD / 16];
    {
        const bf16* qh = a.q + ((size_t(b) * a.S + size_t(s)) * MH + 32 * c.mt + c.l32) * MD + 8 * c.hi;
#pragma unroll
        for (int ks = 0; ks < MD / 16; ++ks) qa[ks] = load_bf16x8(qh + ks * 16);
    }
    floatx16 o[8];
#pragma unroll
    for (int n8 = 0; n8 < 8; ++n8)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[n8][i] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;   // head 32mt + l%32; l_run over this key half
    wait_vm();
    __syncthreads();

    for (int t = 0; t < ntiles; ++t) {
        if (t + 1 < ntiles) load_tile(a, c, codes, kbuf[(t + 1) & 1], c.kb + int64_t(t + 1) * MKT, tile_keys(t + 1));
        attend_tile(a, c, kbuf[t & 1], ptile, xch, qa, o, m_run, l_run, tile_keys(t));
        wait_vm();                        // the next tile has landed
        __syncthreads();                  // ... for every wave; and all are done with this one
    }

    // total denominator of this lane's head: both key halves
    const int mt = c.mt, nt = c.nt, lane = c.lane, l32 = c.l32, hi = c.hi;
    const int head = 32 * mt + l32;
    if (hi == 0) xch[1][nt][head] = l_run;
    __syncthreads();
    const float l_tot = l_run + xch[1][nt ^ 1][head];
    // stage the result in LDS (the key buffers are free now), then coalesced 16-byte stores;
    // lane l holds head `head`, dims 256nt + 32n8 + c_row(i, l) (4 consecutive per q4)
    if (a.n_splits == 1) {
        const float z = a.sinks[head] * kLog2e;
        const float mf = fmaxf(m_run, z);
        const float sc = exp2f(m_run - mf);
        const float f = sc / (l_tot * sc + exp2f(z - mf));
        unsigned char* stage = kbuf[0];                 // bf16 [head][dim], 1040-byte rows
#pragma unroll
        for (int n8 = 0; n8 < 8; ++n8)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4)
                *reinterpret_cast<uint2*>(stage + head * (MD * 2 + 16) +
                                          (256 * nt + 32 * n8 + 8 * q4 + 4 * hi) * 2) =
                    pack4_bf16(o[n8][4 * q4] * f, o[n8][4 * q4 + 1] * f, o[n8][4 * q4 + 2] * f,
                               o[n8][4 * q4 + 3] * f);
        __syncthreads();
        bf16* ob = a.out + (size_t(b) * a.S + size_t(s)) * MH * MD;
        for (int idx = tid; idx < MH * MD / 8; idx += 256) {
            const int h = idx / (MD / 8), d8 = idx % (MD / 8);
            store16(ob + size_t(h) * MD + d8 * 8,
                    *reinterpret_cast<const uint4*>(stage + h * (MD * 2 + 16) + d8 * 16));
        }
    } else {
        if (nt == 0 && hi == 0) {
            a.part_ml[(pbase + head) * 2 + 0] = m_run;
            a.part_ml[(pbase + head) * 2 + 1] = l_tot;
        }
        // fp32 [head][dim]: heads 0..31 staged in kbuf[0], 32..63 in kbuf[1] (32 x 2064 B each)
        unsigned char* st = kbuf[mt];
#pragma unroll
        for (int n8 = 0; n8 < 8; ++n8)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4)
                *reinterpret_cast<float4*>(st + l32 * OPITCH + (256 * nt + 32 * n8 + 8 * q4 + 4 * hi) * 4) =
                    make_float4(o[n8][4 * q4], o[n8][4 * q4 + 1], o[n8][4 * q4 + 2], o[n8][4 * q4 + 3]);
        __syncthreads();
        float* po = a.part_o + pbase * MD;
        for (int idx = tid; idx < MH * MD / 4; idx += 256) {
            const int h = idx / (MD / 4), d4 = idx % (MD / 4);
            const unsigned char* sp = kbuf[h >> 5] + (h & 31) * OPITCH + d4 * 16;
            store16(po + size_t(h) * MD + d4 * 4, *reinterpret_cast<const uint4*>(sp));
        }
    }
}

// Merge the split partials of one query with the sink: weights 2^(m_i - M) / den.  One
// workgroup per (query, group of 8 heads).
__global__ void __launch_bounds__(256)
attn_combine_kernel(AttnMfmaArgs a) {
    __shared__ float wgt[MAX_SPLITS][8];
    const int b = blockIdx.z;
    const int64_t s = blockIdx.y;
    const int h0 = blockIdx.x * 8;
    const size_t base = (size_t(b) * a.S + size_t(s)) * a.n_splits;
    const int tid = threadIdx.x;
    if (tid < 8) {
        const int h = h0 + tid;
        const float z = a.sinks[h] * kLog2e;
        float M = z;
        for (int sp = 0; sp < a.n_splits; ++sp) M = fmaxf(M, a.part_ml[((base + sp) * MH + h) * 2]);
        float den = exp2f(z - M);
        for (int sp = 0; sp < a.n_splits; ++sp) {
            const float m = a.part_ml[((base + sp) * MH + h) * 2];
            const float e = m == -INFINITY ? 0.f : exp2f(m - M);
            den += a.part_ml[((base + sp) * MH + h) * 2 + 1] * e;
            wgt[sp][tid] = e;
        }
        const float inv = 1.f / den;
        for (int sp = 0; sp < a.n_splits; ++sp) wgt[sp][tid] *= inv;
    }
    __syncthreads();
    // 8 heads x 512 dims = 1024 float4 lanes of work; 4 per thread
    bf16* ob = a.out + (size_t(b) * a.S + size_t(s)) * MH * MD + size_t(h0) * MD;
    for (int idx = tid; idx < 8 * MD / 4; idx += 256) {
        const int hh = idx / (MD / 4), d4 = idx % (MD / 4);
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int sp = 0; sp < a.n_splits; ++sp) {
            const float wv = wgt[sp][hh];
            if (wv != 0.f) {
                const float4 v = *reinterpret_cast<const float4*>(a.part_o + ((base + sp) * MH + h0 + hh) * MD + d4 * 4);
                acc.x += wv * v.x;
                acc.y += wv * v.y;
                acc.z += wv * v.z;
                acc.w += wv * v.w;
            }
        }
        const uint32_t lo = uint32_t(bf16_bits(acc.x)) | (uint32_t(bf16_bits(acc.y)) << 16);
        const uint32_t up = uint32_t(bf16_bits(acc.z)) | (uint32_t(bf16_bits(acc.w)) << 16);
        *reinterpret_cast<uint2*>(ob + size_t(hh) * MD + d4 * 4) = make_uint2(lo, up);
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
            hipLaunchKernelGGL(attn_combine_kernel, dim3(MH / 8, unsigned(j.S), nb), dim3(256), 0, st, a);
            trace_end("attn_combine", st);
            e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
        if (j.S == 1) continue;          // the attention kernel stored the decode token
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
