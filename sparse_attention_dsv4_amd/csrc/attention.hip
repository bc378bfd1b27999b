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
// mfma kernels (bf16, 64 heads, 512 latent), all on v_mfma_f32_16x16x32_bf16 with the key
// rows copied straight from memory into LDS tiles: prefill runs one workgroup of 8 waves per
// (query, key split) over 64-key tiles; decode runs one workgroup per (sequence, group of 16
// heads, key split) holding a split of up to 128 keys in LDS whole, and longer splits (large
// batches) in two 64-key buffers, the next filling while one is scored.  The softmax is in
// base 2 with fp32 max and sum; P is rounded to bf16 before P*V (the pages' reference kernel
// does the same, MTPLX PR #216 "Decode path").  A query whose key list is split over several
// workgroups writes partials (fp32 max and sum; the unnormalised output in bf16 for decode,
// fp32 for prefill) that attn_combine_kernel merges with the sink; a query handled by one
// workgroup normalises and writes its output.
//
// The window ring holds Wr >= W slots (token t in slot t % Wr): the W attended tokens plus
// those retained for rollback.  The ring update runs after the attention kernel on the
// stream: writing token t evicts token t - Wr, which an earlier query of the same call may
// still need.
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
    int Wr;            // ring slots
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
    return a.ring + (size_t(b) * a.Wr + size_t(t % a.Wr)) * a.D;
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
    const int64_t first = a.S > a.Wr ? pos0 + a.S - a.Wr : pos0;
    const int64_t t = first + blockIdx.x;
    if (t >= pos0 + a.S) return;
    const T* src = a.kv_new + (size_t(b) * a.S + size_t(t - pos0)) * a.D;
    T* dst = a.ring + (size_t(b) * a.Wr + size_t(t % a.Wr)) * a.D;
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
        a.H = j.H; a.D = j.D; a.W = j.W; a.Wr = j.Wr; a.r = j.r; a.k = j.k; a.scale = j.scale;
        a.q = static_cast<const T*>(j.q) + qoff * j.H * j.D;
        a.kv_new = static_cast<const T*>(j.kv_new) + qoff * j.D;
        a.ring = static_cast<T*>(j.ring) + size_t(b0) * j.Wr * j.D;
        a.rows = j.rows ? static_cast<const T*>(j.rows) + size_t(b0) * j.row_cap * j.D : nullptr;
        a.row_cap = j.row_cap;
        a.sel = j.sel ? j.sel + qoff * j.k : nullptr;
        a.sinks = j.sinks;
        a.out = static_cast<T*>(j.out) + qoff * j.H * j.D;
        a.S = j.S;
        a.nk_cap = int(nrow_max + j.W);
        const size_t lds = size_t(j.D) * 4 + size_t(a.nk_cap) * 8;
        DSV4_LAUNCH("attn_generic", attn_generic_kernel<T>, dim3(unsigned(j.S), unsigned(j.H), nb),
                           dim3(kAttnThreads), lds, st, a, pos, nr);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        const int64_t nupd = std::min<int64_t>(j.S, j.Wr);
        DSV4_LAUNCH("ring_update", ring_update_kernel<T>, dim3(unsigned(nupd), nb), dim3(kAttnThreads), 0,
                           st, a, pos);
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
// The row's global base is wave-uniform (a scalar register pair) and each lane adds its own
// byte offset, so no per-lane 64-bit address arithmetic is spent on the copy.
__device__ __forceinline__ void dma16(const void* sbase, uint32_t voff, const unsigned char* lds_row) {
    const uint32_t la = __builtin_amdgcn_readfirstlane(uint32_t(size_t((const lds_u8*)lds_row)));
    // readfirstlane returns int: zero-extend each half (a sign-extended low half would
    // corrupt the upper word of an address whose bit 31 is set)
    const uint64_t gp = reinterpret_cast<uint64_t>(sbase);
    const uint64_t sb = uint64_t(uint32_t(__builtin_amdgcn_readfirstlane(uint32_t(gp)))) |
                        (uint64_t(uint32_t(__builtin_amdgcn_readfirstlane(uint32_t(gp >> 32)))) << 32);
    // s_nop 4: five wait states between the last (VALU) write of the base registers or m0 and
    // the load that reads them; the compiler does not look inside the asm for this hazard
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 4\n\tglobal_load_lds_dwordx4 %1, %2"
                 :: "s"(la), "v"(voff), "s"(sb) : "memory", "m0");
}
__device__ __forceinline__ void wait_vm() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

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
    int Wr;                               // ring slots (W + tokens retained for rollback)
    float scale_log2;                     // logit scale * log2(e)
    int keys_per_split, n_splits;
    float* part_ml;                       // [B][S][n_splits][H][2]  running max, sum
    float* part_o;                        // [B][S][n_splits][H][D]  unnormalised output
    // decode: compressor frontier stores of this token (lanes of a step completing no row)
    struct Front {
        bf16* state;                      // [B][2][nw][r][W]
        const bf16* a;                    // [B][W] kv lane, then gate lane
        const bf16* g;
        int r, nw, W;
        int vec;                          // W / 4 <= 256 and 16-byte aligned: vector copies
    } fr[2];
    int n_fr;
};

// Barrier for LDS exchanges inside a tile: waits for this wave's LDS operations only, so
// the next tile's direct-to-LDS loads stay in flight.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Where the keys of one query come from.  Key i of the query's list: the window tokens
// first, t0 + i for i < nwin, read from kv_new for tokens of this call and from ring slot
// t % W for earlier ones; then the compressed rows (rank i - nwin: the rank-th valid selected
// row, or row rank when every visible row is attended).  The window goes first because its
// sources are known before the selection is compacted.  All key and token indices fit in 32
// bits (the entry points cap positions below 2^31 and keys per query at 2^30).
struct TileCtx {
    int b, w, lane;
    int nrow, kb;             // attended rows; first key of this workgroup's split (or chunk)
    int nwin, kbs;            // window tokens; selection rank held in codes[0]
    int t0, pos0;             // first window token; first token of this call
    uint32_t slot0, W;        // ring slot of t0; ring length
    bool sel;
    const bf16* rows;         // this sequence's compressed rows
    const bf16* ring;         // this sequence's window ring
    const bf16* kv_new;       // this sequence's tokens of this call
};

__device__ __forceinline__ void key_ctx(TileCtx& c, const AttnMfmaArgs& a, int b, int t0, int pos0) {
    c.t0 = t0;
    c.pos0 = pos0;
    c.W = uint32_t(a.Wr);
    c.slot0 = uint32_t(t0) % c.W;
    c.sel = a.sel != nullptr;
    c.rows = a.rows ? a.rows + size_t(b) * size_t(a.row_cap) * MD : nullptr;
    c.ring = a.ring + size_t(b) * size_t(a.Wr) * MD;
    c.kv_new = a.kv_new + size_t(b) * size_t(a.S) * MD;
}

__device__ __forceinline__ const bf16* key_src(const TileCtx& c, const int32_t* codes, int i) {
    if (i < c.nwin) {
        const int t = c.t0 + i;
        if (t >= c.pos0) return c.kv_new + size_t(t - c.pos0) * MD;
        uint32_t slot = c.slot0 + uint32_t(i);      // < 2W: one wrap at most
        if (slot >= c.W) slot -= c.W;
        return c.ring + size_t(slot) * MD;
    }
    const int j = i - c.nwin;
    return c.rows + size_t(c.sel ? codes[j - c.kbs] : j) * MD;
}

// The next tile's copy, handed to prefill_tile so it can issue it in parts between MFMA groups
// (a wave issuing all of its copies at once stalls on the CU's load pipe and computes nothing).
struct NextTile {
    bool on;
    uint64_t src;
    unsigned char* buf;
    int nkt;
};

// The selection row as this thread's entries e = NT r + tid (-1 past k; k <= MAX_CODES), for
// a workgroup of NT threads.
constexpr int SEL_PER_THREAD = MAX_CODES / 256;
template <int NT = 256>
__device__ __forceinline__ void load_selection(const int32_t* sr, int k, int32_t (&selv)[MAX_CODES / NT]) {
#pragma unroll
    for (int r = 0; r < MAX_CODES / NT; ++r) {
        const int e = NT * r + int(threadIdx.x);
        selv[r] = e < k ? sr[e] : -1;
    }
}

// Compact the valid entries (0 <= j < nv) of one selection row, keeping their order: the
// entry of rank n goes to codes[n - kb] when kb <= n < kb + kps.  Returns the count of valid
// entries.  Ranks come from wave ballots; wsum holds 2 x (NT / 64) per-wave counts.  The
// barriers wait for LDS only, so global loads issued before (q fragments) stay in flight.
template <int NT = 256>
__device__ __forceinline__ int compact_selection(const int32_t (&selv)[MAX_CODES / NT], int k, int nv,
                                                 int kb, int kps, int32_t* codes, int* wsum) {
    constexpr int NW = NT / 64;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    int base = 0;
#pragma unroll
    for (int r = 0; r < MAX_CODES / NT; ++r) {
        if (NT * r >= k) break;
        const int32_t j = selv[r];
        const bool ok = j >= 0 && j < nv;
        const uint64_t m = __ballot(ok);
        int* ws = wsum + (r & 1) * NW;
        if (lane == 0) ws[w] = __popcll(m);
        lds_barrier();
        int off = base;
        for (int v = 0; v < w; ++v) off += ws[v];
        if (ok) {
            const int rank = off + __popcll(m & ((uint64_t(1) << lane) - 1));
            if (rank >= kb && rank < kb + kps) codes[rank - kb] = j;
        }
#pragma unroll
        for (int v = 0; v < NW; ++v) base += ws[v];
    }
    lds_barrier();
    return base;
}

// Lazy rescaling: the running reference max of a head moves only when a tile's max exceeds
// it by more than kLazy (log2 units), so most tiles skip rescaling the output accumulators.
// Every exponent stays <= 2^kLazy, far inside fp32 and bf16 range, and the final division
// uses the same reference, so the result is unchanged.
constexpr float kLazy = 8.0f;
constexpr int SXBYTES = 8 * 2 * 64 * 4 * 4;   // S^T partials: 8 (head group, dim half) x 2 subtiles x 64 lanes x 4 fp32


__device__ __forceinline__ uint2 pack4_bf16(float a, float b, float c, float d) {
    return make_uint2(pack2_bf16(a, b), pack2_bf16(c, d));
}

// 2^x on v_exp_f32 alone: the softmax arguments are <= kLazy and results below 2^-126 only
// lose weights that are far below bf16 resolution of the sum.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

constexpr int DHG = 16;                   // heads per 16x16x32 head group
typedef float floatx4 __attribute__((ext_vector_type(4)));

// v_mfma_f32_16x16x32_bf16: A lane l holds A[l%16][8 (l/16) + 0..7], B lane l holds
// B[8 (l/16) + 0..7][l%16], C lane l register i holds C[4 (l/16) + i][l%16].
__device__ __forceinline__ floatx4 mfma16x16x32(const bf16x8& a, const bf16x8& b, const floatx4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// ------------------------------------------------------------------ prefill path
// One workgroup of 8 waves per (query, key split).  Wave w holds heads 16 (w >> 1) .. +15
// and latent dims 256 (w & 1) .. +255, so its accumulators (16 heads x 256 dims fp32) and q
// fragments fit in 256 registers and two waves share each SIMD: while one waits on a copy,
// an LDS read or a barrier, the other issues MFMAs.  Per 64-key tile, on
// v_mfma_f32_16x16x32_bf16:
//   S^T = K Q^T over the wave's 256 dims for the 4 subtiles of 16 keys; the two dim halves
//   of a head group swap, through LDS, the partials of the key half each does not keep;
//   online softmax over the kept key half, the halves' maxima meet in LDS, P (bf16) to LDS;
//   O^T += V^T P^T for the wave's 256 dims over all 64 keys.
constexpr int PWAVES = 8;
constexpr int PTHREADS = 64 * PWAVES;

// Sources of a tile's rows for 8 waves: lane l < 8 of wave w finds the source of row w + 8 l.
__device__ __forceinline__ uint64_t prow_srcs(const TileCtx& c, const int32_t* codes, int tb, int nkt) {
    const int kk = c.w + PWAVES * (c.lane & 7);
    const bf16* src = kk < nkt ? key_src(c, codes, tb + kk) : c.ring;
    return reinterpret_cast<uint64_t>(src);
}

// Row w + 8 i of a tile (i wave-uniform): one 1 KB copy, or zeros past nkt.
__device__ __forceinline__ void prow_copy(const TileCtx& c, uint64_t src, unsigned char* buf, int nkt, int i) {
    const int kk = c.w + PWAVES * i;
    if (kk < nkt) {
        const uint64_t sp = uint64_t(uint32_t(__builtin_amdgcn_readlane(int(uint32_t(src)), i))) |
                            (uint64_t(uint32_t(__builtin_amdgcn_readlane(int(uint32_t(src >> 32)), i))) << 32);
        dma16(reinterpret_cast<const void*>(sp), uint32_t(c.lane) * 16, buf + kk * KPITCH);
    } else {
        store16(buf + kk * KPITCH + c.lane * 16, make_uint4(0, 0, 0, 0));
    }
}

__device__ __forceinline__ void prefill_load_tile(const TileCtx& c, const int32_t* codes, unsigned char* buf,
                                                  int tb, int nkt) {
    const uint64_t src = prow_srcs(c, codes, tb, nkt);
#pragma unroll
    for (int i = 0; i < MKT / PWAVES; ++i) prow_copy(c, src, buf, nkt, i);
}

// One key tile of the 8-wave prefill workgroup (see above).  nx: the next tile, whose 8 row
// copies of this wave go out two per subtile of the score product: early, so they have the
// rest of the tile to land (issued later, the last ones' latency showed at the tile's end).
__device__ __forceinline__ void prefill_tile(const AttnMfmaArgs& a, const TileCtx& c, const unsigned char* buf,
                                             unsigned char* ptile, float (*xch)[2][MH], const bf16x8 (&qa)[8],
                                             floatx4 (&o)[16], float& m_run, float& l_run, int nkt,
                                             const NextTile& nx) {
    const int lane = c.lane, l16 = lane & 15, g = lane >> 4;
    const int hq = c.w >> 1, nt = c.w & 1;
    const int head = DHG * hq + l16;
    // S^T partials over dims 256 nt .. +255: subtile u = keys 16 u .. 16 u + 15; the K operands
    // of subtile u+1 go out before the MFMAs of subtile u
    floatx4 sp[4];
    const unsigned char* kr0 = buf + l16 * KPITCH + 512 * nt + 16 * g;
    bf16x8 ka[2][8];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) ka[0][ks] = load_bf16x8(kr0 + ks * 64);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        if (u + 1 < 4) {
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) ka[(u + 1) & 1][ks] = load_bf16x8(kr0 + 16 * (u + 1) * KPITCH + ks * 64);
        }
        __builtin_amdgcn_sched_barrier(0);
        sp[u] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) sp[u] = mfma16x16x32(ka[u & 1][ks], qa[ks], sp[u]);
        if (nx.on) {
            prow_copy(c, nx.src, nx.buf, nx.nkt, 2 * u);
            prow_copy(c, nx.src, nx.buf, nx.nkt, 2 * u + 1);
        }
        __builtin_amdgcn_sched_barrier(0);
    }
    // keep key half nt (subtiles 2 nt, 2 nt + 1); the partner wave (other dims) gets the other
    // half.  Exchange region (head group, receiving dim half): [subtile][lane][4] fp32
    // (selects rather than indexing sp by nt: a register array indexed at run time would go
    // to scratch memory)
    const floatx4 keep0 = nt ? sp[2] : sp[0], keep1 = nt ? sp[3] : sp[1];
    const floatx4 give0 = nt ? sp[0] : sp[2], give1 = nt ? sp[1] : sp[3];
    float* sx = reinterpret_cast<float*>(ptile);
    {
        float* give = sx + (hq * 2 + (nt ^ 1)) * 512;
        *reinterpret_cast<floatx4*>(give + lane * 4) = give0;
        *reinterpret_cast<floatx4*>(give + (64 + lane) * 4) = give1;
    }
    lds_barrier();
    float sv[2][4];
    float lmax = -INFINITY;
    {
        const float* take = sx + (hq * 2 + nt) * 512;
#pragma unroll
        for (int v = 0; v < 2; ++v) {
            const floatx4 pv = *reinterpret_cast<const floatx4*>(take + (v * 64 + lane) * 4);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const bool kvalid = 32 * nt + 16 * v + 4 * g + i < nkt;
                sv[v][i] = kvalid ? ((v ? keep1[i] : keep0[i]) + pv[i]) * a.scale_log2 : -INFINITY;
                lmax = fmaxf(lmax, sv[v][i]);
            }
        }
    }
    lmax = max_xor32(max_xor16(lmax));                  // this key half, this head
    if (g == 0) xch[0][nt][head] = lmax;
    lds_barrier();
    const float tmax = fmaxf(lmax, xch[0][nt ^ 1][head]);
    // the decision depends only on (m_run, tmax), equal in both waves of this head group
    if (tmax > m_run + kLazy) {
        const float alpha = fast_exp2(m_run - tmax);    // 0 on the first tile
        m_run = tmax;
        l_run *= alpha;
#pragma unroll
        for (int m = 0; m < 16; ++m)
#pragma unroll
            for (int i = 0; i < 4; ++i) o[m][i] *= alpha;
    }
    float psum = 0.f;
    unsigned char* prow = ptile + head * PPITCH + (32 * nt + 4 * g) * 2;
#pragma unroll
    for (int v = 0; v < 2; ++v) {
        float p4[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            p4[i] = fast_exp2(sv[v][i] - m_run);
            psum += p4[i];
        }
        *reinterpret_cast<uint2*>(prow + 32 * v) = pack4_bf16(p4[0], p4[1], p4[2], p4[3]);
    }
    l_run += psum;                                      // this lane's keys only
    lds_barrier();
    // O^T for dims 256 nt .. +255 (16 tiles of 16 dims) over 2 k-steps of 32 keys; the V^T
    // operands of each group of 8 tiles go out before the previous group's MFMAs
    const unsigned char* pr = ptile + head * PPITCH + 16 * g;
    const bf16x8 pb0 = load_bf16x8(pr), pb1 = load_bf16x8(pr + 64);
    const unsigned char* vb0 = buf + (8 * g + (l16 >> 2)) * KPITCH + (256 * nt + 4 * (l16 & 3)) * 2;
    bf16x8 va[2][8];
    auto load_v = [&](int grp, bf16x8 (&dst)[8]) {     // grp = 2 ks + (tile half)
        const int ks = grp >> 1, m0 = 8 * (grp & 1);
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            const unsigned char* vp = vb0 + 32 * ks * KPITCH + (m0 + m) * 32;
            const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(vp));
            const v4i16 up = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(vp + 4 * KPITCH));
            __builtin_memcpy(&dst[m], &lo, 8);
            __builtin_memcpy(reinterpret_cast<char*>(&dst[m]) + 8, &up, 8);
        }
    };
    load_v(0, va[0]);
#pragma unroll
    for (int grp = 0; grp < 4; ++grp) {
        if (grp + 1 < 4) load_v(grp + 1, va[(grp + 1) & 1]);
        __builtin_amdgcn_sched_barrier(0);
        const bf16x8& pb = (grp >> 1) ? pb1 : pb0;
        const int m0 = 8 * (grp & 1);
#pragma unroll
        for (int m = 0; m < 8; ++m) o[m0 + m] = mfma16x16x32(va[grp & 1][m], pb, o[m0 + m]);
        __builtin_amdgcn_sched_barrier(0);
    }
}

__global__ void __launch_bounds__(PTHREADS)
attn_prefill_kernel(AttnMfmaArgs a, SeqInts pos0v, SeqInts n_rows) {
    __shared__ __attribute__((aligned(16))) unsigned char kbuf[2][KBUF];
    // S^T partials exchanged between the dim halves, then P [head][key] bf16
    __shared__ __attribute__((aligned(16))) unsigned char ptile[SXBYTES > MH * PPITCH ? SXBYTES : MH * PPITCH];
    __shared__ float xch[2][2][MH];       // [max | sum][key half][head]
    __shared__ int32_t codes[MAX_CODES];
    __shared__ int wsum[2 * PWAVES];

    TileCtx c;
    c.b = blockIdx.z;
    const int64_t s = blockIdx.y;
    const int split = blockIdx.x;
    const int tid = threadIdx.x;
    c.lane = tid & 63;
    c.w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: scalar branches
    const int b = c.b, lane = c.lane, l16 = lane & 15, g = lane >> 4;
    const int hq = c.w >> 1, nt = c.w & 1;
    const int head = DHG * hq + l16;
    const int pos0 = pos0v.v[b];
    const int p = pos0 + int(s);

    int nv = 0;
    if (a.r > 0 && a.rows != nullptr) {
        nv = (p + 1) / a.r;
        if (nv > n_rows.v[b]) nv = n_rows.v[b];
    }
    const int t0 = p - a.W + 1 > 0 ? p - a.W + 1 : 0;
    const int nwin = p - t0 + 1;
    key_ctx(c, a, b, t0, pos0);
    c.kb = split * a.keys_per_split;
    c.nwin = nwin;
    c.kbs = c.kb > nwin ? c.kb - nwin : 0;
    c.nrow = nv;
    // issue order: tile 0 when it holds window tokens only (its sources need no selection),
    // the selection entries, then this wave's q fragments (16 heads x 256 dims), so the
    // compaction waits for the selection only and the rest overlaps it
    const bool tile0_early = c.kb + MKT <= nwin;
    if (tile0_early) prefill_load_tile(c, codes, kbuf[0], c.kb, MKT);
    int32_t selv[MAX_CODES / PTHREADS];
    if (a.sel != nullptr) load_selection<PTHREADS>(a.sel + (size_t(b) * a.S + size_t(s)) * a.k, a.k, selv);
    bf16x8 qa[8];                         // Q^T: lane l holds head 16 hq + l%16, dims 256 nt + 32 ks + 8 (l/16)
    {
        const bf16* qh = a.q + ((size_t(b) * a.S + size_t(s)) * MH + head) * MD + 256 * nt + 8 * g;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) qa[ks] = load_bf16x8(qh + 32 * ks);
    }
    if (a.sel != nullptr)
        c.nrow = compact_selection<PTHREADS>(selv, a.k, nv, c.kbs, a.keys_per_split, codes, wsum);
    const int nk = c.nrow + nwin;
    const size_t pbase = ((size_t(b) * a.S + size_t(s)) * a.n_splits + split) * MH;
    if (c.kb >= nk) {                                 // nothing in this split (no tile issued)
        if (tid < MH) {
            a.part_ml[(pbase + tid) * 2 + 0] = -INFINITY;
            a.part_ml[(pbase + tid) * 2 + 1] = 0.f;
        }
        return;
    }
    const int ke = c.kb + a.keys_per_split < nk ? c.kb + a.keys_per_split : nk;
    const int ntiles = (ke - c.kb + MKT - 1) / MKT;
    auto tile_keys = [&](int t) -> int {
        const int left = ke - (c.kb + t * MKT);
        return left < MKT ? left : MKT;
    };
    if (!tile0_early) prefill_load_tile(c, codes, kbuf[0], c.kb, tile_keys(0));
    floatx4 o[16];                        // lane l: dims 256 nt + 16 m + 4 (l/16) + i of its head
#pragma unroll
    for (int m = 0; m < 16; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) o[m][i] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;
    wait_vm();
    __syncthreads();

    for (int t = 0; t < ntiles; ++t) {
        NextTile nx;
        nx.on = t + 1 < ntiles;
        nx.nkt = nx.on ? tile_keys(t + 1) : 0;
        nx.src = nx.on ? prow_srcs(c, codes, c.kb + (t + 1) * MKT, nx.nkt) : 0;
        nx.buf = kbuf[(t + 1) & 1];
        prefill_tile(a, c, kbuf[t & 1], ptile, xch, qa, o, m_run, l_run, tile_keys(t), nx);
        wait_vm();                        // the next tile has landed
        __syncthreads();                  // ... for every wave; and all are done with this one
    }

    // denominator of this lane's head: its lane group's keys, then both key halves
    l_run = sum_xor32(sum_xor16(l_run));
    if (g == 0) xch[1][nt][head] = l_run;
    __syncthreads();
    const float l_tot = xch[1][0][head] + xch[1][1][head];
    // stage the result in LDS (the key buffers are free now), then coalesced 16-byte stores
    if (a.n_splits == 1) {
        const float z = a.sinks[head] * kLog2e;
        const float mf = fmaxf(m_run, z);
        const float sc = exp2f(m_run - mf);
        const float f = sc / (l_tot * sc + exp2f(z - mf));
        unsigned char* stage = kbuf[0];                 // bf16 [head][dim], 1040-byte rows
#pragma unroll
        for (int m = 0; m < 16; ++m)
            *reinterpret_cast<uint2*>(stage + head * (MD * 2 + 16) + (256 * nt + 16 * m + 4 * g) * 2) =
                pack4_bf16(o[m][0] * f, o[m][1] * f, o[m][2] * f, o[m][3] * f);
        __syncthreads();
        bf16* ob = a.out + (size_t(b) * a.S + size_t(s)) * MH * MD;
        for (int idx = tid; idx < MH * MD / 8; idx += PTHREADS) {
            const int h = idx / (MD / 8), d8 = idx % (MD / 8);
            store16(ob + size_t(h) * MD + d8 * 8,
                    *reinterpret_cast<const uint4*>(stage + h * (MD * 2 + 16) + d8 * 16));
        }
    } else {
        if (nt == 0 && g == 0) {
            a.part_ml[(pbase + head) * 2 + 0] = m_run;
            a.part_ml[(pbase + head) * 2 + 1] = l_tot;
        }
        // fp32 [head][dim]: heads 0..31 staged in kbuf[0], 32..63 in kbuf[1] (32 x 2064 B each)
        unsigned char* st = kbuf[head >> 5] + (head & 31) * OPITCH;
#pragma unroll
        for (int m = 0; m < 16; ++m)
            *reinterpret_cast<float4*>(st + (256 * nt + 16 * m + 4 * g) * 4) =
                make_float4(o[m][0], o[m][1], o[m][2], o[m][3]);
        __syncthreads();
        float* po = a.part_o + pbase * MD;
        for (int idx = tid; idx < MH * MD / 4; idx += PTHREADS) {
            const int h = idx / (MD / 4), d4 = idx % (MD / 4);
            const unsigned char* sp = kbuf[h >> 5] + (h & 31) * OPITCH + d4 * 16;
            store16(po + size_t(h) * MD + d4 * 4, *reinterpret_cast<const uint4*>(sp));
        }
    }
}


// ------------------------------------------------------------------ decode path
// One query per sequence: workgroups per (sequence, 16-head group, key split), so the
// partials a split writes are 16 heads x 512 fp32 and enough workgroups run at once.  A
// split's keys (up to DKC of them; longer splits run in chunks) sit in LDS together, so the
// softmax of a chunk is taken once, after all of its scores are known:
//   * wave w copies and scores the 16-key subtiles u = w, w + 4 (S^T = K Q^T on
//     v_mfma_f32_16x16x32_bf16, lane l owns head l%16), waiting only for its own copies;
//   * the scores meet in LDS (one barrier), every wave takes the same max, exponentials and
//     bf16 P of the whole chunk;
//   * wave w accumulates dims 128 w .. 128 w + 127 of O^T = V^T P^T over every key, so no
//     partial output is merged inside the workgroup.
constexpr int DKC = 128;                  // keys of one decode chunk (8 subtiles of 16)
constexpr int SXP = DKC + 4;              // floats per head row of the exchanged scores
constexpr int QPITCH = MD * 2 + 16;       // LDS row of a staged q (offset rows: no bank conflicts)

template <int N>
__device__ __forceinline__ void wait_vm_n() {
    if constexpr (N == 0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    else if constexpr (N == 16) asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(32)" ::: "memory");
}

// Softmax and P*V of one decode chunk of NKS 32-key steps.  Lane (l%16, g) takes keys
// 32 ks + 8 g + e of head l%16 from the exchanged scores, the layout of the P^T operand, so
// every wave computes the same max, exponentials and bf16 P; wave w then accumulates dims
// 128 w .. 128 w + 127 of O^T = V^T P^T (8 tiles of 16 dims per k-step).
template <int NKS>
__device__ __forceinline__ void decode_chunk_pv(const float* sx, const unsigned char* kbuf, int l16, int g, int w,
                                                int nkt, bool first, float& m_run, float& l_run,
                                                floatx4 (&o)[8]) {
    float sv[NKS][8];
    float cmax = -INFINITY;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
        const float* sr = sx + l16 * SXP + 32 * ks + 8 * g;
        const float4 x0 = *reinterpret_cast<const float4*>(sr);
        const float4 x1 = *reinterpret_cast<const float4*>(sr + 4);
        const float xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            sv[ks][e] = 32 * ks + 8 * g + e < nkt ? xs[e] : -INFINITY;
            cmax = fmaxf(cmax, sv[ks][e]);
        }
    }
    cmax = max_xor32(max_xor16(cmax));
    if (first) {
        m_run = cmax;                         // o and l_run are still zero
    } else if (cmax > m_run + kLazy) {
        const float alpha = fast_exp2(m_run - cmax);
        m_run = cmax;
        l_run *= alpha;
#pragma unroll
        for (int m = 0; m < 8; ++m)
#pragma unroll
            for (int i = 0; i < 4; ++i) o[m][i] *= alpha;
    }
    bf16x8 pb[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
        float pe[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            pe[e] = fast_exp2(sv[ks][e] - m_run);
            l_run += pe[e];
        }
        const uint4 pk = make_uint4(pack2_bf16(pe[0], pe[1]), pack2_bf16(pe[2], pe[3]),
                                    pack2_bf16(pe[4], pe[5]), pack2_bf16(pe[6], pe[7]));
        __builtin_memcpy(&pb[ks], &pk, 16);
    }
    // V^T operands of one k-step go out as a block; the next block is issued before this
    // step's MFMAs, and the scheduling barriers keep the compiler from pairing every read
    // with its MFMA (which would expose the full LDS latency per MFMA)
    const unsigned char* vb0 = kbuf + (8 * g + (l16 >> 2)) * KPITCH + (128 * w + 4 * (l16 & 3)) * 2;
    bf16x8 va[2][8];
    auto load_v = [&](int ks, bf16x8 (&dst)[8]) {
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            const unsigned char* vp = vb0 + 32 * ks * KPITCH + m * 32;
            const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(vp));
            const v4i16 up = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(vp + 4 * KPITCH));
            __builtin_memcpy(&dst[m], &lo, 8);
            __builtin_memcpy(reinterpret_cast<char*>(&dst[m]) + 8, &up, 8);
        }
    };
    load_v(0, va[0]);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
        if (ks + 1 < NKS) load_v(ks + 1, va[(ks + 1) & 1]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int m = 0; m < 8; ++m) o[m] = mfma16x16x32(va[ks & 1][m], pb[ks], o[m]);
        __builtin_amdgcn_sched_barrier(0);
    }
}

// The chunk loop of a split that spans several chunks: two LDS buffers of CK = 64 keys.  At
// the start of chunk ci (every wave being done with chunk ci - 1, whose buffer chunk ci + 1
// takes), the selection of chunk ci + 1 is compacted and its copies issued -- wave w copies
// subtile w -- and then chunk ci is scored while they land: each wave waits only for its own
// copies of chunk ci (those of chunk ci + 1, issued after them, may stay in flight), the
// scores meet in LDS, and every wave takes the softmax and its dims of P*V as in the
// one-chunk path.
template <int CK>
__device__ __forceinline__ void decode_db_chunks(const AttnMfmaArgs& a, TileCtx& c, const int32_t (&selv)[SEL_PER_THREAD],
                                                 int32_t* codes, int* wsum, unsigned char* kbuf,
                                                 unsigned char* qs, float* sx, int b, int hg, int nv, int nwin,
                                                 int kb0, int ke, float& m_run, float& l_run, floatx4 (&o)[8]) {
    const int w = c.w, lane = c.lane, l16 = lane & 15, g = lane >> 4;
    const int nch = (ke - kb0 + CK - 1) / CK;
    auto chunk_keys = [&](int ci) { return ke - (kb0 + ci * CK) < CK ? ke - (kb0 + ci * CK) : CK; };
    // copies of chunk ci into its buffer: lane j < 16 finds the source of row 16 w + j (rows
    // past the chunk's keys copy its last key: finite values whose scores are masked); an odd
    // subtile count leaves the second half of the last P*V step, whose rows are zeroed
    auto issue = [&](int ci) {
        unsigned char* buf = kbuf + (ci & 1) * CK * KPITCH;
        const int cb = kb0 + ci * CK, nkt = chunk_keys(ci);
        const int nsub = (nkt + 15) >> 4, nks = (nkt + 31) >> 5;
        if (w < nsub) {
            uint64_t src = 0;
            const int row = 16 * w + (lane & 15);
            if (lane < 16) src = reinterpret_cast<uint64_t>(key_src(c, codes, cb + (row < nkt ? row : nkt - 1)));
            const uint32_t plo = uint32_t(src), phi = uint32_t(src >> 32);
            unsigned char* dst = buf + 16 * w * KPITCH;
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const uint64_t sp = uint64_t(uint32_t(__builtin_amdgcn_readlane(int(plo), j))) |
                                    (uint64_t(uint32_t(__builtin_amdgcn_readlane(int(phi), j))) << 32);
                dma16(reinterpret_cast<const void*>(sp), uint32_t(lane) * 16, dst + j * KPITCH);
            }
        }
        if (2 * nks > nsub && (nsub & 3) == w) {
#pragma unroll 4
            for (int j = 0; j < 16; ++j) store16(buf + (16 * nsub + j) * KPITCH + lane * 16, make_uint4(0, 0, 0, 0));
        }
    };
    {
        // q rows (4 per wave), then chunk 0 (its selection was compacted with the split's start)
        const bf16* qg = a.q + (size_t(b) * MH + DHG * hg) * MD;
#pragma unroll
        for (int i = 0; i < DHG / 4; ++i)
            dma16(qg + size_t(w + 4 * i) * MD, uint32_t(lane) * 16, qs + (w + 4 * i) * QPITCH);
        issue(0);
    }
    for (int ci = 0; ci < nch; ++ci) {
        if (ci > 0) __syncthreads();          // every wave is done with chunk ci - 1 and the scores
        const bool more = ci + 1 < nch;
        int own_next = 0;
        if (more) {
            const int cb = kb0 + (ci + 1) * CK;
            c.kb = cb;
            c.kbs = cb > nwin ? cb - nwin : 0;
            if (a.sel != nullptr) compact_selection(selv, a.k, nv, c.kbs, CK, codes, wsum);
            issue(ci + 1);
            own_next = ((chunk_keys(ci + 1) + 15) >> 4) > w;
        }
        const int nkt = chunk_keys(ci);
        const int nsub = (nkt + 15) >> 4, nks = (nkt + 31) >> 5;
        const int own = nsub > w;
        if (ci == 0) {
            // this wave's q rows precede its copies of chunks 0 and 1
            const int after = own + own_next;
            if (after == 2) wait_vm_n<32>(); else if (after == 1) wait_vm_n<16>(); else wait_vm_n<0>();
            lds_barrier();                    // every wave's q rows have landed
        }
        const unsigned char* buf = kbuf + (ci & 1) * CK * KPITCH;
        if (own) {
            if (own_next) wait_vm_n<16>(); else wait_vm_n<0>();   // this wave's rows of chunk ci
            bf16x8 qb[MD / 32];               // Q^T: lane l holds head 16 hg + l%16, dims 32 ks + 8 g
#pragma unroll
            for (int ks = 0; ks < MD / 32; ++ks) qb[ks] = load_bf16x8(qs + l16 * QPITCH + ks * 64 + 16 * g);
            floatx4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
            const unsigned char* kr = buf + (16 * w + l16) * KPITCH + 16 * g;
            bf16x8 ka[MD / 32];
#pragma unroll
            for (int ks = 0; ks < MD / 32; ++ks) ka[ks] = load_bf16x8(kr + ks * 64);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int ks = 0; ks < MD / 32; ks += 2) {
                s0 = mfma16x16x32(ka[ks], qb[ks], s0);
                s1 = mfma16x16x32(ka[ks + 1], qb[ks + 1], s1);
            }
            __builtin_amdgcn_sched_barrier(0);
            *reinterpret_cast<float4*>(sx + l16 * SXP + 16 * w + 4 * g) =
                make_float4((s0[0] + s1[0]) * a.scale_log2, (s0[1] + s1[1]) * a.scale_log2,
                            (s0[2] + s1[2]) * a.scale_log2, (s0[3] + s1[3]) * a.scale_log2);
        }
        lds_barrier();                        // chunk ci's rows, zero rows and scores are in LDS
        if (nks == 1)
            decode_chunk_pv<1>(sx, buf, l16, g, w, nkt, ci == 0, m_run, l_run, o);
        else
            decode_chunk_pv<2>(sx, buf, l16, g, w, nkt, ci == 0, m_run, l_run, o);
    }
}

// CK = DKC: a chunk of up to 128 keys at a time, copied, then scored (splits of one chunk);
// CK = 64: two buffers of 64 keys, each chunk's copies issued while the chunk before it is
// scored, for splits that span several chunks (large batches).
template <int CK>
__global__ void __launch_bounds__(256)
attn_decode_kernel(AttnMfmaArgs a, SeqInts pos0v, SeqInts n_rows) {
    static_assert(CK == DKC || CK == DKC / 2, "one 128-key chunk or two 64-key buffers");
    constexpr bool DB = CK < DKC;
    __shared__ __attribute__((aligned(16))) unsigned char kbuf[DKC * KPITCH];
    __shared__ __attribute__((aligned(16))) unsigned char qs[DHG * QPITCH];
    __shared__ __attribute__((aligned(16))) float sx[DHG * SXP];   // scaled scores [head][key]
    __shared__ int32_t codes[DKC];
    __shared__ int wsum[8];

    TileCtx c;
    int hg = blockIdx.y;                  // heads 16 hg .. 16 hg + 15
    int split = blockIdx.x;
    c.b = blockIdx.z;
    {
        // workgroup i runs on XCD i mod 8: the four head groups of a (split, sequence), which
        // read the same key rows, are given ids of one residue so they share an XCD's L2 (in
        // the plain order they share one only when the split count is a multiple of 8: at 7
        // splits each row was fetched four times over the fabric)
        const uint32_t ns = gridDim.x, units = ns * gridDim.z;
        if ((units & 7) == 0) {
            const uint32_t id = blockIdx.x + ns * (blockIdx.y + gridDim.y * blockIdx.z);
            const uint32_t j = id >> 3, unit = (id & 7) + 8 * (j >> 2);
            hg = int(j & 3);
            split = int(unit % ns);
            c.b = int(unit / ns);
        }
    }
    const int tid = threadIdx.x;
    c.lane = tid & 63;
    c.w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: scalar branches
    const int b = c.b, w = c.w, lane = c.lane;
    const int l16 = lane & 15, g = lane >> 4;
    const int p = pos0v.v[b];             // one query: pos0 == p

    int nv = 0;
    if (a.r > 0 && a.rows != nullptr) {
        nv = (p + 1) / a.r;
        if (nv > n_rows.v[b]) nv = n_rows.v[b];
    }
    const int t0 = p - a.W + 1 > 0 ? p - a.W + 1 : 0;
    const int nwin = p - t0 + 1;
    key_ctx(c, a, b, t0, p);
    const int kb0 = split * a.keys_per_split;
    c.kb = kb0;
    c.nwin = nwin;
    c.kbs = kb0 > nwin ? kb0 - nwin : 0;
    c.nrow = nv;
    int32_t selv[SEL_PER_THREAD];
    if (a.sel != nullptr) {
        load_selection(a.sel + size_t(b) * a.k, a.k, selv);
        c.nrow = compact_selection(selv, a.k, nv, c.kbs, a.keys_per_split < CK ? a.keys_per_split : CK,
                                   codes, wsum);
    }
    const int nk = c.nrow + nwin;
    const size_t pbase = (size_t(b) * a.n_splits + split) * MH + DHG * hg;
    // The token's latent goes to its ring slot (workgroup split 0, head group 0) and, at a step
    // that completes no row, its compressor lanes to their frontier slots (split 0, head groups
    // 1 .. n_fr): loaded here, stored when the workgroup's attention is done, so these
    // workgroups wait for no round trip of their own before their key copies.  Slot p % Wr
    // holds token p - Wr, which this query does not read (its window is p-W+1 .. p, with p
    // itself taken from kv_new), and nothing here reads the compressor state, so neither store
    // races a read of this launch.
    uint4 tok = make_uint4(0, 0, 0, 0);
    uint4* tok_dst = nullptr;
    if (split == 0 && hg == 0 && tid < MD / 8) {
        tok = reinterpret_cast<const uint4*>(c.kv_new)[tid];
        tok_dst = reinterpret_cast<uint4*>(const_cast<bf16*>(c.ring) + size_t(uint32_t(p) % c.W) * MD) + tid;
    }
    if (split == 0 && hg >= 1 && hg <= a.n_fr) {
        const AttnMfmaArgs::Front f = hg == 1 ? a.fr[0] : a.fr[1];
        bf16* sa = f.state + size_t(b) * (size_t(2) * f.nw * f.r * f.W) + frontier_slot(p, f.r, f.nw, f.W);
        bf16* sg = sa + size_t(f.nw) * f.r * f.W;
        const bf16* la = f.a + size_t(b) * f.W;
        const bf16* lg = f.g + size_t(b) * f.W;
        if (f.vec) {                                  // 16-byte vectors, one per thread
            const int nv8 = f.W / 8;
            if (tid < 2 * nv8) {
                const bool gate = tid >= nv8;
                const int i = gate ? tid - nv8 : tid;
                tok = reinterpret_cast<const uint4*>(gate ? lg : la)[i];
                tok_dst = reinterpret_cast<uint4*>(gate ? sg : sa) + i;
            }
        } else {
            for (int c = tid; c < f.W; c += 256) {
                sa[c] = la[c];
                sg[c] = lg[c];
            }
        }
    }
    if (kb0 >= nk) {
        if (tok_dst != nullptr) *tok_dst = tok;
        if (tid < DHG) {
            a.part_ml[(pbase + tid) * 2 + 0] = -INFINITY;
            a.part_ml[(pbase + tid) * 2 + 1] = 0.f;
        }
        return;
    }
    const int ke = kb0 + a.keys_per_split < nk ? kb0 + a.keys_per_split : nk;

    floatx4 o[8];                             // lane l: dims 128 w + 16 m + 4 g + i of head l%16
#pragma unroll
    for (int m = 0; m < 8; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) o[m][i] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;     // l_run: this lane's keys 8 g + e of every k-step

    if constexpr (DB) {
        decode_db_chunks<CK>(a, c, selv, codes, wsum, kbuf, qs, sx, b, hg, nv, nwin, kb0, ke, m_run, l_run, o);
    } else {
    for (int cb = kb0; cb < ke; cb += DKC) {
        const bool first = cb == kb0;
        if (!first) {
            __syncthreads();                  // every wave is done with the previous chunk
            c.kb = cb;
            c.kbs = cb > nwin ? cb - nwin : 0;
            if (a.sel != nullptr) compact_selection(selv, a.k, nv, c.kbs, DKC, codes, wsum);
        }
        const int nkt = ke - cb < DKC ? ke - cb : DKC;
        const int nsub = (nkt + 15) >> 4;     // 16-key subtiles to score
        const int nks = (nkt + 31) >> 5;      // 32-key steps of P*V
        const int own = (nsub > w) + (nsub > w + 4);
        if (first) {
            const bf16* qg = a.q + (size_t(b) * MH + DHG * hg) * MD;
#pragma unroll
            for (int i = 0; i < DHG / 4; ++i)
                dma16(qg + size_t(w + 4 * i) * MD, uint32_t(lane) * 16, qs + (w + 4 * i) * QPITCH);
        }
        // rows of subtiles w and w + 4: lane 16 v + j finds the source of row 16 (w + 4 v) + j;
        // rows past the chunk's keys copy its last key (finite values; their scores are masked)
        uint64_t src = 0;
        {
            const int v = lane >> 4, row = 16 * (w + 4 * v) + (lane & 15);
            if (lane < 32 && w + 4 * v < nsub) src = reinterpret_cast<uint64_t>(key_src(c, codes, cb + (row < nkt ? row : nkt - 1)));
        }
        const uint32_t plo = uint32_t(src), phi = uint32_t(src >> 32);
#pragma unroll
        for (int v = 0; v < 2; ++v) {
            if (w + 4 * v >= nsub) break;
            unsigned char* dst = kbuf + 16 * (w + 4 * v) * KPITCH;
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const uint64_t sp = uint64_t(uint32_t(__builtin_amdgcn_readlane(int(plo), 16 * v + j))) |
                                    (uint64_t(uint32_t(__builtin_amdgcn_readlane(int(phi), 16 * v + j))) << 32);
                dma16(reinterpret_cast<const void*>(sp), uint32_t(lane) * 16, dst + j * KPITCH);
            }
        }
        // an odd subtile count leaves the second half of the last P*V step: zero rows
        if (2 * nks > nsub && (nsub & 3) == w) {
#pragma unroll 4
            for (int j = 0; j < 16; ++j) store16(kbuf + (16 * nsub + j) * KPITCH + lane * 16, make_uint4(0, 0, 0, 0));
        }
        if (first) {
            // this wave's q rows precede its 16 * own key copies
            if (own == 2) wait_vm_n<32>(); else if (own == 1) wait_vm_n<16>(); else wait_vm_n<0>();
            lds_barrier();                    // every wave's q rows have landed
        }
        bf16x8 qb[MD / 32];                   // Q^T: lane l holds head 16 hg + l%16, dims 32 ks + 8 g
#pragma unroll
        for (int ks = 0; ks < MD / 32; ++ks) qb[ks] = load_bf16x8(qs + l16 * QPITCH + ks * 64 + 16 * g);
#pragma unroll
        for (int v = 0; v < 2; ++v) {
            const int u = w + 4 * v;
            if (u >= nsub) break;
            if (v == 0 && own == 2) wait_vm_n<16>(); else wait_vm_n<0>();
            floatx4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
            const unsigned char* kr = kbuf + (16 * u + l16) * KPITCH + 16 * g;
            // all K operands of the subtile go out before the first MFMA
            bf16x8 ka[MD / 32];
#pragma unroll
            for (int ks = 0; ks < MD / 32; ++ks) ka[ks] = load_bf16x8(kr + ks * 64);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int ks = 0; ks < MD / 32; ks += 2) {
                s0 = mfma16x16x32(ka[ks], qb[ks], s0);
                s1 = mfma16x16x32(ka[ks + 1], qb[ks + 1], s1);
            }
            __builtin_amdgcn_sched_barrier(0);
            // lane (l%16, g) holds keys 16 u + 4 g + i of head l%16
            *reinterpret_cast<float4*>(sx + l16 * SXP + 16 * u + 4 * g) =
                make_float4((s0[0] + s1[0]) * a.scale_log2, (s0[1] + s1[1]) * a.scale_log2,
                            (s0[2] + s1[2]) * a.scale_log2, (s0[3] + s1[3]) * a.scale_log2);
        }
        wait_vm_n<0>();
        lds_barrier();                        // every key row, zero row and score is in LDS

        switch (nks) {
            case 1: decode_chunk_pv<1>(sx, kbuf, l16, g, w, nkt, first, m_run, l_run, o); break;
            case 2: decode_chunk_pv<2>(sx, kbuf, l16, g, w, nkt, first, m_run, l_run, o); break;
            case 3: decode_chunk_pv<3>(sx, kbuf, l16, g, w, nkt, first, m_run, l_run, o); break;
            default: decode_chunk_pv<4>(sx, kbuf, l16, g, w, nkt, first, m_run, l_run, o); break;
        }
    }
    }

    if (tok_dst != nullptr) *tok_dst = tok;

    // denominator of head 16 hg + l%16: sum over the four lane groups
    const float l_tot = sum_xor32(sum_xor16(l_run));
    const int head = DHG * hg + l16;
    if (a.n_splits == 1) {
        const float z = a.sinks[head] * kLog2e;
        const float mf = fmaxf(m_run, z);
        const float sc = exp2f(m_run - mf);
        const float f = sc / (l_tot * sc + exp2f(z - mf));
        bf16* ob = a.out + (size_t(b) * MH + head) * MD + 128 * w + 4 * g;
#pragma unroll
        for (int m = 0; m < 8; ++m)
            *reinterpret_cast<uint2*>(ob + 16 * m) = pack4_bf16(o[m][0] * f, o[m][1] * f, o[m][2] * f, o[m][3] * f);
    } else {
        if (w == 0 && g == 0) {
            a.part_ml[(pbase + l16) * 2 + 0] = m_run;
            a.part_ml[(pbase + l16) * 2 + 1] = l_tot;
        }
        // bf16 partial output, written through to memory (relaxed system-scope stores carry
        // the coherence bits), so the write-back at the kernel's end finds fewer dirty lines
        // in the L2 (launch 9.07 -> 8.88 us at 64K, batch 8); only the combine launch after
        // this one reads them
        bf16* po = reinterpret_cast<bf16*>(a.part_o) + (pbase + l16) * MD + 128 * w + 4 * g;
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            const uint2 v = pack4_bf16(o[m][0], o[m][1], o[m][2], o[m][3]);
            __hip_atomic_store(reinterpret_cast<unsigned long long*>(po + 16 * m),
                               (static_cast<unsigned long long>(v.y) << 32) | v.x, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_SYSTEM);
        }
    }
}

// 8 consecutive partial-output values as fp32
__device__ __forceinline__ void load8_f32(const float* p, float (&v)[8]) {
    const float4 x = *reinterpret_cast<const float4*>(p), y = *reinterpret_cast<const float4*>(p + 4);
    v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w; v[4] = y.x; v[5] = y.y; v[6] = y.z; v[7] = y.w;
}
__device__ __forceinline__ void load8_f32(const bf16* p, float (&v)[8]) {
    const uint4 u = *reinterpret_cast<const uint4*>(p);
    const uint32_t w4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[2 * i] = __uint_as_float(w4[i] << 16);
        v[2 * i + 1] = __uint_as_float(w4[i] & 0xffff0000u);
    }
}

// Merge the split partials of one query with the sink: weights 2^(m_i - M) / den.  One wave
// per (query, head): lane l holds split l's (max, sum) (at most 32 splits) and latent dims
// 8l .. 8l + 7.  The (max, sum) loads go out just before the first 8 splits' partial-output
// loads, one round trip; M and the denominator are VALU reductions over the lanes (no LDS), each
// lane forms its split's weight, and the weights reach every lane by readlane.  An empty split
// (max -inf, sum 0) wrote no output: its stale values are skipped.
template <typename P>
__global__ void __launch_bounds__(64)
attn_combine_kernel(AttnMfmaArgs a) {
    const int b = blockIdx.z;
    const int64_t s = blockIdx.y;
    const int h = blockIdx.x;
    const int lane = threadIdx.x;
    const int n = a.n_splits;
    const size_t base = (size_t(b) * a.S + size_t(s)) * n;
    const P* po = reinterpret_cast<const P*>(a.part_o) + (base * MH + h) * MD + 8 * lane;
    // (max, sum) first, the weights need it first; every load before any wait (no branch, and
    // the fence keeps the compiler from sinking the partial loads below the reductions)
    float2 t = *reinterpret_cast<const float2*>(a.part_ml + ((base + (lane < n ? lane : n - 1)) * MH + h) * 2);
    const float sink = a.sinks[h];
    float v[8][8];
#pragma unroll
    for (int i = 0; i < 8; ++i) load8_f32(po + size_t(i < n ? i : n - 1) * MH * MD, v[i]);
    asm volatile("" ::: "memory");
    if (lane >= n) t = make_float2(-INFINITY, 0.f);
    const float z = sink * kLog2e;
    const float M = fmaxf(wave_max_valu(t.x), z);
    const float e = t.x == -INFINITY ? 0.f : exp2f(t.x - M);
    const float den = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(wave_sum_valu(t.y * e)))) +
                      exp2f(z - M);
    const float wl = e / den;                          // weight of split `lane`
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int g0 = 0; g0 < n; g0 += 8) {
        if (g0 > 0) {
#pragma unroll
            for (int i = 0; i < 8; ++i) load8_f32(po + size_t(g0 + i < n ? g0 + i : n - 1) * MH * MD, v[i]);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float wv = g0 + i < n ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), g0 + i)) : 0.f;
#pragma unroll
            for (int c = 0; c < 8; ++c) acc[c] += wv != 0.f ? wv * v[i][c] : 0.f;
        }
    }
    bf16* ob = a.out + ((size_t(b) * a.S + size_t(s)) * MH + h) * MD + 8 * lane;
    *reinterpret_cast<uint4*>(ob) = make_uint4(pack2_bf16(acc[0], acc[1]), pack2_bf16(acc[2], acc[3]),
                                               pack2_bf16(acc[4], acc[5]), pack2_bf16(acc[6], acc[7]));
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

// Decode key splits: about kDecodeWgs workgroups over (sequence, head group, split), each
// split a whole number of 16-key subtiles.  Keys that fit one LDS chunk (a window-only layer,
// a short context) take one split: the combine launch would cost more than it spreads.  224
// rather than one per CU: at batch 8 (640 keys) 7 splits of 96 keys finish a little sooner
// than 8 of 80 (8.8 against 8.9 us per launch), fewer partials being written and merged.
constexpr int kDecodeWgs = 224;
int decode_splits(int batch, int64_t nk_max, int* keys_per_split) {
    if (nk_max <= DKC) {
        *keys_per_split = DKC;
        return 1;
    }
    const int64_t units = (nk_max + 15) / 16;
    int64_t want = (kDecodeWgs + 4 * batch - 1) / (4 * batch);
    if (want > MAX_SPLITS) want = MAX_SPLITS;
    if (want > units) want = units;
    if (want < 1) want = 1;
    const int64_t per = (units + want - 1) / want;
    *keys_per_split = int(per * 16);
    return int((units + per - 1) / per);
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
        a.ring = static_cast<const bf16*>(j.ring) + size_t(b0) * j.Wr * MD;
        a.rows = j.rows ? static_cast<const bf16*>(j.rows) + size_t(b0) * j.row_cap * MD : nullptr;
        a.row_cap = j.row_cap;
        a.sel = j.sel ? j.sel + qoff * j.k : nullptr;
        a.k = j.k;
        a.sinks = j.sinks;
        a.out = static_cast<bf16*>(j.out) + qoff * MH * MD;
        a.S = j.S;
        a.W = j.W;
        a.Wr = j.Wr;
        a.r = j.r;
        a.scale_log2 = j.scale * kLog2e;
        const bool decode = j.S == 1;
        if (decode)
            a.n_splits = decode_splits(nb, nrow_max + j.W, &a.keys_per_split);
        else
            a.n_splits = mfma_splits(int64_t(nb) * j.S, nrow_max + j.W, &a.keys_per_split);
        a.n_fr = decode ? j.n_fronts : 0;
        for (int f = 0; f < a.n_fr; ++f) {
            const FrontierJob& fj = j.fronts[f];
            a.fr[f].state = static_cast<bf16*>(fj.state) + size_t(b0) * 2 * fj.nw * fj.r * fj.W;
            a.fr[f].a = static_cast<const bf16*>(fj.lane_a) + size_t(b0) * fj.W;
            a.fr[f].g = static_cast<const bf16*>(fj.lane_g) + size_t(b0) * fj.W;
            a.fr[f].r = fj.r;
            a.fr[f].nw = fj.nw;
            a.fr[f].W = fj.W;
            const uintptr_t al = reinterpret_cast<uintptr_t>(fj.state) | reinterpret_cast<uintptr_t>(fj.lane_a) |
                                 reinterpret_cast<uintptr_t>(fj.lane_g);
            a.fr[f].vec = fj.W % 8 == 0 && fj.W / 4 <= 256 && al % 16 == 0;
        }
        float* ws = static_cast<float*>(j.ws);
        a.part_ml = ws;
        a.part_o = ws + size_t(nb) * j.S * a.n_splits * MH * 2;
        hipError_t e;
        if (decode) {
            // splits longer than one 128-key chunk take the double-buffered 64-key chunks
            if (a.keys_per_split > DKC)
                DSV4_LAUNCH("attn_decode", attn_decode_kernel<DKC / 2>, dim3(unsigned(a.n_splits), MH / DHG, nb),
                            dim3(256), 0, st, a, pos, nr);
            else
                DSV4_LAUNCH("attn_decode", attn_decode_kernel<DKC>, dim3(unsigned(a.n_splits), MH / DHG, nb),
                            dim3(256), 0, st, a, pos, nr);
        } else {
            DSV4_LAUNCH("attn_prefill", attn_prefill_kernel, dim3(unsigned(a.n_splits), unsigned(j.S), nb), dim3(PTHREADS),
                               0, st, a, pos, nr);
        }
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        if (a.n_splits > 1) {
            // decode partial outputs are bf16, prefill ones fp32
            if (decode)
                DSV4_LAUNCH("attn_combine", attn_combine_kernel<bf16>, dim3(MH, unsigned(j.S), nb), dim3(64), 0, st, a);
            else
                DSV4_LAUNCH("attn_combine", attn_combine_kernel<float>, dim3(MH, unsigned(j.S), nb), dim3(64), 0, st, a);
            e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
        if (j.S == 1) continue;          // the attention kernel stored the decode token
        AttnArgs<bf16> ra;
        ra.D = MD; ra.W = j.W; ra.Wr = j.Wr; ra.S = j.S;
        ra.kv_new = a.kv_new;
        ra.ring = static_cast<bf16*>(j.ring) + size_t(b0) * j.Wr * MD;
        const int64_t nupd = std::min<int64_t>(j.S, j.Wr);
        DSV4_LAUNCH("ring_update", ring_update_kernel<bf16>, dim3(unsigned(nupd), nb), dim3(256), 0, st, ra, pos);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace

int64_t attn_max_keys(bool bf16_, int H, int D, int k, bool has_sel) {
    // the MFMA kernels index keys in 32 bits
    if (use_mfma(bf16_, H, D)) return has_sel && k > MAX_CODES ? 0 : int64_t(1) << 30;
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
    if (use_mfma(j.bf16, j.H, j.D) && j.S == 1) return run_mfma(j, s);   // stores folded in
    for (int f = 0; f < j.n_fronts; ++f) {
        const hipError_t e = launch_frontier_store(j.fronts[f], j.bf16, j.batch, j.pos0, s);
        if (e != hipSuccess) return e;
    }
    if (use_mfma(j.bf16, j.H, j.D)) return run_mfma(j, s);
    return j.bf16 ? run<bf16>(j, s) : run<float>(j, s);
}

}  // namespace dsv4
