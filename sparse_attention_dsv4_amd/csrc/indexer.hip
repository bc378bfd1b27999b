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
//
// mfma scoring (bf16, 64 heads x 128 dims): heads are the M dimension of
// v_mfma_f32_32x32x16_bf16 and rows the N dimension, so a lane ends with 16 heads of one
// row; ReLU, the folded head weights and the sum over heads happen in registers (one
// cross-half add), and only the fp32 score key leaves the kernel.  Each wave keeps one
// query's 64x128 block as A fragments; 128-row tiles of the lane are staged in LDS and
// shared by the workgroup's queries (prefill: 8 queries, two per wave; decode: one query,
// the 4 waves split the tile).  The per-(query, row) arithmetic is the same in both, so a
// decode step and a prefill chunk give bit-identical scores.  Tiles are double-buffered in
// LDS through direct global-to-LDS loads.
#include "common.hpp"
#include "kernels.hpp"
#include "mfma.hpp"

namespace dsv4 {

namespace {

constexpr int kScoreRows = 64;      // rows per workgroup of the scoring kernel
constexpr int kScoreThreads = 256;

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


// max(x, 0) for finite x as an integer max of the bit pattern (negative floats, -0 included,
// have the sign bit set and compare below 0): one instruction, no IEEE canonicalisation.
__device__ __forceinline__ float relu_bits(float x) {
    const int v = __float_as_int(x);
    return __int_as_float(v > 0 ? v : 0);
}

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


// ------------------------------------------------------------------ mfma scoring
// Prefill scoring: one query per wave (226 VGPRs, two waves per SIMD), eight waves per
// workgroup; tiles of the lane staged through a ring of four LDS buffers.  (Two queries per
// wave, with more operand reuse but one wave per SIMD, measured slower.)
constexpr int kIdxWaves = 8;
constexpr int kIdxStages = 4;
constexpr int IH = 64;                 // indexer heads
constexpr int ID = 128;                // indexer dims
constexpr int IRT = 128;               // rows per LDS tile
constexpr int IROWB = ID * 2;          // bytes per row (unpadded: chunks are XOR-swizzled)

typedef __attribute__((address_space(3))) unsigned char lds_u8;

struct IdxMfmaArgs {
    const bf16* qi;
    const float* w;
    const bf16* rows;
    int64_t row_cap;
    int64_t S;
    int64_t n_stride;
    uint32_t* keys;
    int r;
    float scale;
    int rows_per_block;
    int queries_per_group;     // row-stationary kernel: queries one workgroup scores
    // fused decode scoring: each workgroup's m best rows, in row order, and the largest key
    // of the rest ([queries][n_groups][m] keys and rows, [queries][n_groups] cutoffs)
    uint32_t* cand_key;
    int32_t* cand_row;
    uint32_t* cutoff;
    int n_groups, m;
};

// Direct global -> LDS copy (16 bytes per lane to lds_base + 16 lane), as inline asm so the
// compiler does not serialise LDS reads of the other tile buffer behind it.
__device__ __forceinline__ void idx_dma16(const void* gptr, const unsigned char* lds_base) {
    const uint32_t la = __builtin_amdgcn_readfirstlane(uint32_t(size_t((const lds_u8*)lds_base)));
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
                 :: "s"(la), "v"(gptr) : "memory", "m0");
}

// Wait until at most N vector-memory operations of this wave are pending.
template <int N>
__device__ __forceinline__ void wait_vm_loads() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
// Workgroup barrier for LDS data only (copies to other buffers stay in flight).
__device__ __forceinline__ void idx_lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Row r's 16-byte chunk c sits at chunk position c ^ (r & 15) of its 256-byte LDS row, so
// the 32 rows an MFMA operand read touches spread over all banks.
__device__ __forceinline__ int swz(int row, int chunk) { return chunk ^ (row & 15); }

// Stage rows [j0, j0 + IRT) of the lane (zeros past j_end): each wave instruction moves 4
// rows; lane l fetches chunk swz(row, l%16) of row l/16 so that it lands at position l%16.
template <int WAVES>
__device__ __forceinline__ void idx_load_tile(const IdxMfmaArgs& a, int b, int64_t j0,
                                              int64_t j_end, unsigned char* buf) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
    for (int i = 0; i < IRT / 4 / WAVES; ++i) {          // 4 rows per wave instruction
        const int row0 = 4 * (w + WAVES * i);
        const int row = row0 + (lane >> 4);
        const int64_t jj = j0 + row;
        unsigned char* dst = buf + row0 * IROWB;
        if (j0 + row0 + 3 < j_end) {
            idx_dma16(a.rows + (size_t(b) * a.row_cap + size_t(jj)) * ID + swz(row, lane & 15) * 8, dst);
        } else {
            // the rows past j_end are zero; the load is still issued (from the last row), so
            // every wave issues exactly IRT / 4 / WAVES loads per tile and the pipeline's
            // counted waits stay exact
            const int64_t js = jj < j_end ? jj : j_end - 1;
            uint4 v = *reinterpret_cast<const uint4*>(a.rows + (size_t(b) * a.row_cap + size_t(js)) * ID +
                                                      swz(row, lane & 15) * 8);
            if (jj >= j_end) v = make_uint4(0, 0, 0, 0);
            store16(dst + lane * 16, v);
        }
    }
}

// Prefill scoring over a block of rows: wave w scores query 8 * blockIdx.y + w against
// every 128-row tile of the block, the tiles staged in LDS and shared by the 8 queries.
template <int WAVES, int NSTAGE>
__global__ void __launch_bounds__(64 * WAVES)
index_score_mfma_kernel(IdxMfmaArgs a, SeqInts pos0v, SeqInts n_rows) {
    __shared__ __attribute__((aligned(16))) unsigned char kt[NSTAGE][IRT * IROWB];
    const int b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int l32 = lane & 31, hi = lane >> 5;
    const int64_t pos0 = pos0v.v[b];
    const int64_t qs = int64_t(blockIdx.y) * WAVES + w;
    int64_t s_last = int64_t(blockIdx.y) * WAVES + WAVES - 1;
    if (s_last > a.S - 1) s_last = a.S - 1;
    int64_t nv_max = (pos0 + s_last + 1) / a.r;
    if (nv_max > n_rows.v[b]) nv_max = n_rows.v[b];
    const int64_t j_begin = int64_t(blockIdx.x) * a.rows_per_block;
    if (j_begin >= nv_max) return;
    const int64_t j_end = j_begin + a.rows_per_block < nv_max ? j_begin + a.rows_per_block : nv_max;

    bf16x8 qa[2][ID / 16];
    float wsc[2][16];
    const bool qvalid = qs < a.S;
    int64_t nv = 0;
    if (qvalid) {
        nv = (pos0 + qs + 1) / a.r;
        if (nv > n_rows.v[b]) nv = n_rows.v[b];
    }
    {
        const int64_t sq = qvalid ? qs : 0;
        const bf16* qrow = a.qi + ((size_t(b) * a.S + size_t(sq)) * IH + l32) * ID + 8 * hi;
        const float* wr = a.w + (size_t(b) * a.S + size_t(sq)) * IH;
#pragma unroll
        for (int m = 0; m < 2; ++m) {
#pragma unroll
            for (int ks = 0; ks < ID / 16; ++ks) qa[m][ks] = load_bf16x8(qrow + m * 32 * ID + ks * 16);
#pragma unroll
            for (int i = 0; i < 16; ++i) wsc[m][i] = qvalid ? wr[32 * m + c_row(i, lane)] * a.scale : 0.f;
        }
    }

    // NSTAGE-buffer ring: tile t + NSTAGE - 1 is requested when tile t starts, so each copy
    // has NSTAGE - 1 tiles of compute to land.  Every wave issues exactly OPS loads per tile;
    // tile t has landed once at most the loads of the tiles after it are pending (stores in
    // between can only make the counted wait stricter).
    constexpr int OPS = IRT / 4 / WAVES;
    const int ntiles = int((j_end - j_begin + IRT - 1) / IRT);
#pragma unroll
    for (int t = 0; t < NSTAGE - 1; ++t)
        if (t < ntiles) idx_load_tile<WAVES>(a, b, j_begin + int64_t(t) * IRT, j_end, kt[t]);
    for (int t = 0; t < ntiles; ++t) {
        const int64_t j0 = j_begin + int64_t(t) * IRT;
        const int later = ntiles - 1 - t < NSTAGE - 2 ? ntiles - 1 - t : NSTAGE - 2;
        if (later >= 2) wait_vm_loads<2 * OPS>();
        else if (later == 1) wait_vm_loads<OPS>();
        else wait_vm_loads<0>();
        idx_lds_barrier();                             // tile t visible; tile t-1 fully read
        if (t + NSTAGE - 1 < ntiles)
            idx_load_tile<WAVES>(a, b, j0 + int64_t(NSTAGE - 1) * IRT, j_end, kt[(t + NSTAGE - 1) % NSTAGE]);
        const unsigned char* buf = kt[t % NSTAGE];
        // the tile's four 32-row blocks; the MFMAs of block u+1 are issued before the epilogue
        // of block u, so the matrix pipe stays busy while the VALU reduces the previous block
        floatx16 c[2][2];
        float score[4];
#pragma unroll
        for (int u = 0; u <= 4; ++u) {
            if (u < 4) {
                const int row = 32 * u + l32;
                const unsigned char* kr = buf + row * IROWB;
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    c[u & 1][0][i] = 0.f;
                    c[u & 1][1][i] = 0.f;
                }
#pragma unroll
                for (int ks = 0; ks < ID / 16; ++ks) {
                    const bf16x8 kb = load_bf16x8(kr + swz(row, 2 * ks + hi) * 16);
                    c[u & 1][0] = mfma32x32x16(qa[0][ks], kb, c[u & 1][0]);
                    c[u & 1][1] = mfma32x32x16(qa[1][ks], kb, c[u & 1][1]);
                }
            }
            if (u > 0) {
                // weighted relu sum over the 64 heads of block u-1 (relu as an integer max of
                // the bit pattern: exact, one instruction), kept until the tile's stores
                const int v = u - 1;
                float s0 = 0.f, s1 = 0.f;
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    s0 = fmaf(wsc[0][i], relu_bits(c[v & 1][0][i]), s0);
                    s1 = fmaf(wsc[1][i], relu_bits(c[v & 1][1][i]), s1);
                }
                const float sc = s0 + s1;
                score[v] = sum_xor32(sc);
            }
        }
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int64_t jj = j0 + 32 * v + l32;
            if (hi == 0 && jj < nv)
                a.keys[(size_t(b) * a.S + size_t(qs)) * a.n_stride + size_t(jj)] = score_key(score[v]);
        }
    }
}

// Row-stationary scoring for prefill at long context: a workgroup copies a block of RSB rows
// into LDS once (no copies run while the operands are read) and streams queries through
// registers: wave w scores queries q_lo + w, q_lo + w + WAVES, ... of the workgroup's
// group against every 32-row block of the tile a query can see.  Each query's A operand
// (64 heads x 128 dims) and head weights come from global memory (L2); the two waves of a
// SIMD hide each other's loads.
constexpr int RSB = 512;                      // rows held by one workgroup (128 KB of LDS)
constexpr int64_t kIdxRsMinRows = 4096;       // below, too few row blocks to fill the chip

struct IdxQ {
    bf16x8 qa[2][ID / 16];
    float wsc[2][16];
};

__device__ __forceinline__ void idx_load_query(const IdxMfmaArgs& a, int b, int64_t s, IdxQ& q) {
    const int lane = threadIdx.x & 63, l32 = lane & 31, hi = lane >> 5;
    const bf16* qrow = a.qi + ((size_t(b) * a.S + size_t(s)) * IH + l32) * ID + 8 * hi;
    const float* wr = a.w + (size_t(b) * a.S + size_t(s)) * IH;
#pragma unroll
    for (int m = 0; m < 2; ++m) {
#pragma unroll
        for (int ks = 0; ks < ID / 16; ++ks) q.qa[m][ks] = load_bf16x8(qrow + m * 32 * ID + ks * 16);
#pragma unroll
        for (int g = 0; g < 4; ++g) {           // heads 32 m + 8 g + 4 hi + 0..3
            const float4 v = *reinterpret_cast<const float4*>(wr + 32 * m + 8 * g + 4 * hi);
            q.wsc[m][4 * g + 0] = v.x * a.scale;
            q.wsc[m][4 * g + 1] = v.y * a.scale;
            q.wsc[m][4 * g + 2] = v.z * a.scale;
            q.wsc[m][4 * g + 3] = v.w * a.scale;
        }
    }
}

template <int WAVES>
__global__ void __launch_bounds__(64 * WAVES)
index_score_rs_kernel(IdxMfmaArgs a, SeqInts pos0v, SeqInts n_rows) {
    __shared__ __attribute__((aligned(16))) unsigned char kt[RSB * IROWB];
    const int b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int l32 = lane & 31, hi = lane >> 5;
    const int64_t pos0 = pos0v.v[b];
    const int64_t q_lo = int64_t(blockIdx.y) * a.queries_per_group;
    int64_t q_hi = q_lo + a.queries_per_group < a.S ? q_lo + a.queries_per_group : a.S;
    int64_t nv_max = (pos0 + q_hi) / a.r;                  // rows the group's last query sees
    if (nv_max > n_rows.v[b]) nv_max = n_rows.v[b];
    const int64_t j_begin = int64_t(blockIdx.x) * RSB;
    if (j_begin >= nv_max) return;
    const int64_t j_end = j_begin + RSB < nv_max ? j_begin + RSB : nv_max;
#pragma unroll
    for (int t = 0; t < RSB / IRT; ++t) idx_load_tile<WAVES>(a, b, j_begin + t * IRT, j_end, kt + t * IRT * IROWB);
    wait_vm_loads<0>();
    __syncthreads();

    for (int64_t s = q_lo + w; s < q_hi; s += WAVES) {
        IdxQ cur;
        idx_load_query(a, b, s, cur);
        int64_t nvq = (pos0 + s + 1) / a.r;
        if (nvq > n_rows.v[b]) nvq = n_rows.v[b];
        const int nblk = nvq > j_begin ? int((nvq - j_begin + 31) / 32) : 0;   // blocks it sees
        uint32_t* keys = a.keys + (size_t(b) * a.S + size_t(s)) * a.n_stride;
        floatx16 c[2][2];
#pragma unroll
        for (int u = 0; u <= RSB / 32; ++u) {
            if (u < RSB / 32 && u < nblk) {
                const int row = 32 * (u & (IRT / 32 - 1)) + l32;              // row of its tile
                const unsigned char* kr = kt + (u / (IRT / 32)) * IRT * IROWB + row * IROWB;
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    c[u & 1][0][i] = 0.f;
                    c[u & 1][1][i] = 0.f;
                }
#pragma unroll
                for (int ks = 0; ks < ID / 16; ++ks) {
                    const bf16x8 kb = load_bf16x8(kr + swz(row, 2 * ks + hi) * 16);
                    c[u & 1][0] = mfma32x32x16(cur.qa[0][ks], kb, c[u & 1][0]);
                    c[u & 1][1] = mfma32x32x16(cur.qa[1][ks], kb, c[u & 1][1]);
                }
            }
            if (u > 0 && u - 1 < nblk) {
                const int v = u - 1;
                float s0 = 0.f, s1 = 0.f;
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    s0 = fmaf(cur.wsc[0][i], relu_bits(c[v & 1][0][i]), s0);
                    s1 = fmaf(cur.wsc[1][i], relu_bits(c[v & 1][1][i]), s1);
                }
                float sc = s0 + s1;
                sc = sum_xor32(sc);
                const int64_t jj = j_begin + 32 * v + l32;
                if (hi == 0 && jj < nvq) keys[jj] = score_key(sc);
            }
        }
    }
}

bool use_index_mfma(bool bf16_, int Hi, int di) { return bf16_ && Hi == IH && di == ID; }

// ------------------------------------------------------------------ exact top-k select
// The k-th largest key T of a set by radix select, then compaction in row order: every key
// > T, plus the lowest-placed keys == T until k are taken.  Row-order compaction makes the
// output ascending without a sort; the lowest-placed ties are the lowest rows.

// Inclusive prefix sum over the lanes of a wave in DPP steps: shifts by 1, 2, 4 and 8 lanes
// within each row of 16 lanes, then the last lane of row 0 (2) added to row 1 (3), and the
// last lane of row 1 to rows 2 and 3.  Lanes a step does not reach add 0.
__device__ __forceinline__ int wave_incl_scan(int x) {
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);   // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);   // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);   // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);   // row_shr:8
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);   // row_bcast:15
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);   // row_bcast:31
    return x;
}

// Largest (MAX) or smallest u32 over the lanes of a wave: within each row of 16 lanes by
// DPP, then the four rows' values read back by the scalar unit.
template <bool MAX>
__device__ __forceinline__ uint32_t wave_extreme_u32(uint32_t v) {
    auto pick = [](uint32_t x, uint32_t y) { return MAX ? (x > y ? x : y) : (x < y ? x : y); };
    v = pick(v, uint32_t(__builtin_amdgcn_mov_dpp(int(v), 0xb1, 0xf, 0xf, false)));    // quad_perm [1,0,3,2]
    v = pick(v, uint32_t(__builtin_amdgcn_mov_dpp(int(v), 0x4e, 0xf, 0xf, false)));    // quad_perm [2,3,0,1]
    v = pick(v, uint32_t(__builtin_amdgcn_mov_dpp(int(v), 0x124, 0xf, 0xf, false)));   // row_ror:4
    v = pick(v, uint32_t(__builtin_amdgcn_mov_dpp(int(v), 0x128, 0xf, 0xf, false)));   // row_ror:8
    const uint32_t r0 = uint32_t(__builtin_amdgcn_readlane(int(v), 0));
    const uint32_t r1 = uint32_t(__builtin_amdgcn_readlane(int(v), 16));
    const uint32_t r2 = uint32_t(__builtin_amdgcn_readlane(int(v), 32));
    const uint32_t r3 = uint32_t(__builtin_amdgcn_readlane(int(v), 48));
    return pick(pick(r0, r1), pick(r2, r3));
}

// Given a histogram of `bins` bins and the count `rem` still needed from the keys it covers,
// find the bin holding the rem-th largest key.  Writes the bin, the count still needed inside
// it and the bin's count to sh[0..2].  NT threads, bins a multiple of NT; `tmp` holds NT / 64
// ints.  Thread t sums bins [t per, (t + 1) per); the counts above it are the later waves'
// totals plus the lanes above it in its own wave (a DPP scan): two barriers.
template <int NT>
__device__ __forceinline__ void find_bucket(const uint32_t* hist, int bins, int rem, int* tmp, int* sh) {
    const int per = bins / NT;                        // 1 to 4 bins per thread
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    int part = 0;
    for (int i = 0; i < per; ++i) part += int(hist[t * per + i]);
    const int x = wave_incl_scan(part);
    if (lane == 63) tmp[w] = x;
    __syncthreads();
    int above = __builtin_amdgcn_readlane(x, 63) - x;  // this wave's bins above this thread's
#pragma unroll
    for (int v = 0; v < NT / 64; ++v) above += v > w ? tmp[v] : 0;
    for (int i = per - 1; i >= 0; --i) {
        const int h = int(hist[t * per + i]);
        if (above < rem && above + h >= rem) {
            sh[0] = t * per + i;
            sh[1] = rem - above;
            sh[2] = h;
        }
        above += h;
    }
    __syncthreads();
}

// Number of set bits of a wave mask in the lanes below this one.
__device__ __forceinline__ int lanes_below(uint64_t m) {
    return int(__builtin_amdgcn_mbcnt_hi(uint32_t(m >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(m), 0u)));
}

// Keys held in registers by a workgroup of NT threads, KPT per thread: wave w owns the
// contiguous positions [w C, (w+1) C), C = 64 KPT; within it lane l holds groups of 4
// consecutive positions at w C + 256 i + 4 l (one 16-byte load each, a wave instruction
// reading 1 KB contiguous).  Positions past the set hold key 0, below the key of every score
// (score_key gives 0 only to the NaN with every bit set).  `ngv`: the wave's groups of
// 4 x 64 positions holding any position of the set (the others are skipped and count as
// keys 0, which changes no bin at or above the k-th key when at least k keys are above 0).
struct RegSelect {
    uint32_t thr;              // the k-th largest key
    int rem;                   // keys == thr to take, lowest positions first
};

// Words of LDS the threshold search uses: the three passes' histograms (2048, 2048 and
// 1024 bins), all cleared at the start, and a spare word per lane.
constexpr int kHistBins = 2048 + 2048 + 1024;
constexpr int kHistWords = kHistBins + 64;

// The k-th largest key by radix select over digits fitted to the keys that can matter.
// When k <= NT, the smallest of the threads' largest keys, q, is at or below the k-th
// largest key (the NT threads' largest keys are NT keys >= q), so keys below q are left out
// and the digits are those of key - q over the range [q, max]: pass 1 bins the keys >= q by
// (key - q) >> s1 (s1 fitting max - q to 11 bits), pass 2 bins the keys of the chosen bin by
// the next 11 bits, pass 3 by the rest (at most 10).  Near the threshold the bins are narrow,
// so one pass often suffices.  `tmp` holds 2 NT / 64 ints, `hist` kHistWords (16-byte
// aligned).
// EXACT = false: the returned threshold may instead be one below the lowest key of a bucket
// whose keys are all taken (rem = 0), once a pass finds its bucket's count equal to what is
// still needed -- the same set of keys in fewer passes -- for callers that only compact
// with it.
template <int KPT, int NT, bool EXACT = true>
__device__ RegSelect reg_select_threshold(const uint32_t (&key)[KPT], int ngv, int k,
                                          uint32_t* hist, int* tmp, int* sh) {
    constexpr int G = KPT / 4, NW = NT / 64;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    for (int i = tid; i < kHistBins / 4; i += NT)
        reinterpret_cast<uint4*>(hist)[i] = make_uint4(0u, 0u, 0u, 0u);
    uint32_t m = 0;
#pragma unroll
    for (int e = 0; e < KPT; ++e) m = key[e] > m ? key[e] : m;
    const uint32_t wmax = wave_extreme_u32<true>(m), wmin = wave_extreme_u32<false>(m);
    if (lane == 0) {
        tmp[w] = int(wmax);
        tmp[NW + w] = int(wmin);
    }
    __syncthreads();
    uint32_t kmax = 0, q = 0xffffffffu;
#pragma unroll
    for (int v = 0; v < NW; ++v) {
        const uint32_t x = uint32_t(tmp[v]), y = uint32_t(tmp[NW + v]);
        kmax = x > kmax ? x : kmax;
        q = y < q ? y : q;
    }
    if (k > NT) q = 0;
    q = uint32_t(__builtin_amdgcn_readfirstlane(int(q)));
    kmax = uint32_t(__builtin_amdgcn_readfirstlane(int(kmax)));
    const uint32_t range = kmax - q;
    const int bits = range ? 32 - __builtin_clz(range) : 0;
    const int s1 = bits > 11 ? bits - 11 : 0, s2 = s1 > 11 ? s1 - 11 : 0;
    uint32_t* h1 = hist;
    uint32_t* h2 = hist + 2048;
    uint32_t* h3 = hist + 4096;
    // pass 1: (key - q) >> s1 of every key >= q; a key below q counts into its lane's spare
    // word instead (no branch, and no two lanes of an instruction on one word)
    const uint32_t spare = uint32_t(kHistBins + lane);
#pragma unroll
    for (int i = 0; i < G; ++i)
        if (i < ngv) {
#pragma unroll
            for (int e = 4 * i; e < 4 * i + 4; ++e)
                atomicAdd(&hist[key[e] >= q ? (key[e] - q) >> s1 : spare], 1u);
        }
    __syncthreads();
    find_bucket<NT>(h1, 2048, k, tmp, sh);
    const uint32_t b1 = uint32_t(sh[0]);
    int rem = sh[1];
    const uint32_t lo1 = q + (b1 << s1);               // lowest key of bin b1
    if (!EXACT && sh[2] == rem && lo1 > 0) return RegSelect{lo1 - 1u, 0};
    if (s1 == 0) return RegSelect{lo1, rem};          // a bin per key value
    // pass 2: ((key - q) >> s2) mod 2048 of the keys in bin b1 (2^(s1 - s2) <= 2048 values,
    // aligned, so the order holds)
#pragma unroll
    for (int i = 0; i < G; ++i)
        if (i < ngv) {
            bool in[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) in[j] = key[4 * i + j] >= q && ((key[4 * i + j] - q) >> s1) == b1;
            if (__builtin_amdgcn_ballot_w64(in[0] || in[1] || in[2] || in[3]) == 0) continue;   // usual
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (in[j]) atomicAdd(&h2[((key[4 * i + j] - q) >> s2) & 2047u], 1u);
        }
    __syncthreads();
    find_bucket<NT>(h2, 2048, rem, tmp, sh);
    const uint32_t p2 = ((b1 << (s1 - s2)) & ~2047u) | uint32_t(sh[0]);   // (key - q) >> s2
    rem = sh[1];
    const uint32_t lo2 = q + (p2 << s2);
    if (!EXACT && sh[2] == rem && lo2 > 0) return RegSelect{lo2 - 1u, 0};
    if (s2 == 0) return RegSelect{lo2, rem};
    // pass 3: the low s2 (<= 10) bits of key - q for the keys with (key - q) >> s2 == p2
#pragma unroll
    for (int i = 0; i < G; ++i)
        if (i < ngv) {
            bool in[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) in[j] = key[4 * i + j] >= q && ((key[4 * i + j] - q) >> s2) == p2;
            if (__builtin_amdgcn_ballot_w64(in[0] || in[1] || in[2] || in[3]) == 0) continue;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (in[j]) atomicAdd(&h3[(key[4 * i + j] - q) & ((1u << s2) - 1u)], 1u);
        }
    __syncthreads();
    find_bucket<NT>(h3, 1024, rem, tmp, sh);
    const uint32_t t = lo2 + uint32_t(sh[0]);
    if (!EXACT && sh[2] == sh[1] && t > 0) return RegSelect{t - 1u, 0};   // every tie taken
    return RegSelect{t, sh[1]};
}

// Compaction in position order of the keys taken by `sel`.  Lane masks (the compare results
// themselves) give every count: wave totals first, then each wave walks its groups of 4 x 64
// positions, where position 4 l + j of a group is key j of lane l, so the positions before it
// are those of lower lanes and its own lower j.  emit(slot, e, position) for every taken key
// (e indexes key[]).  Returns, in every lane, the largest key NOT taken (0 if none; only
// meaningful in the lanes of one wave before a block reduction).
template <int KPT, int NT, class Emit>
__device__ uint32_t reg_compact(const uint32_t (&key)[KPT], RegSelect sel, int (*wtot)[NT / 64],
                                Emit emit) {
    constexpr int G = KPT / 4;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    // lane index from mbcnt: positions computed afresh (see reg_compact_gt)
    const int wbase = w * 64 * KPT + 4 * int(__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)));
    const uint32_t thr = sel.thr;
    const int rem = sel.rem;
    int ngt = 0, neq = 0;
#pragma unroll
    for (int e = 0; e < KPT; ++e) {
        ngt += int(__popcll(__builtin_amdgcn_ballot_w64(key[e] > thr)));
        neq += int(__popcll(__builtin_amdgcn_ballot_w64(key[e] == thr)));
    }
    if (lane == 0) {
        wtot[0][w] = ngt;
        wtot[1][w] = neq;
    }
    __syncthreads();
    int o = 0, eqb = 0;                                // keys taken / ties seen before this wave
    for (int v = 0; v < w; ++v) {
        eqb += wtot[1][v];
        o += wtot[0][v];
    }
    o += eqb < rem ? eqb : rem;
    uint32_t rest = 0;                                 // largest key not taken
#pragma unroll
    for (int i = 0; i < G; ++i) {
        uint64_t em[4], any = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            em[j] = __builtin_amdgcn_ballot_w64(key[4 * i + j] == thr);
            any |= em[j] | __builtin_amdgcn_ballot_w64(key[4 * i + j] > thr);
        }
        if (any == 0) {                                // nothing taken in this group
#pragma unroll
            for (int j = 0; j < 4; ++j) rest = key[4 * i + j] > rest ? key[4 * i + j] : rest;
            continue;
        }
        int eq_rank = eqb;                             // ties before this lane's first key
#pragma unroll
        for (int j = 0; j < 4; ++j) eq_rank += lanes_below(em[j]);
        bool take[4];
        int slot = o;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const bool eq = key[4 * i + j] == thr;
            take[j] = key[4 * i + j] > thr || (eq && eq_rank < rem);
            eq_rank += eq;
            const uint64_t tm = __builtin_amdgcn_ballot_w64(take[j]);
            slot += lanes_below(tm);
            o += int(__popcll(tm));
            eqb += int(__popcll(em[j]));
            if (!take[j]) rest = key[4 * i + j] > rest ? key[4 * i + j] : rest;
        }
        const int j0 = wbase + 256 * i;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (take[j]) emit(slot++, 4 * i + j, j0 + j);
    }
    return rest;
}

// Compaction in position order when the keys taken are exactly those above `thr` (no tie
// split at the threshold, rem == 0): one compare per key, its ballot giving both the wave's
// count and, through a chain of mbcnt over a group's four masks, a lane's first slot.
// emit(slot, e, position) for every taken key.  WAVE_SLOTS: the slots are the wave's own,
// 0 .. taken by the wave - 1 (no count pass, no barrier; the caller places the waves' runs);
// else 0 .. taken - 1 over the workgroup, after a count pass (`wtot`: NT / 64 ints).
// Returns the wave's count of keys taken.
template <int KPT, int NT, bool WAVE_SLOTS = false, class Emit>
__device__ int reg_compact_gt(const uint32_t (&key)[KPT], uint32_t thr, int* wtot, Emit emit) {
    constexpr int G = KPT / 4;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    int o = 0;                                         // keys taken by the waves before
    if (!WAVE_SLOTS) {
        int cnt = 0;
#pragma unroll
        for (int e = 0; e < KPT; ++e) cnt += int(__popcll(__builtin_amdgcn_ballot_w64(key[e] > thr)));
        if (lane == 0) wtot[w] = cnt;
        __syncthreads();
#pragma unroll
        for (int v = 0; v < NT / 64; ++v) o += v < w ? wtot[v] : 0;
        o = __builtin_amdgcn_readfirstlane(o);
    }
    const int o0 = o;
    // the lane index from mbcnt rather than threadIdx: positions computed afresh here, not
    // kept in registers from the callers' loads, which compute the same expressions (32 more
    // registers live through the whole select)
    const int wbase = w * 64 * KPT + 4 * int(__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)));
#pragma unroll
    for (int i = 0; i < G; ++i) {
        uint64_t m[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) m[j] = __builtin_amdgcn_ballot_w64(key[4 * i + j] > thr);
        if ((m[0] | m[1] | m[2] | m[3]) == 0) continue;
        uint32_t slot = uint32_t(o);                   // + taken keys of the lower lanes
#pragma unroll
        for (int j = 0; j < 4; ++j)
            slot = __builtin_amdgcn_mbcnt_hi(uint32_t(m[j] >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(m[j]), slot));
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (key[4 * i + j] > thr) emit(int(slot++), 4 * i + j, wbase + 256 * i + j);
            o += int(__popcll(m[j]));
        }
    }
    return o - o0;
}

// Workgroup-wide max of a u32 over NT threads (`red` holds NT / 64 entries).
template <int NT>
__device__ __forceinline__ uint32_t block_max_u32(uint32_t v, uint32_t* red) {
    v = wave_extreme_u32<true>(v);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < NT / 64; ++i) m = red[i] > m ? red[i] : m;
    return m;
}

// The decode scorer's waves per workgroup and the fused indexer's row groups (below).
constexpr int kStreamWaves = 8;
constexpr int kFuseMaxRows = 4096;                    // rows of one workgroup's local select
constexpr int kFuseKpt = kFuseMaxRows / (64 * kStreamWaves);

// Row groups of the fused scorer for a query of nbt 32-row blocks at bpw blocks per wave:
// whole groups of WAVES bpw blocks, and a remainder of at most one block per wave goes to the
// last group (its first waves take one block more: one longer wave instead of every wave's
// count rounded up, which left a fifth of the chip idle at 65,538 rows); a larger remainder
// makes a group of its own.  *extra: the blocks the last group takes beyond WAVES bpw.
// (Only while the longer group still fits the local select's kFuseMaxRows.)
__host__ __device__ inline int64_t fused_groups(int64_t nbt, int bpw, int waves, int* extra) {
    const int64_t per = int64_t(waves) * bpw;
    const int64_t g = nbt / per, r = nbt - g * per;
    if (g > 0 && r <= waves && (bpw + 1) * 32 * waves <= kFuseMaxRows) {
        *extra = int(r);
        return g;
    }
    *extra = 0;
    return g + (r > 0 ? 1 : 0);
}

struct SelArgs {
    int k, r;
    int64_t S;
    int64_t n_stride;
    const uint32_t* keys;
    int32_t* sel;
    int32_t* cand;             // split selection: [B][S][n_chunks][k] candidate rows
    uint32_t* cand_key;        // and their keys (0 for a -1 candidate)
    int chunk, n_chunks;       // rows per chunk, chunks per query
    // fused decode selection: the scorer's per-workgroup candidates (see IdxMfmaArgs)
    const uint32_t* f_key;
    const int32_t* f_row;
    const uint32_t* f_cutoff;
    int f_groups, f_m, f_rows_per_group;
};

// The k best of nv keys in global memory for one query, by NT threads: four 8-bit radix
// passes over the keys, then compaction in row order over contiguous per-thread segments.
// `shm` holds at least 256 + 2 NT + 4 ints.  For any row count.
template <int NT>
__device__ void select_keys_mem(const uint32_t* key, int64_t nv, int k, int32_t* out, int* shm) {
    uint32_t* hist = reinterpret_cast<uint32_t*>(shm);
    int32_t* cnt_gt = shm + 256;
    int32_t* cnt_eq = shm + 256 + NT;
    int32_t* shs = shm + 256 + 2 * NT;
    const int tid = threadIdx.x;
    uint32_t prefix = 0, mask = 0;
    int32_t rem = k;
    for (int shift = 24; shift >= 0; shift -= 8) {
        for (int i = tid; i < 256; i += NT) hist[i] = 0;
        __syncthreads();
        for (int64_t j = tid; j < nv; j += NT) {
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
            shs[0] = d;
            shs[1] = rem - cum;
        }
        __syncthreads();
        prefix |= uint32_t(shs[0]) << shift;
        mask |= 255u << shift;
        rem = shs[1];
        __syncthreads();
    }
    const uint32_t thr = prefix;     // the k-th largest key; take `rem` rows equal to it
    const int64_t seg = (nv + NT - 1) / NT;
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
        for (int i = 0; i < NT; ++i) {
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

// One workgroup selects for one query, keys in global memory (any row count).
constexpr int kSelThreads = 256;
__global__ void __launch_bounds__(kSelThreads)
topk_select_kernel(SelArgs a, SeqInts pos0, SeqInts n_rows) {
    __shared__ int shm[256 + 2 * kSelThreads + 4];
    const int b = blockIdx.y;
    const int64_t s = blockIdx.x;
    const int64_t p = int64_t(pos0.v[b]) + s;
    int64_t nv = (p + 1) / a.r;
    if (nv > n_rows.v[b]) nv = n_rows.v[b];
    int32_t* out = a.sel + (size_t(b) * a.S + size_t(s)) * a.k;
    if (nv <= a.k) {                                  // dense regime: every visible row
        for (int i = threadIdx.x; i < a.k; i += blockDim.x) out[i] = i < nv ? i : -1;
        return;
    }
    select_keys_mem<kSelThreads>(a.keys + (size_t(b) * a.S + size_t(s)) * a.n_stride, nv, a.k, out, shm);
}

// ------------------------------------------------------------------ select with keys in registers
// For up to NT * KPT visible rows.  Split selection, for few queries over many rows: stage 1
// (SEL_CHUNK) selects the k best of each chunk of a.chunk rows into a candidate list, stage 2
// (SEL_MERGE) the k best of those candidates.  The order (key descending, then row ascending)
// is total, so a row among a query's k best is among the k best of its chunk, and the
// candidate lists, chunk after chunk and ascending within one, are in row order: the lower
// position wins a tie, and the rows come out ascending.  Stage 1 stores each candidate's key
// beside its row; a candidate -1 (a chunk with k rows or fewer) has key 0.
enum SelMode { SEL_DIRECT = 0, SEL_CHUNK = 1, SEL_MERGE = 2 };
constexpr int64_t kSelRegMaxRows = 1024 * 68;   // largest lane the register select holds

template <int KPT, int NT, int MODE>
__global__ void __launch_bounds__(NT)
topk_select_reg_kernel(SelArgs a, SeqInts pos0, SeqInts n_rows) {
    constexpr int G = KPT / 4;                         // groups of 4 keys per lane
    __shared__ __align__(16) uint32_t hist[kHistWords];
    __shared__ int tmp[2 * NT / 64];
    __shared__ int sh[4];
    __shared__ int wtot[2][NT / 64];
    const int b = blockIdx.y;
    const int s = blockIdx.x;
    const int p = pos0.v[b] + s;
    int nv = (p + 1) / a.r;
    if (nv > n_rows.v[b]) nv = n_rows.v[b];
    const size_t q = size_t(b) * a.S + size_t(s);
    const uint32_t* gk = a.keys + q * a.n_stride;
    const size_t cbase = q * size_t(a.n_chunks) * a.k;   // this query's candidates
    const int32_t* cq = a.cand + cbase;
    int32_t* out = a.sel + q * a.k;
    uint32_t* okey = nullptr;                          // stage 1: keys of the candidates
    int base = 0;                                      // row of key 0 (stage 1)
    int n = nv;                                        // keys selected among
    if (MODE == SEL_CHUNK) {
        base = int(blockIdx.z) * a.chunk;
        n = nv - base < a.chunk ? nv - base : a.chunk;
        n = n > 0 ? n : 0;
        gk += base;
        out = a.cand + cbase + blockIdx.z * size_t(a.k);
        okey = a.cand_key + cbase + blockIdx.z * size_t(a.k);
    }
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    if (n <= a.k) {
        for (int i = tid; i < a.k; i += blockDim.x) {
            out[i] = i < n ? base + i : -1;
            if (MODE == SEL_CHUNK) okey[i] = i < n ? gk[i] : 0u;
        }
        return;
    }
    if (MODE == SEL_MERGE) n = a.n_chunks * a.k;       // candidate positions
    const int wbase = w * 64 * KPT + 4 * lane;
    uint32_t key[KPT];
    int32_t crow[KPT];                                 // stage 2: the candidates' rows
#pragma unroll
    for (int i = 0; i < G; ++i) {
        const int j = wbase + 256 * i;
        if (MODE == SEL_MERGE) {
            const uint32_t* ck = a.cand_key + cbase;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                key[4 * i + e] = j + e < n ? ck[j + e] : 0u;
                crow[4 * i + e] = j + e < n ? cq[j + e] : -1;
            }
        } else {
            uint4 v = make_uint4(0u, 0u, 0u, 0u);
            if (j < n) v = *reinterpret_cast<const uint4*>(gk + j);   // stride, chunk % 4 == 0
            key[4 * i + 0] = v.x;
            key[4 * i + 1] = j + 1 < n ? v.y : 0u;
            key[4 * i + 2] = j + 2 < n ? v.z : 0u;
            key[4 * i + 3] = j + 3 < n ? v.w : 0u;
        }
    }
    const int ngv = __builtin_amdgcn_readfirstlane(
        max(0, min(G, (n - w * 64 * KPT + 255) / 256)));   // groups holding a position below n
    const RegSelect rs = reg_select_threshold<KPT, NT, false>(key, ngv, a.k, hist, tmp, sh);
    constexpr int NW = NT / 64;
    const int seg = a.k < 64 * KPT ? a.k : 64 * KPT;  // most keys one wave can take
    if (rs.rem == 0 && NW * seg * (MODE == SEL_CHUNK ? 2 : 1) <= kHistWords) {
        // exactly k keys lie above the threshold: each wave stages the values of those it
        // holds in its own run of the histogram's memory (free once the threshold is known),
        // in position order; then the workgroup stores the runs one after another, coalesced
        int32_t* st = reinterpret_cast<int32_t*>(hist);
        int32_t* sw = st + w * seg;
        const int cnt = reg_compact_gt<KPT, NT, true>(key, rs.thr, nullptr, [&](int slot, int e, int pos) {
            sw[slot] = MODE == SEL_MERGE ? crow[e] : base + pos;
            if (MODE == SEL_CHUNK) sw[NW * seg + slot] = int32_t(key[e]);
        });
        if (lane == 0) wtot[0][w] = cnt;
        __syncthreads();
        int wc[NW];
#pragma unroll
        for (int v = 0; v < NW; ++v) wc[v] = wtot[0][v];
        for (int i = tid; i < a.k; i += NT) {
            int src = i, run = 0;                      // run v holds slots [sum wc[< v], + wc[v])
#pragma unroll
            for (int v = 0; v < NW - 1; ++v)
                if (run == v && src >= wc[v]) {
                    src -= wc[v];
                    run = v + 1;
                }
            out[i] = st[run * seg + src];
            if (MODE == SEL_CHUNK) okey[i] = uint32_t(st[NW * seg + run * seg + src]);
        }
        return;
    }
    if (rs.rem == 0 && a.k * (MODE == SEL_CHUNK ? 2 : 1) <= kHistWords) {
        // the same with workgroup slots (a count pass first) when the waves' runs do not fit
        int32_t* st = reinterpret_cast<int32_t*>(hist);
        reg_compact_gt<KPT, NT>(key, rs.thr, wtot[0], [&](int slot, int e, int pos) {
            st[slot] = MODE == SEL_MERGE ? crow[e] : base + pos;
            if (MODE == SEL_CHUNK) st[a.k + slot] = int32_t(key[e]);
        });
        __syncthreads();
        for (int i = tid; i < a.k; i += NT) {
            out[i] = st[i];
            if (MODE == SEL_CHUNK) okey[i] = uint32_t(st[a.k + i]);
        }
        return;
    }
    reg_compact<KPT, NT>(key, rs, wtot, [&](int slot, int e, int pos) {
        if (MODE == SEL_CHUNK) okey[slot] = key[e];
        out[slot] = MODE == SEL_MERGE ? crow[e] : base + pos;
    });
}

// Fused decode selection, stage 2: the k best of the scorer's per-workgroup candidates
// (each group's m best rows in row order, groups in row order, so the list is in row order
// and a tie goes to the lower row).  The result is exact when every row the scorer did not
// pass on ranks below every candidate taken: each group's cutoff (its largest key not passed
// on) must be at or below the threshold when the k taken are exactly the candidates above
// it, and below the k-th candidate key when a tie is split there; a query where some cutoff
// fails that selects from its full score keys instead (select_keys_mem), with the same
// result.
template <int KPT, int NT>
__global__ void __launch_bounds__(NT)
topk_fused_merge_kernel(SelArgs a, SeqInts pos0, SeqInts n_rows) {
    constexpr int G = KPT / 4;
    __shared__ __align__(16) uint32_t hist[kHistWords];
    __shared__ int tmp[2 * NT / 64];
    __shared__ int sh[4];
    __shared__ int wtot[2][NT / 64];
    __shared__ uint32_t red[NT / 64];
    const int b = blockIdx.y;
    const int s = blockIdx.x;
    const int p = pos0.v[b] + s;
    int nv = (p + 1) / a.r;
    if (nv > n_rows.v[b]) nv = n_rows.v[b];
    const size_t q = size_t(b) * a.S + size_t(s);
    int32_t* out = a.sel + q * a.k;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    if (nv <= a.k) {                                   // dense regime: every visible row
        for (int i = tid; i < a.k; i += NT) out[i] = i < nv ? i : -1;
        return;
    }
    int extra_blocks;
    const int groups = int(fused_groups((nv + 31) / 32, a.f_rows_per_group / (32 * kStreamWaves), kStreamWaves,
                                        &extra_blocks));
    const int n = groups * a.f_m;                      // candidate positions (<= NT * KPT)
    const uint32_t* ck = a.f_key + q * size_t(a.f_groups) * a.f_m;
    const int32_t* cr = a.f_row + q * size_t(a.f_groups) * a.f_m;
    const int wbase = w * 64 * KPT + 4 * lane;
    uint32_t key[KPT];
    int32_t crow[KPT];
#pragma unroll
    for (int i = 0; i < G; ++i) {
        const int j = wbase + 256 * i;
        uint4 kv = make_uint4(0u, 0u, 0u, 0u);
        int4 rv = make_int4(-1, -1, -1, -1);
        if (j < n) {                                   // n is a multiple of 4 (m is)
            kv = *reinterpret_cast<const uint4*>(ck + j);
            rv = *reinterpret_cast<const int4*>(cr + j);
        }
        key[4 * i + 0] = kv.x; key[4 * i + 1] = kv.y; key[4 * i + 2] = kv.z; key[4 * i + 3] = kv.w;
        crow[4 * i + 0] = rv.x; crow[4 * i + 1] = rv.y; crow[4 * i + 2] = rv.z; crow[4 * i + 3] = rv.w;
    }
    uint32_t cut = 0;                                  // largest key the scorer did not pass on
    for (int g = tid; g < groups; g += NT) {
        const uint32_t c = a.f_cutoff[q * size_t(a.f_groups) + g];
        cut = c > cut ? c : cut;
    }
    cut = block_max_u32<NT>(cut, red);
    const int ngv = __builtin_amdgcn_readfirstlane(max(0, min(G, (n - w * 64 * KPT + 255) / 256)));
    const RegSelect rs = reg_select_threshold<KPT, NT, false>(key, ngv, a.k, hist, tmp, sh);
    if (rs.rem == 0 && cut <= rs.thr && a.k <= kHistWords) {
        // the k candidates above rs.thr are taken, every row not passed on is at or below it
        int32_t* st = reinterpret_cast<int32_t*>(hist);
        reg_compact_gt<KPT, NT>(key, rs.thr, wtot[0], [&](int slot, int e, int) { st[slot] = crow[e]; });
        __syncthreads();
        for (int i = tid; i < a.k; i += NT) out[i] = st[i];
        return;
    }
    if (rs.rem > 0 && cut < rs.thr) {                  // a tie split at the k-th key rs.thr
        reg_compact<KPT, NT>(key, rs, wtot, [&](int slot, int e, int) { out[slot] = crow[e]; });
        return;
    }
    // some row not passed on reaches the k-th candidate key: select from every score key
    __syncthreads();
    select_keys_mem<NT>(a.keys + q * a.n_stride, nv, a.k, out, reinterpret_cast<int*>(hist));
}

// ------------------------------------------------------------------ decode scoring
// Decode scoring (each query's rows read once, no sharing between queries): the workgroup
// stages its query's 64 x 128 fragment in LDS once (16-byte chunks XOR-swizzled by head),
// then every wave streams its own contiguous run of 32-row blocks straight into registers,
// with the next block's loads in flight while the current one is scored.  MFMA k slots are
// ordered so that a lane holds 64 contiguous bytes of its row per 64-dim half: k slot
// 8 hi + e of MFMA ks = 4 d + j is dim 64 d + 32 hi + 8 j + e, in the query operand alike.
//
// FUSE (the fused indexer): the workgroup's rows (a contiguous run of rows_per_block) keep
// their keys in LDS as well, and after the scan the workgroup selects its m best (key
// descending, row ascending) by the same radix select and passes them on in row order, with
// the largest key it leaves out; the merge kernel above takes the query's k best of those.

__device__ __forceinline__ void idx_stream_block(const bf16* rows, int64_t blk, int64_t nv, uint4 (&kb)[8]) {
    const int lane = threadIdx.x & 63, l32 = lane & 31, hi = lane >> 5;
    int64_t j = blk * 32 + l32;
    j = j < nv ? j : nv - 1;                          // rows past the visible ones: scores not stored
    const bf16* rp = rows + size_t(j) * ID + 32 * hi;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        kb[c] = *reinterpret_cast<const uint4*>(rp + 8 * c);
        kb[4 + c] = *reinterpret_cast<const uint4*>(rp + 64 + 8 * c);
    }
}

template <int WAVES, bool FUSE>
__device__ __forceinline__ void index_score_stream_body(const IdxMfmaArgs& a, const SeqInts& pos0v,
                                                        const SeqInts& n_rows) {
    constexpr int NT = 64 * WAVES;
    const int b = blockIdx.z;
    const int64_t s = blockIdx.y;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int l32 = lane & 31, hi = lane >> 5;
    int64_t nv = (int64_t(pos0v.v[b]) + s + 1) / a.r;
    if (nv > n_rows.v[b]) nv = n_rows.v[b];
    const int64_t nbt = (nv + 31) / 32;                // 32-row blocks of this query
    const int bpw = a.rows_per_block / (32 * WAVES);   // blocks per wave
    int extra = 0;                                     // the fused last group's added blocks
    const int64_t ngroups = FUSE ? fused_groups(nbt, bpw, WAVES, &extra)
                                 : (nbt + int64_t(WAVES) * bpw - 1) / (int64_t(WAVES) * bpw);
    if (int64_t(blockIdx.x) >= ngroups) return;        // whole workgroup: no rows
    const int ex = int64_t(blockIdx.x) == ngroups - 1 ? extra : 0;
    __shared__ __attribute__((aligned(16))) unsigned char qs[IH * IROWB];
    {
        const bf16* qg = a.qi + (size_t(b) * a.S + size_t(s)) * IH * ID;
        for (int i = threadIdx.x; i < IH * 16; i += NT) {
            const int h = i >> 4, c = i & 15;
            const uint4 v = *reinterpret_cast<const uint4*>(qg + h * ID + c * 8);
            store16(qs + h * IROWB + ((c ^ (h & 15)) * 16), v);
        }
    }
    __syncthreads();
    const int64_t blk0 = int64_t(blockIdx.x) * WAVES * bpw + int64_t(w) * bpw + (w < ex ? w : ex);
    const int wb = bpw + (w < ex ? 1 : 0);
    const int nb = blk0 >= nbt ? 0 : int(nbt - blk0 < wb ? nbt - blk0 : wb);     // this wave's blocks
    const int64_t row0 = int64_t(blockIdx.x) * a.rows_per_block;                // the workgroup's first row
    __shared__ __attribute__((aligned(16))) uint32_t kl[FUSE ? kFuseMaxRows : 4];
    if (nb > 0) {
        // query operand in the permuted k order, head weights
        bf16x8 qa[2][8];
        float wsc[2][16];
#pragma unroll
        for (int m = 0; m < 2; ++m) {
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) {
                const int h = 32 * m + l32, c = 8 * (ks >> 2) + 4 * hi + (ks & 3);
                const uint4 v = *reinterpret_cast<const uint4*>(qs + h * IROWB + ((c ^ (h & 15)) * 16));
                __builtin_memcpy(&qa[m][ks], &v, 16);
            }
            const float* wr = a.w + (size_t(b) * a.S + size_t(s)) * IH;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const float4 v = *reinterpret_cast<const float4*>(wr + 32 * m + 8 * g + 4 * hi);
                wsc[m][4 * g + 0] = v.x * a.scale;
                wsc[m][4 * g + 1] = v.y * a.scale;
                wsc[m][4 * g + 2] = v.z * a.scale;
                wsc[m][4 * g + 3] = v.w * a.scale;
            }
        }
        const bf16* rows = a.rows + size_t(b) * a.row_cap * ID;
        uint32_t* keys = a.keys + (size_t(b) * a.S + size_t(s)) * a.n_stride;
        auto score = [&](const uint4 (&kb)[8], int64_t blk) {
            floatx16 c0, c1;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                c0[i] = 0.f;
                c1[i] = 0.f;
            }
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) {
                bf16x8 kv;
                __builtin_memcpy(&kv, &kb[ks], 16);
                c0 = mfma32x32x16(qa[0][ks], kv, c0);
                c1 = mfma32x32x16(qa[1][ks], kv, c1);
            }
            float s0 = 0.f, s1 = 0.f;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                s0 = fmaf(wsc[0][i], relu_bits(c0[i]), s0);
                s1 = fmaf(wsc[1][i], relu_bits(c1[i]), s1);
            }
            float sc = s0 + s1;
            sc = sum_xor32(sc);
            const int64_t jj = blk * 32 + l32;
            if (hi == 0 && jj < nv) {
                const uint32_t kk = score_key(sc);
                keys[jj] = kk;
                if (FUSE) kl[jj - row0] = kk;
            }
        };
        uint4 kb0[8], kb1[8];
        idx_stream_block(rows, blk0, nv, kb0);
        for (int u = 0; u < nb; u += 2) {
            if (u + 1 < nb) idx_stream_block(rows, blk0 + u + 1, nv, kb1);
            score(kb0, blk0 + u);
            if (u + 1 < nb) {
                if (u + 2 < nb) idx_stream_block(rows, blk0 + u + 2, nv, kb0);
                score(kb1, blk0 + u + 1);
            }
        }
    }
    if constexpr (FUSE) {
        __shared__ __align__(16) uint32_t hist[kHistWords];
        __shared__ int tmp[2 * WAVES];
        __shared__ int sh[4];
        __shared__ int wtot[2][WAVES];
        __shared__ uint32_t red[WAVES];
        __syncthreads();                               // every key of the workgroup in kl
        int64_t n64 = nv - row0;
        const int64_t cap = a.rows_per_block + 32 * int64_t(ex);
        n64 = n64 < cap ? n64 : cap;
        const int n = int(n64);                        // > 0: the workgroup has rows
        const size_t q = size_t(b) * a.S + size_t(s);
        uint32_t* ck = a.cand_key + (q * a.n_groups + blockIdx.x) * size_t(a.m);
        int32_t* cr = a.cand_row + (q * a.n_groups + blockIdx.x) * size_t(a.m);
        if (n <= a.m) {                                // every row passed on
            for (int i = threadIdx.x; i < a.m; i += NT) {
                ck[i] = i < n ? kl[i] : 0u;
                cr[i] = i < n ? int32_t(row0 + i) : -1;
            }
            if (threadIdx.x == 0) a.cutoff[q * a.n_groups + blockIdx.x] = 0u;
            return;
        }
        constexpr int KPT = kFuseKpt, G = KPT / 4;
        const int wbase = w * 64 * KPT + 4 * lane;
        uint32_t key[KPT];
#pragma unroll
        for (int i = 0; i < G; ++i) {
            const int j = wbase + 256 * i;
            uint4 v = make_uint4(0u, 0u, 0u, 0u);
            if (j < n) v = *reinterpret_cast<const uint4*>(kl + j);
            key[4 * i + 0] = v.x;
            key[4 * i + 1] = j + 1 < n ? v.y : 0u;
            key[4 * i + 2] = j + 2 < n ? v.z : 0u;
            key[4 * i + 3] = j + 3 < n ? v.w : 0u;
        }
        const int ngv = __builtin_amdgcn_readfirstlane(max(0, min(G, (n - w * 64 * KPT + 255) / 256)));
        const RegSelect rs = reg_select_threshold<KPT, NT, false>(key, ngv, a.m, hist, tmp, sh);
        uint32_t rest = 0;                             // largest key not passed on
        if (rs.rem == 0) {
            reg_compact_gt<KPT, NT>(key, rs.thr, wtot[0], [&](int slot, int e, int pos) {
                ck[slot] = key[e];
                cr[slot] = int32_t(row0 + pos);
            });
#pragma unroll
            for (int e = 0; e < KPT; ++e) rest = key[e] <= rs.thr && key[e] > rest ? key[e] : rest;
        } else {
            rest = reg_compact<KPT, NT>(key, rs, wtot, [&](int slot, int e, int pos) {
                ck[slot] = key[e];
                cr[slot] = int32_t(row0 + pos);
            });
        }
        rest = block_max_u32<NT>(rest, red);
        if (threadIdx.x == 0) a.cutoff[q * a.n_groups + blockIdx.x] = rest;
    }
}

// The plain streamed scorer (score keys to the workspace) and the fused one (each workgroup
// passes on its best rows): one body, two kernels, so each has a name of its own in traces.
template <int WAVES>
__global__ void __launch_bounds__(64 * WAVES)
index_score_stream_kernel(IdxMfmaArgs a, SeqInts pos0v, SeqInts n_rows) {
    index_score_stream_body<WAVES, false>(a, pos0v, n_rows);
}

template <int WAVES>
__global__ void __launch_bounds__(64 * WAVES)
index_score_fused_kernel(IdxMfmaArgs a, SeqInts pos0v, SeqInts n_rows) {
    index_score_stream_body<WAVES, true>(a, pos0v, n_rows);
}


constexpr int kSelChunk = 8192;                       // rows per chunk of a split selection
constexpr int kMergeThreads = 512;                    // workgroup of the merge stages
static_assert(kSelChunk % 2048 == 0 && kSelChunk <= 512 * 64, "chunk: 512 threads x 4k keys");

// Chunks per query of a split selection, 0 for one workgroup per query.  The split pays where
// a call has too few queries to fill the chip (at most 64) and many rows each (above 16,384),
// and its merge stage holds all n_chunks x k candidates in registers (64 per thread).
int64_t topk_chunks(int64_t queries, int64_t n_max, int k) {
    if (queries > 64 || n_max <= 16384) return 0;
    const int64_t c = (n_max + kSelChunk - 1) / kSelChunk;
    return c * k <= kMergeThreads * 64 ? c : 0;
}

// The fused decode indexer's shape for a call: fewer than 8 queries per sequence (decode),
// the MFMA scorer, and each scoring workgroup passing on m rows, m the smallest multiple of
// 32 of at least three times the workgroup's expected share of the k best (k * rows_per_group
// / n for the sparsest sequence of the call), so that a group's m best hold all of its share
// but with vanishing probability (the merge checks it).  At most 128 rows per group and 8192
// candidates per query.
struct FusedPlan {
    bool on = false;
    int bpw = 0, rows_per_group = 0, m = 0;
    int64_t groups = 0;
};

FusedPlan fused_plan(bool mfma, int64_t S, int batch, int64_t n_max, int64_t n_min_sparse, int k) {
    FusedPlan f;
    if (!mfma || S >= kIdxWaves || n_max <= k || n_min_sparse <= k) return f;
    const int64_t queries = int64_t(batch < kSeqSlice ? batch : kSeqSlice) * S;
    const int64_t nbt = (n_max + 31) / 32;
    // blocks per wave: the fewest whose row groups still give at most one workgroup per CU over
    // the call's queries, else an even share rounded up
    int64_t bpw = nbt * queries / (256 * kStreamWaves);
    bpw = bpw < 1 ? 1 : bpw;
    int extra;
    if (bpw * 32 * kStreamWaves > kFuseMaxRows ||
        fused_groups(nbt, int(bpw), kStreamWaves, &extra) * queries > 256)
        bpw = (nbt * queries + 256 * kStreamWaves - 1) / (256 * kStreamWaves);
    if (bpw * 32 * kStreamWaves > kFuseMaxRows) return f;
    f.bpw = int(bpw);
    f.rows_per_group = f.bpw * 32 * kStreamWaves;
    // m >= 3 k rows_per_group / n_min_sparse, rounded up to a multiple of 32
    const int64_t m = ((3 * int64_t(k) * f.rows_per_group + n_min_sparse - 1) / n_min_sparse + 31) / 32 * 32;
    if (m > 128) return f;
    f.m = int(m < 32 ? 32 : m);
    f.groups = fused_groups(nbt, f.bpw, kStreamWaves, &extra);
    if (f.groups * f.m > 8192) return f;
    f.on = true;
    return f;
}

// Candidate area of a fused call: keys and rows [queries][groups][m], cutoffs [queries][groups].
size_t fused_cand_bytes(int64_t groups, int m, int batch, int64_t S) {
    const size_t qg = size_t(batch) * size_t(S) * size_t(groups);
    return qg * size_t(m) * 2 * sizeof(uint32_t) + qg * sizeof(uint32_t);
}

// Bytes of the score-key part of the workspace (the candidate lists follow, 256-aligned).
size_t index_keys_bytes(int batch, int64_t S, int64_t n_stride) {
    return (size_t(batch) * size_t(S) * size_t(n_stride) * sizeof(uint32_t) + 255) & ~size_t(255);
}

template <typename T>
hipError_t run(const IndexJob& j, hipStream_t st) {
    const bool mfma = use_index_mfma(j.bf16, j.Hi, j.di);
    // rows of the sequences in the sparse regime at their first query
    int64_t n_min_sparse = int64_t(1) << 62;
    for (int b = 0; b < j.batch; ++b) {
        const int64_t nv = std::min<int64_t>((j.pos0[b] + 1) / j.r, j.n_rows[b]);
        if (nv > j.k) n_min_sparse = std::min(n_min_sparse, nv);
    }
    const FusedPlan fp = fused_plan(mfma, j.S, j.batch, j.n_max, n_min_sparse, j.k);
    const int64_t n_chunks = fp.on ? 0 : topk_chunks(int64_t(j.batch) * j.S, j.n_max, j.k);
    char* tail = reinterpret_cast<char*>(j.keys) + index_keys_bytes(j.batch, j.S, j.n_stride);
    int32_t* cand = reinterpret_cast<int32_t*>(tail);
    // fused candidates: keys, rows, cutoffs
    uint32_t* f_key = reinterpret_cast<uint32_t*>(tail);
    const size_t fq = size_t(j.batch) * j.S * size_t(fp.groups);
    int32_t* f_row = reinterpret_cast<int32_t*>(f_key + fq * fp.m);
    uint32_t* f_cut = reinterpret_cast<uint32_t*>(f_row + fq * fp.m);
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
        if (nv_max > j.k && mfma) {
            IdxMfmaArgs a{};
            a.qi = static_cast<const bf16*>(j.qi) + qoff * IH * ID;
            a.w = j.w + qoff * IH;
            a.rows = static_cast<const bf16*>(j.rows) + size_t(b0) * j.row_cap * ID;
            a.row_cap = j.row_cap;
            a.S = j.S;
            a.n_stride = j.n_stride;
            a.keys = j.keys + qoff * j.n_stride;
            a.r = j.r;
            a.scale = 1.0f / sqrtf(float(j.di)) / sqrtf(float(j.Hi));
            if (j.S >= kIdxWaves && nv_max >= kIdxRsMinRows) {
                // row-stationary: RSB-row blocks x query groups, about one workgroup per CU
                const int64_t rb = (nv_max + RSB - 1) / RSB;
                int64_t ng = (256 + rb * nb - 1) / (rb * nb);
                const int64_t max_groups = (j.S + kIdxWaves - 1) / kIdxWaves;
                if (ng > max_groups) ng = max_groups;
                if (ng < 1) ng = 1;
                int64_t qpg = (j.S + ng - 1) / ng;
                qpg = (qpg + kIdxWaves - 1) / kIdxWaves * kIdxWaves;
                a.queries_per_group = int(qpg);
                ng = (j.S + qpg - 1) / qpg;
                DSV4_LAUNCH("index_score_rs", index_score_rs_kernel<kIdxWaves>, dim3(unsigned(rb), unsigned(ng), nb),
                            dim3(64 * kIdxWaves), 0, st, a, pos, nr);
            } else if (j.S >= kIdxWaves) {
                // query-stationary: blocks of rows x groups of 8 queries, ~2048 workgroups
                const int64_t groups = (j.S + kIdxWaves - 1) / kIdxWaves;
                int64_t blocks = (2048 + groups * nb - 1) / (groups * nb);
                const int64_t tiles = (nv_max + IRT - 1) / IRT;
                if (blocks > tiles) blocks = tiles;
                if (blocks < 1) blocks = 1;
                a.rows_per_block = int(((tiles + blocks - 1) / blocks) * IRT);
                const unsigned gx = unsigned((nv_max + a.rows_per_block - 1) / a.rows_per_block);
                DSV4_LAUNCH("index_score_mfma", (index_score_mfma_kernel<kIdxWaves, kIdxStages>),
                            dim3(gx, unsigned(groups), nb), dim3(64 * kIdxWaves), 0, st, a, pos, nr);
            } else if (fp.on) {
                // fused decode scoring: groups of rows_per_group rows, each passing on its m best
                a.rows_per_block = fp.rows_per_group;
                a.cand_key = f_key + qoff * fp.groups * fp.m;
                a.cand_row = f_row + qoff * fp.groups * fp.m;
                a.cutoff = f_cut + qoff * fp.groups;
                a.n_groups = int(fp.groups);
                a.m = fp.m;
                DSV4_LAUNCH("index_score_fused", (index_score_fused_kernel<kStreamWaves>),
                            dim3(unsigned(fp.groups), unsigned(j.S), nb), dim3(64 * kStreamWaves), 0, st,
                            a, pos, nr);
            } else {
                // decode: blocks per wave so the chip gets about 256 workgroups
                const int64_t nbt = (nv_max + 31) / 32;
                int64_t bpw = (nbt * j.S * nb + 256 * kStreamWaves - 1) / (256 * kStreamWaves);
                if (bpw < 1) bpw = 1;
                if (bpw > (int64_t(1) << 20)) bpw = int64_t(1) << 20;   // rows_per_block fits an int
                a.rows_per_block = int(bpw * 32 * kStreamWaves);
                const unsigned sx = unsigned((nbt + bpw * kStreamWaves - 1) / (bpw * kStreamWaves));
                DSV4_LAUNCH("index_score_stream", (index_score_stream_kernel<kStreamWaves>),
                            dim3(sx, unsigned(j.S), nb), dim3(64 * kStreamWaves), 0, st, a, pos, nr);
            }
            hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
        } else if (nv_max > j.k) {
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
            DSV4_LAUNCH("index_score", index_score_kernel<T>, dim3(gx, unsigned(j.S), nb),
                               dim3(kScoreThreads), lds, st, a, pos, nr);
            hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
        SelArgs sa{};
        sa.k = j.k; sa.r = j.r; sa.S = j.S; sa.n_stride = j.n_stride;
        sa.keys = j.keys + qoff * j.n_stride;
        sa.sel = j.sel + qoff * j.k;
        sa.chunk = kSelChunk;
        sa.n_chunks = int(n_chunks);
        sa.cand = cand + qoff * size_t(n_chunks) * j.k;
        sa.cand_key = reinterpret_cast<uint32_t*>(cand + size_t(j.batch) * j.S * n_chunks * j.k) +
                      qoff * size_t(n_chunks) * j.k;
        constexpr int MT = kMergeThreads;
        if (fp.on) {
            sa.f_key = f_key + qoff * fp.groups * fp.m;
            sa.f_row = f_row + qoff * fp.groups * fp.m;
            sa.f_cutoff = f_cut + qoff * fp.groups;
            sa.f_groups = int(fp.groups);
            sa.f_m = fp.m;
            sa.f_rows_per_group = fp.rows_per_group;
            const int64_t nc = fp.groups * fp.m;
            if (nc <= MT * 4)
                DSV4_LAUNCH("topk_fused_merge", (topk_fused_merge_kernel<4, MT>),
                            dim3(unsigned(j.S), nb), dim3(MT), 0, st, sa, pos, nr);
            else if (nc <= MT * 8)
                DSV4_LAUNCH("topk_fused_merge", (topk_fused_merge_kernel<8, MT>),
                            dim3(unsigned(j.S), nb), dim3(MT), 0, st, sa, pos, nr);
            else
                DSV4_LAUNCH("topk_fused_merge", (topk_fused_merge_kernel<16, MT>),
                            dim3(unsigned(j.S), nb), dim3(MT), 0, st, sa, pos, nr);
        } else if (n_chunks > 0) {
            // stage 1 over (query, chunk), stage 2 over the n_chunks x k candidates
            DSV4_LAUNCH("topk_select_reg", (topk_select_reg_kernel<kSelChunk / 512, 512, SEL_CHUNK>),
                        dim3(unsigned(j.S), nb, unsigned(n_chunks)), dim3(512), 0, st, sa, pos, nr);
            hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
            const int64_t nc = n_chunks * j.k;
            if (nc <= MT * 8)
                DSV4_LAUNCH("topk_merge", (topk_select_reg_kernel<8, MT, SEL_MERGE>),
                            dim3(unsigned(j.S), nb), dim3(MT), 0, st, sa, pos, nr);
            else if (nc <= MT * 16)
                DSV4_LAUNCH("topk_merge", (topk_select_reg_kernel<16, MT, SEL_MERGE>),
                            dim3(unsigned(j.S), nb), dim3(MT), 0, st, sa, pos, nr);
            else if (nc <= MT * 32)
                DSV4_LAUNCH("topk_merge", (topk_select_reg_kernel<32, MT, SEL_MERGE>),
                            dim3(unsigned(j.S), nb), dim3(MT), 0, st, sa, pos, nr);
            else
                DSV4_LAUNCH("topk_merge", (topk_select_reg_kernel<64, MT, SEL_MERGE>),
                            dim3(unsigned(j.S), nb), dim3(MT), 0, st, sa, pos, nr);
        } else if (nv_max <= 512 * 32) {
            // keys in registers: 512 threads x 4 .. 64 keys, 1024 threads x 68 keys (69,632
            // rows, which covers a 262,144-token ratio-4 lane plus its decode steps); beyond,
            // in memory.  Wave w holds rows 64 KPT w .. 64 KPT (w + 1) - 1, so KPT follows the
            // row count: every wave of the workgroup shares the histogram atomics
            if (nv_max <= 512 * 4)
                DSV4_LAUNCH("topk_select_reg", (topk_select_reg_kernel<4, 512, SEL_DIRECT>),
                            dim3(unsigned(j.S), nb), dim3(512), 0, st, sa, pos, nr);
            else if (nv_max <= 512 * 8)
                DSV4_LAUNCH("topk_select_reg", (topk_select_reg_kernel<8, 512, SEL_DIRECT>),
                            dim3(unsigned(j.S), nb), dim3(512), 0, st, sa, pos, nr);
            else if (nv_max <= 512 * 16)
                DSV4_LAUNCH("topk_select_reg", (topk_select_reg_kernel<16, 512, SEL_DIRECT>),
                            dim3(unsigned(j.S), nb), dim3(512), 0, st, sa, pos, nr);
            else
                DSV4_LAUNCH("topk_select_reg", (topk_select_reg_kernel<32, 512, SEL_DIRECT>),
                            dim3(unsigned(j.S), nb), dim3(512), 0, st, sa, pos, nr);
        } else if (nv_max <= 512 * 64) {
            DSV4_LAUNCH("topk_select_reg", (topk_select_reg_kernel<64, 512, SEL_DIRECT>),
                        dim3(unsigned(j.S), nb), dim3(512), 0, st, sa, pos, nr);
        } else if (nv_max <= kSelRegMaxRows) {
            DSV4_LAUNCH("topk_select_reg", (topk_select_reg_kernel<68, 1024, SEL_DIRECT>),
                        dim3(unsigned(j.S), nb), dim3(1024), 0, st, sa, pos, nr);
        } else {
            DSV4_LAUNCH("topk_select", topk_select_kernel, dim3(unsigned(j.S), nb), dim3(kSelThreads), 0,
                        st, sa, pos, nr);
        }
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace

int64_t index_key_stride(int64_t n_max) { return ((n_max < 1 ? 1 : n_max) + 3) & ~int64_t(3); }

size_t index_workspace_bytes(int Hi, int di, int k, int batch, int64_t S, int64_t n_max) {
    // a fused call's groups follow n_max alone; its m grows as the call's sparsest sequence
    // gets shorter, up to 128: the area is sized for that bound
    const FusedPlan fp = fused_plan(use_index_mfma(true, Hi, di), S, batch, n_max, n_max, k);
    const int64_t c = topk_chunks(int64_t(batch) * S, n_max, k);
    const size_t split = 2 * size_t(batch) * size_t(S) * size_t(c) * size_t(k) * sizeof(int32_t);
    const size_t fused = fp.on ? fused_cand_bytes(fp.groups, 128, batch, S) : 0;
    return index_keys_bytes(batch, S, index_key_stride(n_max)) + (split > fused ? split : fused);
}

hipError_t launch_index_topk(const IndexJob& j, hipStream_t s) {
    return j.bf16 ? run<bf16>(j, s) : run<float>(j, s);
}

}  // namespace dsv4
