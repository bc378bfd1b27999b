// The layer's neighbours on either side of the attention (gfx950, wave64):
//   rope_kernel          RoPE of the last rd dims of every head of every token (q, kv, qi),
//                        or its inverse (the attention output): interleaved pairs turned by
//                        position * inv_freq, angle and rotation in fp32, rounded to storage;
//   gproj_small_kernel   grouped (block-diagonal) output projection for up to 32 tokens
//                        (decode): weight streaming, HBM-bound -- each 32-row block of a
//                        group's weight is read once, straight into registers, by 8 waves
//                        that split K and meet in LDS;
//   gproj_tile_kernel    the same for more tokens (prefill): MFMA-bound 256 x 256 tiles of
//                        8 waves (128 x 128 of 4 waves for smaller grids), both operands
//                        staged in LDS by direct global-to-LDS copies, a ring of k blocks;
//   gproj_generic_kernel any shape or fp32: one thread per output.
// Every product accumulates in fp32 (v_mfma_f32_32x32x16_bf16 on the bf16 paths); outputs
// are rounded once to the storage type.
#include "common.hpp"
#include "mfma.hpp"
#include "proj.hpp"

namespace dsv4 {

namespace {

// ------------------------------------------------------------------ RoPE
constexpr int kRopeHeadsPerThread = 8;   // one angle serves 8 heads of the token

template <typename T>
struct RopeArgs {
    int H, D, rd;
    bool inverse;
    T* x;
    const float* inv_freq;
    int64_t S;
};

template <typename T>
__global__ void __launch_bounds__(256) rope_kernel(RopeArgs<T> a, SeqInts pos0) {
    const int P = a.rd / 2;
    const int HC = (a.H + kRopeHeadsPerThread - 1) / kRopeHeadsPerThread;
    const int item = int(blockIdx.x) * 256 + int(threadIdx.x);      // (head chunk, pair)
    if (item >= HC * P) return;
    const int hc = item / P, i = item % P;
    const int64_t s = blockIdx.y;
    const int b = blockIdx.z;
    T* base = a.x + (size_t(b) * a.S + size_t(s)) * a.H * a.D + (a.D - a.rd) + 2 * i;
    const int h0 = hc * kRopeHeadsPerThread;
    const int nh = a.H - h0 < kRopeHeadsPerThread ? a.H - h0 : kRopeHeadsPerThread;
    // every head's pair is loaded before any is stored (in place: a load after a store to the
    // same array would wait for it, one round trip per head); heads past H load the last one,
    // unconditionally, so no load sits in a branch that waits for it
    float x0[kRopeHeadsPerThread], x1[kRopeHeadsPerThread];
#pragma unroll
    for (int k = 0; k < kRopeHeadsPerThread; ++k) {
        const T* px = base + size_t(k < nh ? h0 + k : a.H - 1) * a.D;
        x0[k] = to_f32(px[0]);
        x1[k] = to_f32(px[1]);
    }
    // fp32 angle of the fp32 position, as the compressor's rows
    const float p = float(int64_t(pos0.v[b]) + s);
    float sn, cs;
    sincosf(p * a.inv_freq[i], &sn, &cs);
    if (a.inverse) sn = -sn;
#pragma unroll
    for (int k = 0; k < kRopeHeadsPerThread; ++k) {
        if (k < nh) {
            T* px = base + size_t(h0 + k) * a.D;
            px[0] = from_f32<T>(x0[k] * cs - x1[k] * sn);
            px[1] = from_f32<T>(x0[k] * sn + x1[k] * cs);
        }
    }
}

// ------------------------------------------------------------------ grouped projection
struct GprojArgs {
    int G, K, R;
    const bf16* x;             // [T][G][K]
    const bf16* w;             // [G][R][K]
    bf16* y;                   // [T][G][R]
    int64_t T;
    const bf16* w2;            // with G = 1: a second weight [R][K] and output [T][R] over the
    bf16* y2;                  // same x, taken by the workgroups of blockIdx.z = 1 (else null)
};

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4& v) {
    bf16x8 r;
    __builtin_memcpy(&r, &v, 16);
    return r;
}

// MFMA k-slot order: in a 64-wide k block, lane (m, hh) of MFMA j holds k = 32 hh + 8 j + e,
// so the 4 MFMAs of a block take a lane's 64 contiguous bytes of its row (A and B alike).
constexpr int kSmallWaves = 8;          // (16 measured: no change)
constexpr int kSmallMaxT = 32;

// Up to 32 tokens: workgroup (32-row block, group); wave w of the W waves multiplies k in
// [w K/W, (w+1) K/W) (KBW blocks of 64), the W partial 32 x 32 tiles meet in LDS.
template <int KBW>
__global__ void __launch_bounds__(64 * kSmallWaves) gproj_small_kernel(GprojArgs a) {
    __shared__ float part[kSmallWaves][32 * 33];
    const int rb = blockIdx.x, g = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int m = lane & 31, hh = lane >> 5;
    const int k0 = w * 64 * KBW + 32 * hh;
    const bf16* wrow = a.w + (size_t(g) * a.R + size_t(rb) * 32 + m) * a.K + k0;
    const bool tv = m < a.T;
    const bf16* xrow = a.x + (size_t(tv ? m : 0) * a.G + g) * a.K + k0;
    uint4 wv[KBW][4];
#pragma unroll
    for (int kb = 0; kb < KBW; ++kb)
#pragma unroll
        for (int c = 0; c < 4; ++c) wv[kb][c] = *reinterpret_cast<const uint4*>(wrow + kb * 64 + 8 * c);
    floatx16 acc;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.f;
#pragma unroll
    for (int kb = 0; kb < KBW; ++kb) {
        uint4 xv[4];
#pragma unroll
        for (int c = 0; c < 4; ++c)   // lanes past T read token 0 (their columns are not stored)
            xv[c] = *reinterpret_cast<const uint4*>(xrow + kb * 64 + 8 * c);
#pragma unroll
        for (int j = 0; j < 4; ++j) acc = mfma32x32x16(as_bf16x8(wv[kb][j]), as_bf16x8(xv[j]), acc);
    }
    // C[row][token]: register i of lane l is row c_row(i, l), token l % 32
#pragma unroll
    for (int i = 0; i < 16; ++i) part[w][c_row(i, lane) * 33 + m] = acc[i];
    __syncthreads();
    for (int o = tid; o < 32 * 32; o += 64 * kSmallWaves) {
        const int t = o >> 5, row = o & 31;
        if (t >= a.T) continue;
        float s = 0.f;
#pragma unroll
        for (int v = 0; v < kSmallWaves; ++v) s += part[v][row * 33 + t];
        a.y[(size_t(t) * a.G + g) * a.R + size_t(rb) * 32 + row] = from_f32<bf16>(s);
    }
}

// More tokens: workgroup tile of 32 TM WT tokens x 32 RN WR rows of one group, WT x WR waves,
// each a block of 32 TM tokens x 32 RN rows (TM x RN MFMA blocks; C[token][row]).  k in
// blocks of KD (64 or 128), ST of them resident in LDS as a ring.  A stage holds the tile's
// token rows and weight rows of 2 KD bytes, the 16-byte chunks of each row XOR-swizzled (see
// TileShape::swz) so the 16 rows of one MFMA operand read phase hit 16 different 16-byte
// bank groups.  Token rows past T load row T - 1 (finite values whose outputs are not
// stored).
constexpr int kTileK = 64;                               // k multiple every tile shape takes
constexpr int kOperandLead = 1;                          // k steps of operands read ahead

template <int WT, int WR, int TM, int RN, int ST, int KD>
struct TileShape {
    static constexpr int waves = WT * WR;
    static constexpr int T = 32 * TM * WT, R = 32 * RN * WR;
    static constexpr int stages = ST;                          // k blocks resident in LDS
    static constexpr int kd = KD;                              // k per block
    static constexpr int row_bytes = KD * 2;                   // bytes per staged row
    static constexpr int cpr = row_bytes / 16;                 // 16-byte chunks per row
    static constexpr int rows_per_op = 1024 / row_bytes;       // rows per 1 KB copy
    static constexpr int stage_bytes = (T + R) * row_bytes;
    static constexpr int ops = (T + R) / rows_per_op / waves;  // 1 KB copies per wave per stage
    static_assert(KD % kTileK == 0 && (KD == 64 || KD == 128), "k block of 64 or 128");
    static_assert((T + R) % (rows_per_op * waves) == 0, "whole copies per wave");
    static_assert(ST >= 2 && (ST - 2) * ops < 64, "copies in flight fit the wait counter");
    // the 16 rows of one MFMA operand read phase land in 16 different 16-byte bank groups
    __device__ static int swz(int row, int chunk) { return chunk ^ ((row / (16 / cpr)) % cpr); }
};

typedef __attribute__((address_space(3))) unsigned char lds_u8;

__device__ __forceinline__ void dma16(const void* gptr, const unsigned char* lds_base) {
    const uint32_t la = __builtin_amdgcn_readfirstlane(uint32_t(size_t((const lds_u8*)lds_base)));
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
                 :: "s"(la), "v"(gptr) : "memory", "m0");
}

template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Copy k block kb of the tile into stage buffer buf: 1 KB copies of rows_per_op rows; wave w
// takes copies w, w + waves, ... (the token rows first, then the weight rows).
template <class SH>
__device__ __forceinline__ void tile_load(const GprojArgs& a, const bf16* wg, int g, int64_t t0, int r0, int kb,
                                          unsigned char* buf) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
    for (int i = 0; i < SH::ops; ++i) {
        const int op = w + SH::waves * i;
        const int row = SH::rows_per_op * op + lane / SH::cpr;   // row of the stage
        const int c = SH::swz(row, lane % SH::cpr);      // logical chunk landing at lane % cpr
        const bf16* src;
        if (row < SH::T) {
            int64_t t = t0 + row;
            t = t < a.T ? t : a.T - 1;
            src = a.x + (size_t(t) * a.G + g) * a.K + size_t(kb) * SH::kd + 8 * c;
        } else {
            const int r = r0 + row - SH::T;
            src = wg + (size_t(g) * a.R + r) * a.K + size_t(kb) * SH::kd + 8 * c;
        }
        dma16(src, buf + op * 1024);
    }
}

template <int WT, int WR, int TM, int RN, int ST, int KD>
__global__ void __launch_bounds__(64 * WT * WR) gproj_tile_kernel(GprojArgs a) {
    using SH = TileShape<WT, WR, TM, RN, ST, KD>;
    __shared__ __attribute__((aligned(16))) unsigned char st[ST][SH::stage_bytes];
    // blockIdx.z: the group, or with a second pair (G = 1) which of the two products
    const bool second = a.w2 != nullptr && blockIdx.z == 1;
    const int g = a.w2 != nullptr ? 0 : int(blockIdx.z);
    const bf16* wsel = second ? a.w2 : a.w;
    bf16* ysel = second ? a.y2 : a.y;
    const int64_t t0 = int64_t(blockIdx.x) * SH::T;
    const int r0 = int(blockIdx.y) * SH::R;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int m = lane & 31, hh = lane >> 5;
    const int wt = w % WT, wr = w / WT;                  // wave tile: tokens 32 TM wt, rows 32 RN wr
    const int nk = a.K / SH::kd;
    floatx16 acc[TM][RN];
#pragma unroll
    for (int u = 0; u < TM; ++u)
#pragma unroll
        for (int v = 0; v < RN; ++v)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[u][v][i] = 0.f;
#pragma unroll
    for (int s = 0; s < ST - 1; ++s)
        if (s < nk) tile_load<SH>(a, wsel, g, t0, r0, s, st[s]);
    for (int kb = 0; kb < nk; ++kb) {
        // block kb has landed once at most the copies of the ST - 2 blocks behind it are
        // outstanding (near the end, where fewer follow it, wait for every copy)
        if (kb + ST - 2 < nk) wait_vm<(ST - 2) * SH::ops>(); else wait_vm<0>();
        lds_barrier();                                   // block kb visible; kb-1 fully read
        if (kb + ST - 1 < nk) tile_load<SH>(a, wsel, g, t0, r0, kb + ST - 1, st[(kb + ST - 1) % ST]);
        const unsigned char* buf = st[kb % ST];
        constexpr int NJ = SH::kd / 16;                  // MFMA k steps of this block
        bf16x8 xa[NJ][TM], wb[NJ][RN];
        auto load_step = [&](int j) {
            const int lc = 2 * j + hh;                   // logical chunk of this lane
#pragma unroll
            for (int u = 0; u < TM; ++u) {
                const int row = 32 * TM * wt + 32 * u + m;
                xa[j][u] = load_bf16x8(buf + row * SH::row_bytes + SH::swz(row, lc) * 16);
            }
#pragma unroll
            for (int v = 0; v < RN; ++v) {
                const int row = SH::T + 32 * RN * wr + 32 * v + m;
                wb[j][v] = load_bf16x8(buf + row * SH::row_bytes + SH::swz(row, lc) * 16);
            }
        };
        // a k step's operands are read kOperandLead steps ahead of its MFMAs, so their LDS
        // latency hides behind the MFMAs of the steps before (the scheduling barriers keep the
        // compiler from moving each read next to its MFMA)
#pragma unroll
        for (int j = 0; j < kOperandLead; ++j) load_step(j);
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            if (j + kOperandLead < NJ) load_step(j + kOperandLead);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int u = 0; u < TM; ++u)
#pragma unroll
                for (int v = 0; v < RN; ++v) acc[u][v] = mfma32x32x16(xa[j][u], wb[j][v], acc[u][v]);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    // C[token][row]: register i of lane l is token c_row(i, l), row l % 32
#pragma unroll
    for (int u = 0; u < TM; ++u)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int64_t t = t0 + 32 * TM * wt + 32 * u + c_row(i, lane);
            if (t >= a.T) continue;
            bf16* yr = ysel + (size_t(t) * a.G + g) * a.R + r0 + 32 * RN * wr + m;
#pragma unroll
            for (int v = 0; v < RN; ++v) yr[32 * v] = from_f32<bf16>(acc[u][v][i]);
        }
}

template <typename T>
struct GenericArgs {
    int G, K, R;
    const T* x;
    const T* w;
    T* y;
    int64_t T_;
};

template <typename T>
__global__ void __launch_bounds__(256) gproj_generic_kernel(GenericArgs<T> a) {
    const int64_t o = int64_t(blockIdx.x) * 256 + threadIdx.x;    // (t, g, r), r fastest
    const int64_t n = a.T_ * a.G * a.R;
    if (o >= n) return;
    const int r = int(o % a.R);
    const int g = int((o / a.R) % a.G);
    const int64_t t = o / (int64_t(a.R) * a.G);
    const T* xr = a.x + (size_t(t) * a.G + g) * a.K;
    const T* wr = a.w + (size_t(g) * a.R + r) * a.K;
    float s = 0.f;
    for (int k = 0; k < a.K; ++k) s = fmaf(to_f32(xr[k]), to_f32(wr[k]), s);
    a.y[o] = from_f32<T>(s);
}

template <typename T>
hipError_t rope_run(const RopeJob& j, hipStream_t st) {
    const int HC = (j.H + kRopeHeadsPerThread - 1) / kRopeHeadsPerThread;
    const unsigned gx = unsigned((HC * (j.rd / 2) + 255) / 256);
    for (int b0 = 0; b0 < j.batch; b0 += kSeqSlice) {
        const int nb = std::min(kSeqSlice, j.batch - b0);
        SeqInts pos{};
        for (int i = 0; i < nb; ++i) pos.v[i] = int32_t(j.pos0[b0 + i]);
        RopeArgs<T> a;
        a.H = j.H; a.D = j.D; a.rd = j.rd; a.inverse = j.inverse;
        a.x = static_cast<T*>(j.x) + size_t(b0) * j.S * j.H * j.D;
        a.inv_freq = j.inv_freq;
        a.S = j.S;
        DSV4_LAUNCH("rope", rope_kernel<T>, dim3(gx, unsigned(j.S), nb), dim3(256), 0, st, a, pos);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace

hipError_t launch_rope(const RopeJob& j, hipStream_t s) {
    if (j.rd == 0) return hipSuccess;
    return j.bf16 ? rope_run<bf16>(j, s) : rope_run<float>(j, s);
}

namespace {

// 256 x 256 tiles: 8 waves of 64 tokens x 128 rows
constexpr int kBigWT = 4, kBigWR = 2, kBigTM = 2, kBigRN = 4;

template <int WT, int WR, int TM, int RN, int ST, int KD>
hipError_t launch_tile_shape(const GprojArgs& a, int gz, hipStream_t s) {
    using SH = TileShape<WT, WR, TM, RN, ST, KD>;
    const dim3 grid(unsigned((a.T + SH::T - 1) / SH::T), unsigned(a.R / SH::R), unsigned(gz));
    DSV4_LAUNCH("gproj_tile", (gproj_tile_kernel<WT, WR, TM, RN, ST, KD>), grid, dim3(64 * SH::waves), 0, s, a);
    return hipGetLastError();
}

// The tiled product over gz grid layers (groups, or the two products of a pair): 256 x 256
// tiles (two k blocks of 64 in LDS, 2 x 64 KB) where that gives about a workgroup per CU or
// more; else 128 x 128 tiles of 4 waves (64 x 64 each), one workgroup per CU, with k blocks
// of 128 (two in LDS) when K allows, else a ring of four blocks of 64 -- both keep 64-96 KB
// of copies in flight
hipError_t launch_tiled(const GprojArgs& a, int gz, hipStream_t s) {
    const int64_t big_tiles = (a.T + 255) / 256 * (a.R / 256) * gz;
    if (a.R % 256 == 0 && big_tiles >= 256) return launch_tile_shape<kBigWT, kBigWR, kBigTM, kBigRN, 2, 64>(a, gz, s);
    if (a.K % 128 == 0) return launch_tile_shape<2, 2, 2, 2, 2, 128>(a, gz, s);
    return launch_tile_shape<2, 2, 2, 2, 4, 64>(a, gz, s);
}

}  // namespace

hipError_t launch_grouped_proj(const GprojJob& j, hipStream_t s) {
    constexpr int kSmallK = 64 * kSmallWaves;          // k per KBW step of the workgroup
    if (j.w2 != nullptr) {
        // two products over one x: one launch of the tiled kernel (twice the workgroups, so
        // shapes that leave half the chip idle alone fill it), else one call each
        const bool tiled = j.bf16 && j.G == 1 && j.T > kSmallMaxT && j.K % kTileK == 0 && j.R % 128 == 0;
        if (!tiled) {
            GprojJob one = j;
            one.w2 = nullptr;
            one.y2 = nullptr;
            hipError_t e = launch_grouped_proj(one, s);
            if (e != hipSuccess) return e;
            one.w = j.w2;
            one.y = j.y2;
            return launch_grouped_proj(one, s);
        }
        GprojArgs a{1, j.K, j.R, static_cast<const bf16*>(j.x), static_cast<const bf16*>(j.w),
                    static_cast<bf16*>(j.y), j.T, static_cast<const bf16*>(j.w2), static_cast<bf16*>(j.y2)};
        return launch_tiled(a, 2, s);
    }
    if (j.bf16 && j.T <= kSmallMaxT && j.K % kSmallK == 0 && j.K <= 8 * kSmallK && j.R % 32 == 0) {
        GprojArgs a{j.G, j.K, j.R, static_cast<const bf16*>(j.x), static_cast<const bf16*>(j.w),
                    static_cast<bf16*>(j.y), j.T, nullptr, nullptr};
        const dim3 grid(unsigned(j.R / 32), unsigned(j.G));
        const dim3 block(64 * kSmallWaves);
        switch (j.K / kSmallK) {
            case 1: DSV4_LAUNCH("gproj_small", gproj_small_kernel<1>, grid, block, 0, s, a); break;
            case 2: DSV4_LAUNCH("gproj_small", gproj_small_kernel<2>, grid, block, 0, s, a); break;
            case 3: DSV4_LAUNCH("gproj_small", gproj_small_kernel<3>, grid, block, 0, s, a); break;
            case 4: DSV4_LAUNCH("gproj_small", gproj_small_kernel<4>, grid, block, 0, s, a); break;
            case 5: DSV4_LAUNCH("gproj_small", gproj_small_kernel<5>, grid, block, 0, s, a); break;
            case 6: DSV4_LAUNCH("gproj_small", gproj_small_kernel<6>, grid, block, 0, s, a); break;
            case 7: DSV4_LAUNCH("gproj_small", gproj_small_kernel<7>, grid, block, 0, s, a); break;
            default: DSV4_LAUNCH("gproj_small", gproj_small_kernel<8>, grid, block, 0, s, a); break;
        }
        return hipGetLastError();
    }
    if (j.bf16 && j.K % kTileK == 0 && j.R % 128 == 0) {
        GprojArgs a{j.G, j.K, j.R, static_cast<const bf16*>(j.x), static_cast<const bf16*>(j.w),
                    static_cast<bf16*>(j.y), j.T, nullptr, nullptr};
        return launch_tiled(a, j.G, s);
    }
    const int64_t n = j.T * j.G * j.R;
    const unsigned blocks = unsigned((n + 255) / 256);
    if (j.bf16) {
        GenericArgs<bf16> a{j.G, j.K, j.R, static_cast<const bf16*>(j.x), static_cast<const bf16*>(j.w),
                            static_cast<bf16*>(j.y), j.T};
        DSV4_LAUNCH("gproj_generic", gproj_generic_kernel<bf16>, dim3(blocks), dim3(256), 0, s, a);
    } else {
        GenericArgs<float> a{j.G, j.K, j.R, static_cast<const float*>(j.x), static_cast<const float*>(j.w),
                             static_cast<float*>(j.y), j.T};
        DSV4_LAUNCH("gproj_generic", gproj_generic_kernel<float>, dim3(blocks), dim3(256), 0, s, a);
    }
    return hipGetLastError();
}

}  // namespace dsv4
