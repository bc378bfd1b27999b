// Gated-pooling compressor (one lane): rows for completed windows + frontier state update.
//
// Pages: MTPLX PR #216 "What V4 adds" (rows pooled with learned gates over windows of 4
// that overlap or of 128 that do not; the lanes grow token by token in prefill and decode);
// mlx-lm PR #1189 Thump604's fix list (ratio-4 lanes are 2*D wide), aidiffuser's indexer
// path (each overlapping row also pools the window before its own; the tail and previous window
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
//                         channel with a softmax, then norm and RoPE in LDS;
//   compress_state_kernel copies the new tokens of the last nw windows into the state.
// The second runs after the first on the stream, because a row of this call may read a
// state slot that the update overwrites.  With one new token per sequence (decode): the
// frontier store alone, or, when a sequence completes a row, the row kernel with the store
// folded in (ratio 4: a row's few slots need no more than one workgroup), or for longer rows
// compress_pool_kernel (the store and the pooling, spread over channel blocks) then
// compress_finish_kernel (norm and RoPE).
#include "common.hpp"
#include "kernels.hpp"

namespace dsv4 {

namespace {

constexpr int kCompThreads = 256;     // an emitting workgroup (prefill row or decode finish)
constexpr int kMaxDim = 4096;         // largest latent (the configs' dim bound)
constexpr int kPairs = 1024;          // (channel group, slot group) pairs of a row

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
    int store_new;             // decode (n_new = 1): the row's workgroup also stores the token
};

// VEC consecutive storage elements (16 bytes, aligned; VEC = 1: one element anywhere): a raw
// load, and element e of it as a float.
template <typename T, int VEC>
struct RawVec {
    uint4 u;
    __device__ __forceinline__ void load(const T* p) { u = *reinterpret_cast<const uint4*>(p); }
    __device__ __forceinline__ float get(int e) const {
        if constexpr (sizeof(T) == 2) {
            const uint32_t x = (e >> 1) == 0 ? u.x : (e >> 1) == 1 ? u.y : (e >> 1) == 2 ? u.z : u.w;
            return __uint_as_float((e & 1) ? (x & 0xffff0000u) : (x << 16));
        } else {
            const uint32_t x = e == 0 ? u.x : e == 1 ? u.y : e == 2 ? u.z : u.w;
            return __uint_as_float(x);
        }
    }
};
template <typename T>
struct RawVec<T, 1> {
    T v;
    __device__ __forceinline__ void load(const T* p) { v = *p; }
    __device__ __forceinline__ float get(int) const { return to_f32(v); }
};

// Pooling of one row.  The coff*r slots of a channel are split over SG slot groups (slot
// group g: slots g, g + SG, ...); each (channel group of VEC channels, slot group) keeps a
// softmax state (max, sum, weighted sum) in base-2 units (logits times log2 e), updated a
// batch of UNR slots at a time: the batch's own max, its exponentials, then one rescale --
// about 1.25 exponentials per slot, each a bare exp2.  The groups' states then merge per
// channel in the fixed order g = 0 .. SG-1.  Prefill rows and decode emissions run this same
// arithmetic per channel (whichever workgroup computes it), so their rows are bit-identical.
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kUnr = 8;

// Channel groups (VEC channels) and slot groups of a row of D channels and nslots slots:
// about kPairs pairs in all, at most 256 slot groups and no more than a batch of kUnr slots
// per group needs (a ratio-4 row's 8 slots: one group) -- a function of the lane shape
// alone, so every kernel that pools a row splits it the same way.
__host__ __device__ inline void slot_groups(int D, int vec, int nslots, int& ncg, int& SG) {
    ncg = D / vec;
    SG = kPairs / ncg;
    SG = SG < 1 ? 1 : (SG > 256 ? 256 : SG);
    const int need = (nslots + kUnr - 1) / kUnr;
    SG = SG < need ? SG : (need < 1 ? 1 : need);
}

template <typename T, int VEC>
__device__ __forceinline__ void pool_part(const CompArgs<T>& a, int b, int j, int lb, int cg, int g,
                                          int SG, float (&m)[VEC], float (&l)[VEC], float (&acc)[VEC]) {
    const int D = a.D, W = a.coff * a.D, r = a.r;
    const size_t st = size_t(2) * a.nw * r * W;
    const T* sa0 = a.state + size_t(b) * st;                 // kv lane of this sequence
    const T* sg0 = sa0 + size_t(a.nw) * r * W;               // gate lane
    const int nslots = a.coff * r;
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
        m[e] = -INFINITY;
        l[e] = 0.f;
        acc[e] = 0.f;
    }
    // slot u = g + SG i is position sl of half `half` (u = half r + sl), advanced without
    // division; the frontier window of each half is fixed for the row
    const int wmod1 = j % a.nw;                                  // window j
    const int wmod0 = j >= 1 ? (j - 1) % a.nw : 0;               // window j - 1 (overlap)
    const int dh = SG / r, ds = SG - dh * r;
    int half = g / r, sl = g - (g / r) * r;
    for (int u0 = g; u0 < nslots; u0 += SG * kUnr) {
        RawVec<T, VEC> v[kUnr], gt[kUnr], ap[kUnr];
        bool ok[kUnr];
#pragma unroll
        for (int q = 0; q < kUnr; ++q) {
            const int u = u0 + q * SG;
            // overlap: half 0 <- window j-1, half 1 <- window j; plain: half 0 <- window j
            const bool prev = a.coff == 2 && half == 0;
            const int win = prev ? j - 1 : j;
            ok[q] = u < nslots && win >= 0;
            // every slot's loads go out unconditionally, their sources chosen by selects (loads
            // under per-lane branches were each waited for before the next slot's went out); a
            // slot that does not exist reads in bounds (channel group cg of the state's first
            // slot and of the first APE row) and is masked below
            const int col = ok[q] ? half * D + cg * VEC : cg * VEC;
            const int t = win * r + sl;
            const bool in_state = !ok[q] || t < lb;
            const size_t os = ok[q] ? (size_t(prev ? wmod0 : wmod1) * r + size_t(sl)) * W + col : size_t(col);
            const size_t ol = (size_t(b) * a.n_new + size_t(in_state ? 0 : t - lb)) * W + col;
            v[q].load(in_state ? sa0 + os : a.lane_a + ol);
            gt[q].load(in_state ? sg0 + os : a.lane_g + ol);
            ap[q].load(a.ape + size_t(ok[q] ? sl : 0) * W + col);
            sl += ds;
            half += dh;
            if (sl >= r) {
                sl -= r;
                ++half;
            }
        }
        bool any = false;
#pragma unroll
        for (int q = 0; q < kUnr; ++q) any |= ok[q];
        if (!any) continue;
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            float c[kUnr];
            float mb = -INFINITY;
#pragma unroll
            for (int q = 0; q < kUnr; ++q) {
                c[q] = (gt[q].get(e) + ap[q].get(e)) * kLog2e;
                if (ok[q]) mb = fmaxf(mb, c[q]);
            }
            float lb_ = 0.f, ab = 0.f;
#pragma unroll
            for (int q = 0; q < kUnr; ++q)
                if (ok[q]) {
                    const float x = __builtin_amdgcn_exp2f(c[q] - mb);
                    lb_ += x;
                    ab = fmaf(x, v[q].get(e), ab);
                }
            const float M = fmaxf(m[e], mb);
            const float f = m[e] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m[e] - M);
            const float fb = __builtin_amdgcn_exp2f(mb - M);
            l[e] = fmaf(l[e], f, lb_ * fb);
            acc[e] = fmaf(acc[e], f, ab * fb);
            m[e] = M;
        }
    }
}

// Merge of the slot groups' states of channel c (part: [3][SG][D]): the pooled value.
__device__ __forceinline__ float merge_part(const float* part, int SG, int D, int c) {
    float mx = -INFINITY;
    for (int i = 0; i < SG; ++i) mx = fmaxf(mx, part[(0 * SG + i) * D + c]);
    float ls = 0.f, as = 0.f;
    for (int i = 0; i < SG; ++i) {
        const float mi = part[(0 * SG + i) * D + c];
        const float f = mi == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mi - mx);
        ls = fmaf(part[(1 * SG + i) * D + c], f, ls);
        as = fmaf(part[(2 * SG + i) * D + c], f, as);
    }
    return as / ls;
}

// Per-thread constants of the row epilogue for channels tid + k*NT: gamma (raw, converted
// where it is used) and the RoPE frequency, loaded when the workgroup starts so their
// latency overlaps the pooling.  The loads sit under a workgroup-uniform guard and read an
// in-bounds (clamped) element in every lane: a conversion or a per-lane select inside the
// guard would make each block wait for its load before the next is issued.
constexpr int kChan = kMaxDim / kCompThreads;
template <typename T>
struct RowConst {
    T gam[kChan];
    float frq[kChan];
};
template <typename T>
__device__ __forceinline__ void load_row_const(const CompArgs<T>& a, RowConst<T>& rc) {
    const int r0 = a.D - a.rd;
#pragma unroll
    for (int k = 0; k < kChan; ++k) {
        if (k * kCompThreads >= a.D) break;
        int c = int(threadIdx.x) + k * kCompThreads;
        c = c < a.D ? c : a.D - 1;
        rc.gam[k] = a.gamma[c];
        rc.frq[k] = a.rd > 0 ? a.inv_freq[c >= r0 ? (c - r0) >> 1 : 0] : 0.f;
    }
}

// The rest of row j once its pooled (rounded) values are in zrow and each thread's sum of
// squares (channels tid, tid + NT, ...) in ss: RMSNorm * gamma (rounded), RoPE of the last rd
// dims at position j*r (rounded), stored.
template <typename T>
__device__ __forceinline__ void finish_row(const CompArgs<T>& a, const RowConst<T>& rc, int b, int j, float ss,
                                           float* zrow, float* red) {
    constexpr int NT = kCompThreads;
    const int D = a.D, tid = threadIdx.x;
    const float tot = block_sum(ss, red);
    const float den = sqrtf(tot / float(D) + a.eps);
#pragma unroll
    for (int k = 0; k < kChan; ++k) {
        const int c = tid + k * NT;
        if (c < D) zrow[c] = round_to<T>(zrow[c] / den * to_f32(rc.gam[k]));
    }
    __syncthreads();
    const int r0 = D - a.rd;
    const float pos = float(int64_t(j) * a.r);
    T* out = a.rows + (size_t(b) * a.row_cap + size_t(j)) * D;
#pragma unroll
    for (int k = 0; k < kChan; ++k) {
        const int c = tid + k * NT;
        if (c >= D) break;
        float v = zrow[c];
        if (c >= r0) {
            const int i = (c - r0) >> 1;
            const float x0 = zrow[r0 + 2 * i], x1 = zrow[r0 + 2 * i + 1];
            float sn, cs;
            sincosf(pos * rc.frq[k], &sn, &cs);
            v = ((c - r0) & 1) ? (x0 * sn + x1 * cs) : (x0 * cs - x1 * sn);
        }
        out[c] = from_f32<T>(v);
    }
}

// Row j of sequence b by one workgroup (prefill): pooled per channel (pool_part for every
// (channel group, slot group) pair, merge_part), rounded, then finish_row.  Slot s of window
// w is token w*r + s: tokens before the call (t < lb) sit in state window (w % nw) at
// position s, later ones in the new lanes at t - lb.
template <typename T, int VEC>
__device__ __forceinline__ void emit_row(const CompArgs<T>& a, int b, int j, int lb,
                                         float* zrow, float* part, float* red) {
    constexpr int NT = kCompThreads;
    const int D = a.D, tid = threadIdx.x;
    RowConst<T> rc;
    load_row_const(a, rc);
    int ncg, SG;
    slot_groups(D, VEC, a.coff * a.r, ncg, SG);
    for (int pr = tid; pr < ncg * SG; pr += NT) {
        const int cg = pr % ncg, g = pr / ncg;
        float m[VEC], l[VEC], acc[VEC];
        pool_part<T, VEC>(a, b, j, lb, cg, g, SG, m, l, acc);
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            const int c = cg * VEC + e;
            part[(0 * SG + g) * D + c] = m[e];
            part[(1 * SG + g) * D + c] = l[e];
            part[(2 * SG + g) * D + c] = acc[e];
        }
    }
    __syncthreads();
    float ss = 0.f;
    for (int c = tid; c < D; c += NT) {
        const float y = round_to<T>(merge_part(part, SG, D, c));
        zrow[c] = y;
        ss += y * y;
    }
    finish_row<T>(a, rc, b, j, ss, zrow, red);
}

// A token's kv and gate lanes (W values each) copied into its frontier slot by threads
// i0, i0 + step, ...: four values of each lane per thread are loaded before any is stored,
// so up to 4 * step values cost one round trip (the stores may alias the loads as far as the
// compiler knows, so a load placed after a store waits for it).
template <typename T>
__device__ __forceinline__ void copy_token_lanes(T* sa, T* sg, const T* la, const T* lg, int W, int i0, int step) {
    for (int c0 = i0; c0 < W; c0 += 4 * step) {
        T va[4], vg[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int c = c0 + k * step;
            if (c < W) {
                va[k] = la[c];
                vg[k] = lg[c];
            }
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int c = c0 + k * step;
            if (c < W) {
                sa[c] = va[k];
                sg[c] = vg[k];
            }
        }
    }
}

// A token's two lanes between an early load and a late store into its frontier slot, so the
// load's round trip overlaps the workgroup's other work: up to 4 values of each lane per
// thread in registers (wider lanes are copied at once by copy_token_lanes).
template <typename T>
struct HeldLanes {
    T va[4], vg[4];
    T* sa = nullptr;
    T* sg = nullptr;
    int W = 0, i0 = 0, step = 0;
    bool held = false;
    __device__ void begin(T* sa_, T* sg_, const T* la, const T* lg, int W_, int i0_, int step_) {
        sa = sa_;
        sg = sg_;
        W = W_;
        i0 = i0_;
        step = step_;
        held = W <= 4 * step;
        if (!held) {
            copy_token_lanes(sa, sg, la, lg, W, i0, step);
            return;
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int c = i0 + k * step;
            if (c < W) {
                va[k] = la[c];
                vg[k] = lg[c];
            }
        }
    }
    __device__ void finish() const {
        if (!held) return;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int c = i0 + k * step;
            if (c < W) {
                sa[c] = va[k];
                sg[c] = vg[k];
            }
        }
    }
};

template <typename T, int VEC>
__global__ void __launch_bounds__(kCompThreads)
compress_rows_kernel(CompArgs<T> a, SeqInts len_before) {
    extern __shared__ float smem[];                  // zrow [D], then part [3][SG][D]
    __shared__ float red[16];
    float* zrow = smem;
    float* part = smem + a.D;
    const int b = blockIdx.y;
    const int lb = len_before.v[b];
    // the token's frontier slot (decode): the row reads the state only at earlier tokens and
    // takes this one from the lane, so the store cannot race it; stored after the row
    HeldLanes<T> tok;
    if (a.store_new && blockIdx.x == 0) {
        const int W = a.coff * a.D;
        T* sa = a.state + size_t(b) * (size_t(2) * a.nw * a.r * W) + frontier_slot(lb, a.r, a.nw, W);
        tok.begin(sa, sa + size_t(a.nw) * a.r * W, a.lane_a + size_t(b) * W, a.lane_g + size_t(b) * W, W,
                  int(threadIdx.x), kCompThreads);
    }
    const int j = lb / a.r + int(blockIdx.x);  // row index
    if (int64_t(j + 1) * a.r > lb + a.n_new) {
        tok.finish();
        return;
    }
    emit_row<T, VEC>(a, b, j, lb, zrow, part, red);
    tok.finish();
}

// A decode step in two launches when some sequence completes a row.  compress_pool_kernel:
// one workgroup per (block of channel groups, sequence) pools its channels exactly as
// emit_row does and stores the rounded pooled values in the row's place; the workgroups of a
// sequence also store the token in the frontier (the row reads the state only at earlier
// tokens and takes this token from the lane, so the store cannot race it).
// compress_finish_kernel: one workgroup per emitting sequence reads the pooled row back and
// finishes it (finish_row, the same channel-to-thread mapping as emit_row).
template <typename T, int VEC>
__global__ void __launch_bounds__(256)
compress_pool_kernel(CompArgs<T> a, SeqInts len_before) {
    extern __shared__ float part[];           // [3][SG][CGW * VEC]
    const int b = blockIdx.y;
    const int lb = len_before.v[b];
    const int W = a.coff * a.D;
    // the token's frontier slot, spread over the sequence's workgroups; stored after the pooling
    HeldLanes<T> tok;
    {
        T* sa = a.state + size_t(b) * (size_t(2) * a.nw * a.r * W) + frontier_slot(lb, a.r, a.nw, W);
        tok.begin(sa, sa + size_t(a.nw) * a.r * W, a.lane_a + size_t(b) * W, a.lane_g + size_t(b) * W, W,
                  int(blockIdx.x * blockDim.x + threadIdx.x), int(gridDim.x * blockDim.x));
    }
    if ((lb + 1) % a.r != 0) {
        tok.finish();
        return;
    }
    const int j = lb / a.r;
    int ncg, SG;
    slot_groups(a.D, VEC, a.coff * a.r, ncg, SG);
    const int CGW = int(blockDim.x) / SG;                 // channel groups per workgroup
    const int cl = threadIdx.x % CGW, g = threadIdx.x / CGW;
    const int cg = int(blockIdx.x) * CGW + cl;
    const int CW = CGW * VEC;                             // channels of this workgroup
    if (cg < ncg) {
        float m[VEC], l[VEC], acc[VEC];
        pool_part<T, VEC>(a, b, j, lb, cg, g, SG, m, l, acc);
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            const int c = cl * VEC + e;
            part[(0 * SG + g) * CW + c] = m[e];
            part[(1 * SG + g) * CW + c] = l[e];
            part[(2 * SG + g) * CW + c] = acc[e];
        }
    }
    __syncthreads();
    T* row = a.rows + (size_t(b) * a.row_cap + size_t(j)) * a.D;
    const int c0 = int(blockIdx.x) * CW;
    for (int c = threadIdx.x; c < CW && c0 + c < a.D; c += blockDim.x)
        row[c0 + c] = from_f32<T>(merge_part(part, SG, CW, c));
    tok.finish();
}

template <typename T>
__global__ void __launch_bounds__(kCompThreads)
compress_finish_kernel(CompArgs<T> a, SeqInts len_before) {
    __shared__ float zrow[kMaxDim];
    __shared__ float red[16];
    const int b = blockIdx.x;
    const int lb = len_before.v[b];
    if ((lb + 1) % a.r != 0) return;
    const int j = lb / a.r;
    RowConst<T> rc;
    load_row_const(a, rc);
    const T* row = a.rows + (size_t(b) * a.row_cap + size_t(j)) * a.D;
    float ss = 0.f;
    for (int c = threadIdx.x; c < a.D; c += kCompThreads) {
        const float y = to_f32(row[c]);
        zrow[c] = y;
        ss += y * y;
    }
    finish_row<T>(a, rc, b, j, ss, zrow, red);
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
    copy_token_lanes(sa, sa + size_t(a.nw) * a.r * W, a.lane_a + src, a.lane_g + src, W, int(threadIdx.x),
                     int(blockDim.x));
}

// The frontier store of a decode step alone (no row completes): one workgroup per sequence.
template <typename T>
__global__ void __launch_bounds__(kCompThreads)
frontier_store_kernel(FrontierJob f, SeqInts pos) {
    const int b = blockIdx.x;
    const size_t st = size_t(2) * f.nw * f.r * f.W;
    T* sa = static_cast<T*>(f.state) + size_t(b) * st + frontier_slot(pos.v[b], f.r, f.nw, f.W);
    copy_token_lanes(sa, sa + size_t(f.nw) * f.r * f.W, static_cast<const T*>(f.lane_a) + size_t(b) * f.W,
                     static_cast<const T*>(f.lane_g) + size_t(b) * f.W, f.W, int(threadIdx.x), int(blockDim.x));
}

// Dynamic LDS beyond the default 64 KB must be allowed per kernel and device before its
// launch (once: the limit is raised to the largest size asked for so far on that device).
template <typename K>
hipError_t allow_lds(K* kernel, size_t bytes) {
    constexpr size_t kDefault = 64 * 1024;
    static size_t allowed[64];
    if (bytes <= kDefault) return hipSuccess;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    if (bytes <= allowed[dev]) return hipSuccess;
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                            int(bytes));
    if (e == hipSuccess) allowed[dev] = bytes;
    return e;
}

// 16-byte vectors of the storage type where every lane column is a multiple of them (the
// lanes and the APE are rows of coff*D elements, so D % VEC == 0 aligns every slot).
template <typename T> constexpr int kVec = 16 / int(sizeof(T));
template <typename T> bool vec_ok(int D) { return D % kVec<T> == 0; }

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
            bool emits = false;
            for (int i = 0; i < nb; ++i) emits |= (j.len_before[b0 + i] + 1) % j.r == 0;
            if (!emits) {                                   // the frontier store alone
                FrontierJob f;
                f.state = a.state; f.lane_a = a.lane_a; f.lane_g = a.lane_g;
                f.r = j.r; f.nw = j.nw; f.W = W;
                hipError_t e = launch_frontier_store(f, sizeof(T) == 2, nb, j.len_before + b0, s);
                if (e != hipSuccess) return e;
                continue;
            }
            const int vec = vec_ok<T>(j.D) ? kVec<T> : 1;
            int ncg, SG;
            slot_groups(j.D, vec, j.coff * j.r, ncg, SG);
            a.store_new = 1;
            if (ncg * SG <= kCompThreads) {
                // a row of at most one pair per thread (ratio 4): the prefill row kernel, one
                // workgroup per sequence, which also stores the token -- one launch
                const size_t lds = size_t(j.D) * (1 + 3 * SG) * sizeof(float);
                hipError_t e = vec > 1 ? allow_lds(compress_rows_kernel<T, kVec<T>>, lds)
                                       : allow_lds(compress_rows_kernel<T, 1>, lds);
                if (e != hipSuccess) return e;
                if (vec > 1)
                    DSV4_LAUNCH("compress_rows", (compress_rows_kernel<T, kVec<T>>), dim3(1, nb),
                                dim3(kCompThreads), lds, s, a, lb);
                else
                    DSV4_LAUNCH("compress_rows", (compress_rows_kernel<T, 1>), dim3(1, nb),
                                dim3(kCompThreads), lds, s, a, lb);
                e = hipGetLastError();
                if (e != hipSuccess) return e;
                continue;
            }
            // longer rows (ratio 128): the pooling spread over channel blocks, one
            // (channel group, slot group) pair per thread -- a wave of 64 / SG channel groups,
            // or SG threads for one channel group -- then the norm and RoPE
            const int CGW = SG >= 64 ? 1 : 64 / SG;
            const int nt = CGW * SG;
            const size_t lds = size_t(3) * nt * vec * sizeof(float);
            const dim3 grid(unsigned((ncg + CGW - 1) / CGW), nb);
            if (vec > 1)
                DSV4_LAUNCH("compress_pool", (compress_pool_kernel<T, kVec<T>>), grid, dim3(nt), lds, s, a, lb);
            else
                DSV4_LAUNCH("compress_pool", (compress_pool_kernel<T, 1>), grid, dim3(nt), lds, s, a, lb);
            hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
            DSV4_LAUNCH("compress_finish", compress_finish_kernel<T>, dim3(nb), dim3(kCompThreads), 0, s,
                        a, lb);
            e = hipGetLastError();
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
        a.store_new = 0;
        if (max_rows > 0) {
            // LDS: the row, then the slot groups' states (ratio-4 rows: one group, 8 KB at D = 512)
            const int vec = vec_ok<T>(j.D) ? kVec<T> : 1;
            int ncg, SG;
            slot_groups(j.D, vec, j.coff * j.r, ncg, SG);
            const size_t lds = size_t(j.D) * (1 + 3 * SG) * sizeof(float);
            hipError_t e = vec > 1 ? allow_lds(compress_rows_kernel<T, kVec<T>>, lds)
                                   : allow_lds(compress_rows_kernel<T, 1>, lds);
            if (e != hipSuccess) return e;
            if (vec > 1)
                DSV4_LAUNCH("compress_rows", (compress_rows_kernel<T, kVec<T>>), dim3(unsigned(max_rows), nb),
                            dim3(kCompThreads), lds, s, a, lb);
            else
                DSV4_LAUNCH("compress_rows", (compress_rows_kernel<T, 1>), dim3(unsigned(max_rows), nb),
                            dim3(kCompThreads), lds, s, a, lb);
            e = hipGetLastError();
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
