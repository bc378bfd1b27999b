// Shared device/host helpers for the CSA kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>

#include <cstdint>
#include <string>

namespace dsv4 {

// ------------------------------------------------------------------ storage types
// bf16 is carried as its raw 16-bit pattern; arithmetic is always fp32.
struct bf16 {
    uint16_t x;
};

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16 v) { return __uint_as_float(uint32_t(v.x) << 16); }

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
// Round to nearest, ties to even (inputs are finite; NaN maps to a quiet NaN).
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float v) {
    uint32_t u = __float_as_uint(v);
    if ((u & 0x7fffffffu) > 0x7f800000u) return bf16{uint16_t(0x7fc0)};
    u += 0x7fffu + ((u >> 16) & 1u);
    return bf16{uint16_t(u >> 16)};
}
// Value after a round trip through the storage type.
template <typename T> __device__ __forceinline__ float round_to(float v) {
    return to_f32(from_f32<T>(v));
}

// Order-preserving map of an fp32 score to a u32 key (larger score -> larger key).
// -0.0 is folded onto +0.0 so the two compare equal.
__device__ __forceinline__ uint32_t score_key(float s) {
    uint32_t u = __float_as_uint(s == 0.0f ? 0.0f : s);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ------------------------------------------------------------------ per-sequence host ints
// Host-side per-sequence integers travel as kernel arguments, one launch per slice of at
// most kSeqSlice sequences, so no device buffer is needed for them.
constexpr int kSeqSlice = 128;
struct SeqInts {
    int32_t v[kSeqSlice];
};

// ------------------------------------------------------------------ reductions
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}
// A lane's value combined with that of lane ^ 16 (lane ^ 32) through the VALU, no LDS:
// v_permlane16_swap (v_permlane32_swap) applied to one register twice leaves the two values of
// each lane pair in its two results; for max and sum their order does not matter, and every
// lane of a pair combines them in the same order.
__device__ __forceinline__ float max_xor16(float v) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor16(float v) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor32(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Max and sum over the 64 lanes through the VALU: DPP steps within each row of 16 lanes
// (quad swaps, then rotations by 4 and 8), then the rows combined by the swaps above.  The
// sum's association differs between lanes (the last bit may too): take one lane's value
// where every lane must agree.
__device__ __forceinline__ float wave_max_valu(float v) {
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xb1, 0xf, 0xf, false)));    // quad_perm [1,0,3,2]
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4e, 0xf, 0xf, false)));    // quad_perm [2,3,0,1]
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x124, 0xf, 0xf, false)));   // row_ror:4
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x128, 0xf, 0xf, false)));   // row_ror:8
    return max_xor32(max_xor16(v));
}
__device__ __forceinline__ float wave_sum_valu(float v) {
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xb1, 0xf, 0xf, false));
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4e, 0xf, 0xf, false));
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x124, 0xf, 0xf, false));
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x128, 0xf, 0xf, false));
    return sum_xor32(sum_xor16(v));
}

// Block-wide reductions for blockDim.x a multiple of 64, up to 1024; `red` holds 16 floats.
__device__ __forceinline__ float block_sum(float v, float* red) {
    v = wave_sum(v);
    const int w = threadIdx.x >> 6, nw = blockDim.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[w] = v;
    __syncthreads();
    float t = 0.f;
    for (int i = 0; i < nw; ++i) t += red[i];
    return t;
}
__device__ __forceinline__ float block_max(float v, float* red) {
    v = wave_max(v);
    const int w = threadIdx.x >> 6, nw = blockDim.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[w] = v;
    __syncthreads();
    float t = -INFINITY;
    for (int i = 0; i < nw; ++i) t = fmaxf(t, red[i]);
    return t;
}

// ------------------------------------------------------------------ launch bookkeeping
// Kernel trace: while it is on, trace_events hands out a start/stop event pair for the next
// launch of `name` and returns true.  DSV4_LAUNCH attaches the pair to the dispatch itself
// (hipExtLaunchKernelGGL), so the recorded time is the kernel's own duration, without the
// queue gaps that events recorded around the launch would add.
bool trace_events(const char* name, hipEvent_t* start, hipEvent_t* stop);

#define DSV4_LAUNCH(name, kernel, grid, block, shmem, stream, ...)                              \
    do {                                                                                         \
        hipEvent_t ev0_, ev1_;                                                                   \
        if (::dsv4::trace_events(name, &ev0_, &ev1_))                                           \
            hipExtLaunchKernelGGL(kernel, grid, block, shmem, stream, ev0_, ev1_, 0, __VA_ARGS__); \
        else                                                                                     \
            hipLaunchKernelGGL(kernel, grid, block, shmem, stream, __VA_ARGS__);                 \
    } while (0)

}  // namespace dsv4
