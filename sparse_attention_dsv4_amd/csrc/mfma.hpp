// bf16 MFMA helpers for gfx950 (CDNA4), wave64.
//
// v_mfma_f32_32x32x16_bf16 lane layout (checked on the hardware):
//   A (32 x 16): lane l holds A[l % 32][8 * (l / 32) + 0..7]
//   B (16 x 32): lane l holds B[8 * (l / 32) + 0..7][l % 32]
//   C (32 x 32): lane l, register i holds C[8 * (i / 4) + 4 * (l / 32) + i % 4][l % 32]
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace dsv4 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx2 __attribute__((ext_vector_type(2)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ floatx16 mfma32x32x16(const bf16x8& a, const bf16x8& b, const floatx16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Row of C held by register i of lane l (see the layout above).
__device__ __forceinline__ int c_row(int i, int lane) { return 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3); }

__device__ __forceinline__ bf16x8 load_bf16x8(const void* p) {
    const uint4 v = *reinterpret_cast<const uint4*>(p);
    bf16x8 r;
    __builtin_memcpy(&r, &v, 16);
    return r;
}

__device__ __forceinline__ void store16(void* p, const uint4& v) { *reinterpret_cast<uint4*>(p) = v; }

// Two floats to bf16 (round to nearest even) in one v_cvt_pk_bf16_f32; a in the low half.
__device__ __forceinline__ uint32_t pack2_bf16(float a, float b) {
    const floatx2 v = {a, b};
    const bf16x2 r = __builtin_convertvector(v, bf16x2);
    uint32_t u;
    __builtin_memcpy(&u, &r, 4);
    return u;
}

__device__ __forceinline__ uint16_t bf16_bits(float v) {
    uint32_t u = __float_as_uint(v);
    u += 0x7fffu + ((u >> 16) & 1u);
    return uint16_t(u >> 16);
}

}  // namespace dsv4
