// Host-side launchers of the layer's neighbours on either side of the attention: RoPE of the
// per-head inputs and of the attention output, and the grouped output projection.  Arguments
// reaching these have been validated by the C ABI layer (api.cpp).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace dsv4 {

struct RopeJob {
    int H, D, rd;              // heads, head width, rotary dims (the last rd of each head)
    bool inverse;              // turn each pair back by its angle
    bool bf16;
    void* x;                   // [B][S][H][D], rotated in place
    const float* inv_freq;     // [rd/2]
    int64_t S;
    int batch;
    const int64_t* pos0;       // host [B]: position of token 0 of each sequence
};
hipError_t launch_rope(const RopeJob& j, hipStream_t s);

struct GprojJob {
    int G, K, R;               // groups, inputs per group, outputs per group
    bool bf16;
    const void* x;             // [T][G][K]
    const void* w;             // [G][R][K]
    void* y;                   // [T][G][R]
    int64_t T;
    // optional second (weight, output) pair over the same x (G = 1): y2 = x w2^T, launched
    // together with the first where the tiled kernel applies
    const void* w2 = nullptr;
    void* y2 = nullptr;
};
hipError_t launch_grouped_proj(const GprojJob& j, hipStream_t s);

}  // namespace dsv4
