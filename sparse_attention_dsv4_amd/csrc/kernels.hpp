// Host-side launchers of the CSA kernels.  Arguments reaching these have been validated by
// the C ABI layer (api.cpp); the launchers only split the batch and enqueue kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace dsv4 {

// Frontier state of one compressor lane for one sequence: [lane (kv, gate)][nw][r][coff*D]
// elements (nw windows: the coff pooled ones plus those retained for rollback).  Token t
// sits in window slot (t / r) % nw at position t % r; this is the element offset of its
// kv-lane entry (the gate lane's is nw * r * coff*D further).
__host__ __device__ inline size_t frontier_slot(int64_t t, int r, int nw, int W) {
    return (size_t((t / r) % nw) * size_t(r) + size_t(t % r)) * size_t(W);
}

// One lane's frontier store of a decode step (the token's kv and gate lanes into its slot).
struct FrontierJob {
    void* state;               // [B][2][nw][r][coff*D]
    const void* lane_a;        // [B][coff*D]
    const void* lane_g;
    int r, nw, W;              // W = coff*D
};
hipError_t launch_frontier_store(const FrontierJob& f, bool bf16, int batch, const int64_t* pos,
                                 hipStream_t s);

struct CompressJob {
    int r, coff, nw, D, rd;
    float eps;
    bool bf16;
    void* state;               // [B][2][nw][r][coff*D]
    const void* lane_a;        // [B][n_new][coff*D]
    const void* lane_g;
    const void* ape;           // [r][coff*D]
    const void* gamma;         // [D]
    const float* inv_freq;     // [rd/2]
    void* rows;                // [B][row_cap][D]
    int64_t row_cap;
    int64_t n_new;
    int batch;
    const int64_t* len_before; // host [B]
};
hipError_t launch_compress(const CompressJob& j, hipStream_t s);

struct IndexJob {
    int Hi, di, k, r;
    bool bf16;
    const void* qi;            // [B][S][Hi][di]
    const float* w;            // [B][S][Hi]
    const void* rows;          // [B][row_cap][di]
    int64_t row_cap;
    int64_t S;
    int64_t n_stride;          // row stride of the score workspace (>= max n_rows)
    int64_t n_max;             // max n_rows, as given to index_workspace_bytes
    int batch;
    const int64_t* n_rows;     // host [B]
    const int64_t* pos0;       // host [B]
    int32_t* sel;              // [B][S][k]
    uint32_t* keys;            // workspace: keys [B][S][n_stride], then candidate lists
};
hipError_t launch_index_topk(const IndexJob& j, hipStream_t s);
size_t index_workspace_bytes(int Hi, int di, int k, int batch, int64_t S, int64_t n_max);
// Row stride (in keys) of the score-key workspace: a multiple of 4, so rows are 16-byte aligned.
int64_t index_key_stride(int64_t n_max);

struct AttnJob {
    int H, D, W, r, k;
    int Wr;                    // ring slots: W + the tokens retained for rollback
    float scale;
    bool bf16;
    const void* q;             // [B][S][H][D]
    const void* kv_new;        // [B][S][D]
    void* ring;                // [B][Wr][D]
    const void* rows;          // [B][row_cap][D] or null
    int64_t row_cap;
    const int32_t* sel;        // [B][S][k] or null
    const float* sinks;        // [H]
    void* out;                 // [B][S][H][D]
    int64_t S;
    int batch;
    const int64_t* n_rows;     // host [B] or null
    const int64_t* pos0;       // host [B]
    void* ws;
    size_t ws_bytes;
    int n_fronts = 0;          // decode only: frontier stores folded into the launch
    FrontierJob fronts[2];
};
hipError_t launch_attention(const AttnJob& j, hipStream_t s);
size_t attn_workspace_bytes(bool bf16, int H, int D, int W, int r, int k, int batch, int64_t S);
// Largest key count (window + rows) one query may have for the attention kernels (0 when
// the configuration is not supported at all).
int64_t attn_max_keys(bool bf16, int H, int D, int k, bool has_sel);

}  // namespace dsv4
