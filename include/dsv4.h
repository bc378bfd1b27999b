/*
 * dsv4.h - C ABI of libdsv4.so: the DeepSeek-V4-Flash compressed sparse attention (CSA)
 * layer on one AMD Instinct MI355X (gfx950).
 *
 * The layer, as the pages describe it (mlx-lm PR #1189 "feat: add DeepSeek-V4 (Pro/Flash)
 * model support" and MTPLX PR #216 "DeepSeek-V4-Flash: native deepseek_v4 AR backend"):
 *   - a learned gated-pooling compressor turns each completed window of r tokens into one
 *     compressed row (overlapping windows at ratio 4, plain windows at ratio 128), RMS-
 *     normalised and RoPE'd at the window start;
 *   - an indexer scores the compressed rows a query may see and keeps the top k;
 *   - MQA-shaped attention of H query heads over one shared latent row (key = value) per
 *     key, over a W-token sliding window plus the selected rows, with one sink logit per
 *     head that enters the softmax denominator only.
 *
 * Conventions for every call
 *   - Pointers are DEVICE pointers unless the comment says "host".  The caller allocates
 *     and owns every buffer (state, rows, ring, workspace, outputs); the library allocates
 *     no device memory in these calls and keeps no per-call state.
 *   - All tensors are dense, row-major, with the shapes given.  Storage dtype is
 *     cfg->dtype (bf16 or fp32) for every activation tensor; norm weights, APE, window
 *     ring and rows share it.  inv_freq, indexer weights w and sinks are always fp32.
 *   - Lengths and positions are HOST integers: they are deterministic (rows = tokens / r)
 *     and host-side validation needs them.  Positions are absolute, 0-based token indices.
 *   - Every call validates all arguments on the host before it launches anything; on an
 *     error it returns a negative dsv4_status, launches nothing and leaves every buffer
 *     untouched.  dsv4_last_error() then returns a message (thread-local).  Nothing is
 *     clamped: a length beyond a capacity is an error.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the legacy default stream) and is
 *     asynchronous.  A launch failure returns DSV4_EHIP.
 *   - Calls on different streams with disjoint buffers may run concurrently.
 *   - batch == 0, or zero new tokens / queries, is a valid no-op returning DSV4_OK.
 */
#ifndef DSV4_H
#define DSV4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    DSV4_OK = 0,
    DSV4_EINVAL = -1,        /* bad pointer, shape, length or position */
    DSV4_EUNSUPPORTED = -2,  /* valid but outside what the kernels implement (sizes listed per call) */
    DSV4_ECAPACITY = -3,     /* a row or token count would exceed a caller-given capacity */
    DSV4_EHIP = -4,          /* the HIP runtime reported an error */
    DSV4_EWORKSPACE = -5     /* workspace pointer NULL or smaller than the *_workspace_bytes() size */
} dsv4_status;

typedef enum { DSV4_BF16 = 0, DSV4_F32 = 1 } dsv4_dtype;

/* Compressor of one lane (the attention lane at width D, or the indexer's own lane at
 * width d_i).  Pages: PR #216 "What V4 adds" (gated pooling, overlapping ratio-4 and
 * plain ratio-128 windows); PR #1189 Thump604's fix list (ratio-4 lanes are 2*D wide:
 * ape (4, 1024), wkv/wgate (1024, 4096)); PR #1189 OmarB97 note 2 (rows RoPE'd at birth at
 * position j*r on their last rope_dim dims). */
typedef struct {
    int32_t ratio;     /* r >= 1 tokens per window                                        */
    int32_t overlap;   /* 1: row j pools window j-1 (lane half 0) and window j (half 1);
                          0: row j pools window j.  coff = overlap ? 2 : 1                  */
    int32_t dim;       /* D, row width; lanes are coff*D wide.  1 <= D <= 4096             */
    int32_t rope_dim;  /* rd, even, 0 <= rd <= D: RoPE on the last rd dims                 */
    float   eps;       /* RMSNorm epsilon (>= 0)                                           */
    int32_t dtype;     /* dsv4_dtype                                                      */
    int32_t retain;    /* tokens of rollback the frontier state keeps (0..2^20): the state
                          holds nw = coff + ceil(retain / r) windows, so a trim of up to
                          `retain` tokens back across window boundaries finds them again
                          (MTPLX PR #216 speculative-decode comment: exact trim)          */
} dsv4_comp_cfg;

/* Indexer.  Pages: PR #1189 stepnoy's patch ("Reference scoring") and aidiffuser's indexer
 * path: score(p,j) = sum_h w_h(p) * d_i^-1/2 * H_i^-1/2 * relu(qi_h(p) . K_j) in fp32,
 * over rows causally visible to p ((j+1)*r <= p+1), top k per query.  The scale is fixed
 * by (heads, dim) and is not a parameter. */
typedef struct {
    int32_t heads;     /* H_i, 1..256                                                      */
    int32_t dim;       /* d_i, 1..1024: width of qi heads and of indexer rows              */
    int32_t topk;      /* k >= 1: width of each sel row                                    */
    int32_t ratio;     /* r >= 1 of the lane the rows came from                            */
    int32_t dtype;     /* dsv4_dtype of qi and rows                                        */
} dsv4_index_cfg;

/* Attention.  Pages: PR #216 opening and "What V4 adds" (64 heads over one 512-dim latent,
 * 128-token window, per-head sinks); PR #216 "Decode dispatch reduction" (A) (sink = an
 * extra all-zero-value key column: denominator only); PR #1189 stepnoy's patch (selected
 * rows attended beside the window, causal visibility of rows). */
typedef struct {
    int32_t heads;     /* H >= 1                                                           */
    int32_t dim;       /* D: latent width (key = value), 1..4096                           */
    int32_t window;    /* W >= 1: tokens (p-W, p] are attended, self included              */
    int32_t ratio;     /* r of the compressed lane; 0 = the layer has no compressed lane   */
    int32_t topk;      /* k: width of sel rows (ignored when sel == NULL)                  */
    float   scale;     /* logit scale applied to q . x                                     */
    int32_t dtype;     /* dsv4_dtype                                                      */
    int32_t retain;    /* tokens of rollback the window ring keeps (0..2^20): the ring has
                          W + retain slots, token t in slot t % (W + retain); retention and
                          attendance are separate, only W tokens are attended (MTPLX PR
                          #216 speculative-decode comment)                                 */
} dsv4_attn_cfg;

/* Library identification and the thread-local message of the last failed call. */
const char* dsv4_version(void);
const char* dsv4_last_error(void);

/* Bytes of compressor state for `batch` sequences: per sequence, the raw kv and gate lane
 * values of the last coff windows, [2 lanes][coff][r][coff*D] of cfg->dtype.  The state
 * needs no initialisation: entries are only read once written. Returns 0 on a bad cfg. */
size_t dsv4_comp_state_bytes(const dsv4_comp_cfg* cfg, int32_t batch);

/* Workspace bytes dsv4_index_topk needs for `batch` x `s` queries over at most `n_max`
 * rows per sequence (n_max >= the largest n_rows passed).  Returns 0 on a bad cfg. */
size_t dsv4_index_workspace_bytes(const dsv4_index_cfg* cfg, int32_t batch, int64_t s,
                                  int64_t n_max);

/* Workspace bytes the attention calls need for `batch` x `s` queries (s = 1 for decode).
 * May be 0, in which case ws may be NULL. */
size_t dsv4_attn_workspace_bytes(const dsv4_attn_cfg* cfg, int32_t batch, int64_t s);

/* Compress n_new new tokens of every sequence.
 *   state      [batch] x dsv4_comp_state_bytes(cfg,1) bytes, carried between calls
 *   kv_lane    [batch, n_new, coff*D]  kv lane of tokens len_before[b] .. len_before[b]+n_new-1
 *   gate_lane  [batch, n_new, coff*D]  gate lane of the same tokens
 *   len_before host [batch]: tokens of sequence b already compressed (0 for a new one)
 *   ape        [r, coff*D]   absolute position embedding of the slot within its window
 *   norm_w     [D]           RMSNorm gain
 *   inv_freq   [rd/2] fp32   RoPE frequencies; row j turns pair i by (j*r)*inv_freq[i]
 *   rows       [batch, row_cap, D]: row j of sequence b is written for every window that
 *              completes in this call, j in [len_before/r, (len_before+n_new)/r)
 * Row j: per channel, softmax over the window slots of (gate + ape), weighted sum of the
 * kv values in fp32, rounded to the storage dtype, RMSNorm * norm_w (rounded), RoPE of the
 * last rd dims at position j*r (rounded).  Windows align to absolute positions, so any
 * chunking of a sequence gives the same rows.
 * Errors: EINVAL (NULL pointer, bad cfg, n_new < 0, len_before < 0), ECAPACITY (a row index
 * >= row_cap or a position >= 2^31 - 1), EHIP. */
int dsv4_compress_prefill(const dsv4_comp_cfg* cfg, void* state, const void* kv_lane,
                          const void* gate_lane, int32_t batch, int64_t n_new,
                          const int64_t* len_before, const void* ape, const void* norm_w,
                          const float* inv_freq, void* rows, int64_t row_cap, void* stream);

/* One decode token per sequence: dsv4_compress_prefill with n_new = 1 (same rows, bit for
 * bit).  kv_lane and gate_lane are [batch, coff*D]. */
int dsv4_compress_step(const dsv4_comp_cfg* cfg, void* state, const void* kv_lane,
                       const void* gate_lane, int32_t batch, const int64_t* len_before,
                       const void* ape, const void* norm_w, const float* inv_freq,
                       void* rows, int64_t row_cap, void* stream);

/* Indexer scoring and top-k selection for s queries per sequence at positions
 * pos0[b] .. pos0[b]+s-1.
 *   qi        [batch, s, H_i, d_i]   indexer queries (cfg->dtype)
 *   w         [batch, s, H_i] fp32   per-head weights (raw projection output)
 *   idx_rows  [batch, row_cap, d_i]  the indexer lane's rows
 *   n_rows    host [batch]: rows present; must be >= (pos0[b]+s)/r and <= row_cap
 *   pos0      host [batch]
 *   sel       [batch, s, k] int32 out: for query p, the visible rows (j < (p+1)/r) if there
 *             are at most k of them, else the k visible rows with the largest scores, ties
 *             to the lower row index; ascending, then -1 padding.  -0.0 ties +0.0.
 *   ws        workspace of at least dsv4_index_workspace_bytes(cfg, batch, s, max n_rows)
 *             bytes, 16-byte aligned (EINVAL otherwise); no initialisation needed
 * Errors: EINVAL, ECAPACITY (n_rows > row_cap), EWORKSPACE, EUNSUPPORTED (H_i or d_i out
 * of range), EHIP. */
int dsv4_index_topk(const dsv4_index_cfg* cfg, const void* qi, const float* w,
                    const void* idx_rows, int64_t row_cap, const int64_t* n_rows,
                    const int64_t* pos0, int32_t batch, int64_t s, int32_t* sel, void* ws,
                    size_t ws_bytes, void* stream);

/* dsv4_index_topk without the workspace argument, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation).  The scratch is a fixed array inside the library, one per GPU, of
 * dsv4_index_topk_noalloc_scratch_bytes() bytes (16 MiB), held by each GPU the library runs
 * on until the process ends; its address is looked up on the first call on a device.  The
 * call allocates nothing: no hipMalloc, hipFree or allocating library routine.  Same
 * arguments, results and errors as dsv4_index_topk, and EWORKSPACE, before any launch, when
 * dsv4_index_workspace_bytes() of the call exceeds the fixed size (about four million
 * (query, row) score keys: e.g. decode of 64 sequences over 65,536 rows fits, a 2048-query
 * prefill chunk over 16K rows does not).  Every call on one GPU uses that GPU's one array,
 * which keeps the last call's contents (the call writes every entry it reads): calls that
 * overlap on one GPU, on any streams, race and must not be issued. */
size_t dsv4_index_topk_noalloc_scratch_bytes(void);
int dsv4_index_topk_noalloc(const dsv4_index_cfg* cfg, const void* qi, const float* w,
                            const void* idx_rows, int64_t row_cap, const int64_t* n_rows,
                            const int64_t* pos0, int32_t batch, int64_t s, int32_t* sel,
                            void* stream);

/* Decode attention: one query per sequence at position pos[b].
 *   q        [batch, H, D]     query heads
 *   kv_new   [batch, D]        latent of token pos[b]; written into win_ring slot pos % W
 *   win_ring [batch, W+retain, D] slot t % (W+retain) holds token t for the tokens before pos[b]
 *                              (slots of tokens < 0 are never read)
 *   rows     [batch, row_cap, D] compressed rows (NULL when cfg->ratio == 0)
 *   sel      [batch, k] int32 or NULL: NULL attends every visible row (j < (pos+1)/r);
 *            otherwise the listed rows (entries outside [0, (pos+1)/r) are skipped)
 *   n_rows   host [batch] or NULL when ratio == 0: rows present (<= row_cap, and
 *            >= (pos+1)/r)
 *   sinks    [H] fp32 sink logits
 *   out      [batch, H, D]
 * out_h = sum_x e^(l_x - m) x / (e^(z_h - m) + sum_x e^(l_x - m)), l_x = scale * q_h . x,
 * m = max(z_h, max l), over x in the window and the rows.
 * Errors: EINVAL, ECAPACITY, EWORKSPACE, EUNSUPPORTED, EHIP. */
int dsv4_csa_attn_decode(const dsv4_attn_cfg* cfg, const void* q, const void* kv_new,
                         void* win_ring, const void* rows, int64_t row_cap,
                         const int32_t* sel, const int64_t* n_rows, const int64_t* pos,
                         const float* sinks, void* out, int32_t batch, void* ws,
                         size_t ws_bytes, void* stream);

/* A compressor lane's decode step folded into dsv4_csa_attn_decode_store. */
typedef struct {
    const dsv4_comp_cfg* cfg;  /* the lane's compressor (ratio and dtype as the attention's)  */
    void* state;               /* [batch] frontier states, as dsv4_compress_step              */
    const void* kv_lane;       /* [batch, coff*D] kv lane of token pos[b]                     */
    const void* gate_lane;     /* [batch, coff*D] gate lane of the same token                 */
} dsv4_frontier_store;

/* Decode attention (as dsv4_csa_attn_decode) together with the compressor steps of the same
 * token for n_stores lanes (0..2: the attention lane and the indexer lane), for a step at
 * which no sequence completes a compressed row: (pos[b] + 1) % ratio != 0 for every b.  Such
 * a step only stores the token's lanes in the frontier state (dsv4_compress_step writes no
 * row then), which nothing in the attention reads, so the stores ride in the attention
 * launch instead of one launch per lane.  The result is bit for bit that of
 * dsv4_compress_step for each lane (len_before = pos) followed by dsv4_csa_attn_decode.
 * Pages: MTPLX PR #216 "What V4 adds" (the compressor frontier carried across decode steps;
 * a row is emitted only when its window completes).
 * Errors: as dsv4_csa_attn_decode; EINVAL also for n_stores outside 0..2, a NULL store
 * pointer, a store whose cfg is invalid or whose ratio or dtype differs from cfg's, or a
 * sequence that completes a row at pos[b] (call dsv4_compress_step, then
 * dsv4_csa_attn_decode).  Nothing is launched on an error. */
int dsv4_csa_attn_decode_store(const dsv4_attn_cfg* cfg, const void* q, const void* kv_new,
                               void* win_ring, const void* rows, int64_t row_cap,
                               const int32_t* sel, const int64_t* n_rows, const int64_t* pos,
                               const float* sinks, void* out, int32_t batch, void* ws,
                               size_t ws_bytes, const dsv4_frontier_store* stores,
                               int32_t n_stores, void* stream);

/* Prefill attention for s queries per sequence at positions pos0[b] .. pos0[b]+s-1.
 *   q       [batch, s, H, D];  kv_new [batch, s, D] latents of those tokens
 *   win_ring as in decode, holding the W tokens before pos0[b]; after the call it holds
 *           the W tokens before pos0[b]+s
 *   sel     [batch, s, k] int32 or NULL (as in decode, per query)
 *   out     [batch, s, H, D]
 * Each query p attends kv of tokens max(0,p-W+1)..p (from kv_new for t >= pos0, from the
 * ring before) and its rows.  Errors as decode. */
int dsv4_csa_attn_prefill(const dsv4_attn_cfg* cfg, const void* q, const void* kv_new,
                          void* win_ring, const void* rows, int64_t row_cap,
                          const int32_t* sel, const int64_t* n_rows, const int64_t* pos0,
                          const float* sinks, void* out, int32_t batch, int64_t s, void* ws,
                          size_t ws_bytes, void* stream);

/* The layer's neighbours on either side of the attention.
 * Pages: mlx-lm PR #1189 (OmarB97's note 2 and stepnoy's patch: the rotary dims are the last
 * rd of each head, interleaved pairs turned by position * inv_freq; Thump604's fix list:
 * the attention output's rotary dims turned back); MTPLX PR #216 opening ("What V4
 * adds": grouped output-LoRA, 8 groups of rank 1024) and "Decode path: reference-faithful
 * bf16 activation storage" item 2 (wo_a [8192, 4096]); deepseek-v41-mlx "Why this exists"
 * (the rope inverse on the attention output; wo_a block-diagonal). */
typedef struct {
    int32_t heads;     /* H, 1..65535                                                      */
    int32_t dim;       /* D: head width, 1..4096                                           */
    int32_t rope_dim;  /* rd, even, 0..D: the last rd dims of each head turn               */
    int32_t inverse;   /* 0: turn by +angle (q, kv, qi before attention); 1: turn back by
                          the same angle (the attention output)                            */
    int32_t dtype;     /* dsv4_dtype                                                       */
} dsv4_rope_cfg;

/* RoPE in place on x [batch, s, H, D]: token t of sequence b (position pos0[b] + t) has the
 * pairs (x[D-rd+2i], x[D-rd+2i+1]) of every head turned by theta_i = fp32(position) *
 * inv_freq[i] (fp32 product), result (x0 cos - x1 sin, x0 sin + x1 cos) in fp32 (with -theta
 * when inverse), rounded to the storage dtype; other dims untouched.  inv_freq [rd/2] fp32.
 * Errors: EINVAL (NULL pointer, bad cfg, negative batch/s/position), ECAPACITY (a position
 * >= 2^31 - 1), EUNSUPPORTED (s > 65535), EHIP. */
int dsv4_rope(const dsv4_rope_cfg* cfg, void* x, const int64_t* pos0, int32_t batch, int64_t s,
              const float* inv_freq, void* stream);

typedef struct {
    int32_t groups;    /* G >= 1                                                           */
    int32_t in_dim;    /* K: inputs per group (H/G heads x D of the attention output)      */
    int32_t out_dim;   /* R: outputs per group (the rank)                                  */
    int32_t dtype;     /* dsv4_dtype of x, w and y                                         */
} dsv4_gproj_cfg;

/* Grouped (block-diagonal) projection: y[t, g, r] = sum_k w[g, r, k] * x[t, g, k], fp32
 * accumulation, rounded once to the storage dtype.
 *   x [tokens, G, K]  (the attention output [tokens, H, D] after the inverse rotation is
 *                      this with K = H/G * D: group g holds heads g*H/G .. (g+1)*H/G - 1)
 *   w [G, R, K]       (wo_a [G*R, K] read as G blocks of R rows)
 *   y [tokens, G, R]
 * Errors: EINVAL (NULL pointer, bad cfg, tokens < 0), EUNSUPPORTED (tokens x G x R above
 * 2^39), EHIP. */
int dsv4_grouped_proj(const dsv4_gproj_cfg* cfg, const void* x, const void* w, void* y,
                      int64_t tokens, void* stream);

/* Both lanes of one compressor from the layer's hidden states in one call: a = x w_kv^T and
 * g = x w_gate^T, fp32 accumulation, each rounded once to the storage dtype.  Pages: mlx-lm
 * PR #1189, Thump604's fix list (the ratio-4 compressor's wkv and wgate are [1024, 4096]
 * projections of the hidden state, the lanes 2*D wide); MTPLX PR #216 "What V4 adds" (the
 * gated pooling takes a kv lane and a gate lane per token).
 *   cfg   groups = 1, in_dim = hidden size K, out_dim = lane width W (coff * D), dtype
 *   x [tokens, K]; w_kv, w_gate [W, K]; a, g [tokens, W] (caller-owned device buffers, the
 *   lanes dsv4_compress_prefill / dsv4_compress_step read)
 * The two products share one launch where the tiled kernel applies (bf16, more than 32
 * tokens, K a multiple of 64, W of 128); otherwise they run as two dsv4_grouped_proj-style
 * launches with the same arithmetic.
 * Errors: EINVAL (NULL pointer, groups != 1, bad cfg, tokens < 0), EUNSUPPORTED (tokens x W
 * above 2^39), EHIP. */
int dsv4_lane_proj(const dsv4_gproj_cfg* cfg, const void* x, const void* w_kv, const void* w_gate, void* a,
                   void* g, int64_t tokens, void* stream);

/* Kernel timing for measurement.  While enabled, every kernel the library launches carries
 * a start/stop HIP event pair attached to its own dispatch (hipExtLaunchKernelGGL), so each
 * record is that kernel's execution time on its launch stream.  dsv4_trace_read() waits for the
 * recorded events and returns, for the kernels whose name contains `name_substr` (all when
 * NULL or ""; "=name" selects the kernel of exactly that name), the launch count and the
 * summed GPU duration in milliseconds.  Tracing
 * creates HIP events (it is the one facility that allocates); leave it off in production. */
int dsv4_trace_enable(int32_t on);
int dsv4_trace_reset(void);
int dsv4_trace_read(const char* name_substr, int64_t* launches, double* total_ms);
/* Name of the i-th distinct traced kernel (NULL past the end), for listing. */
const char* dsv4_trace_kernel_name(int32_t i);

#ifdef __cplusplus
}
#endif
#endif /* DSV4_H */
