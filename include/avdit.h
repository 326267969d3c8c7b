/*
 * avdit.h -- C-ABI of the MI355X (gfx950) joint audio-video DiT denoising step.
 *
 * Pages cited (by title and section):
 *   [P1] TeleFuser PR #38, "perf(minimax-h3): add conservative DiT velocity reuse"
 *   [P2] 1Cat-vLLM PR #584, "[Video] Add native H3 request-scoped TeaCache and Cache-DiT"
 *   [P3] TeleFuser PR #23, "[FEAT] Add MiniMax H3 joint audio-video generation"
 *
 * Conventions shared by every entry point:
 *  - "dev" pointers are HIP device memory, "host" pointers are ordinary CPU memory.
 *  - bf16 tensors are passed as uint16_t bit patterns (bfloat16, round-to-nearest-even
 *    on every store). All math inside the kernels is fp32.
 *  - Tensors are row-major and token-major. Weights use the [out, in] layout, so both
 *    operands of every projection are contiguous along the reduction axis.
 *  - The packed sequence has seq_pad rows: video rows 0..n_video-1 (modality 0), audio
 *    rows n_video..n_valid-1 (modality 1), then a tail up to seq_pad ([P3] "Motivation",
 *    packed joint token layout; [P1] section 2, zero tail). Every output tensor has an
 *    exactly-zero tail, whatever the input tail holds.
 *  - Ownership: the caller allocates and owns every buffer, the workspace and the
 *    stream. The library allocates no device memory and keeps no state between calls
 *    except a thread-local error string. Device work is enqueued asynchronously on the
 *    given stream (NULL = the default stream); calls return after enqueueing.
 *  - Alignment: activations (x_in, x_out, latents, velocities), temb tables, and the fp32
 *    parameters norm1_g, norm2_g, q_g, k_g, ada (and the head's norm_g, ada, bias and its
 *    bf16 w_out) are read or written with 16-byte vector accesses and must be 16-byte aligned
 *    (DIT_ERR_INVALID otherwise). The block's bf16 weight matrices may have any 2-byte
 *    alignment; unaligned ones take a slower loader.
 *  - Size limits: the kernels address their large operands through 32-bit byte offsets,
 *    so each of these must span less than 2 GiB, else DIT_ERR_UNSUPPORTED: the weights
 *    w_qkv, w_gate_up, w_down; the block activations [rows, D] and the SwiGLU activations
 *    [rows, F] (rows = all rows of the call, batch * seq_pad for a batch); one request's
 *    q/k/v rows [seq_pad, 3D] (at hidden 3072: seq_pad <= 116,508). The workspace-size
 *    functions apply the same limits and return 0. (The velocity head addresses its input
 *    per 64 rows, and one modality's weight [C, D] stays below 1 GiB: no limit.)
 *  - Errors: every argument is validated before anything is enqueued. On failure
 *    nothing is enqueued, a negative status is returned and dit_last_error() describes
 *    it. A launch failure reported by the runtime after enqueueing maps to
 *    DIT_ERR_DEVICE. There are no environment variables and no fallback paths.
 */
#ifndef AVDIT_H
#define AVDIT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  DIT_OK = 0,
  DIT_ERR_INVALID = -1,      /* a null pointer, inconsistent sizes or out-of-range values */
  DIT_ERR_UNSUPPORTED = -2,  /* a well-formed request this library does not implement */
  DIT_ERR_WORKSPACE = -3,    /* the workspace is smaller than dit_workspace_size() */
  DIT_ERR_DEVICE = -4        /* the HIP runtime rejected a launch */
};

enum { DIT_ATTN_VALID_ONLY = 0, DIT_ATTN_FIXED_VALID = 1 };
enum { DIT_CACHE_OFF = 0, DIT_CACHE_VELOCITY = 1, DIT_CACHE_EXTRAPOLATE = 2 };

/* Model dimensions. hidden = heads * head_dim; head_dim is 64 or 128; n_mod is 2 (video,
 * audio). norm_eps is the RMSNorm epsilon of the token norms, qk_eps that of the per-head
 * Q/K norms, rope_base the NeoX rotary base. */
typedef struct {
  int32_t hidden, heads, head_dim, ffn, n_mod;
  float norm_eps, qk_eps, rope_base;
} dit_dims;

/* Packed-sequence layout ([P3] "Motivation"; [P1] section 2). positions: dev int32
 * [seq_pad] rotary positions, or NULL for position(l) = l. Request-static: built once per
 * request and reused by every block and every step ([P3] "Changes Made"). */
typedef struct {
  int32_t n_video, n_audio, seq_pad;
  const int32_t* positions;
} dit_layout;

/* One block's parameters (all dev). Matrices are bf16, the rest fp32 (precision-sensitive
 * parameters stay fp32, [P3] "Motivation").
 *   w_qkv [3D, D]: rows 0..D-1 produce q, D..2D-1 k, 2D..3D-1 v; inside each, the output
 *                  feature is head * head_dim + d.
 *   w_o [D, D]; w_gate_up [2F, D] with the gate rows first; w_down [D, F].
 *   norm1_g, norm2_g [D]; q_g, k_g [head_dim];
 *   ada [n_mod, 6, D]: the block's modulation table, chunks ordered shift_msa, scale_msa,
 *                      gate_msa, shift_mlp, scale_mlp, gate_mlp. */
typedef struct {
  const uint16_t* w_qkv;
  const uint16_t* w_o;
  const uint16_t* w_gate_up;
  const uint16_t* w_down;
  const float* norm1_g;
  const float* norm2_g;
  const float* q_g;
  const float* k_g;
  const float* ada;
} dit_block_weights;

/* Velocity-reuse cache policy ([P1] section 3, MiniMaxH3DiTCacheConfig). mode DIT_CACHE_OFF,
 * DIT_CACHE_VELOCITY ("conservative" is an alias resolved by the caller) or
 * DIT_CACHE_EXTRAPOLATE. Reuse happens only for progress i/N in [start_ratio, end_ratio), with a
 * forced refresh every refresh_interval steps and at most max_consecutive_reuse reuses in a
 * row. DIT_CACHE_VELOCITY reuses the last refresh's velocity v_r; DIT_CACHE_EXTRAPOLATE reuses
 * on the same intervals but continues the velocity to first order from the last two refreshes
 * r' < r, v_r + (i - r) / (r - r') (v_r - v_r') (plain reuse while only one refresh exists; a
 * velocity-level reading of the order-1 TaylorSeer predictor, [P2] "Purpose", "Test
 * Result"). threshold must be NaN (the pages define only threshold=None). */
typedef struct {
  int32_t mode;
  double start_ratio, end_ratio;
  int32_t refresh_interval, max_consecutive_reuse;
  double threshold;
} dit_cache_policy;

/* Work accounting of one denoise_loop call ([P2] "Purpose": only executed useful
 * matrix/attention work counts). useful_flops = dit_calls * n_blocks *
 * (8 V D^2 + 6 V D F + 4 V^2 D) with V = n_valid. step_hit: host uint8 [n_intervals] or NULL;
 * when set it receives 1 for every reused interval. */
typedef struct {
  int32_t dit_calls, cache_hits;
  int64_t executed_blocks, skipped_blocks;
  double useful_flops;
  uint8_t* step_hit;
} dit_loop_stats;

/* Byte offsets of the intermediates inside a workspace, for inspection after a call. Each
 * is a row-major tensor with seq_pad rows whose tail rows are 0 after a block call:
 *   h [L, D] bf16 (norm1 output), qkv [L, 3D] bf16 (q and k after Q/K norm and RoPE),
 *   attn_out [L, D] bf16, x1 [L, D] fp32 (mid-block residual, kept fp32), h2 [L, D] bf16,
 *   act [L, ffn_ld] bf16 (SwiGLU output, row stride ffn_ld; columns >= ffn undefined),
 *   then the loop buffers (present when n_blocks >= 1): x_bf16 [L, D] bf16, then ping, pong,
 *   velocity, velocity_prev, each [L, D] and sized for fp32 (bf16 rows in denoise_loop, fp32
 *   rows in denoise_loop_f32; velocity_prev holds the older refresh's velocity under
 *   DIT_CACHE_EXTRAPOLATE, the two velocity buffers alternating). */
typedef struct {
  size_t h, qkv, attn_out, x1, h2, act, x_bf16, ping, pong, velocity, velocity_prev, total;
  int64_t ffn_ld;
} dit_workspace_map;

/* Parameters of the velocity head, all dev: the final AdaLN layer and the output projection
 * that turn the stack output into the velocity ([P2] "Test Result": the model ends in a final
 * AdaLN layer with a table of its own; [P1] section 1: the DiT predicts the flow-matching
 * velocity).
 *   norm_g [D]; ada [n_mod, 2, D], rows shift then scale;
 *   w_out bf16 [n_mod, out_channels, D], 16-byte aligned: one [out, in] matrix per modality;
 *   bias fp32 [n_mod, out_channels], 16-byte aligned, or NULL for none;
 *   out_channels: a positive multiple of 8, at most 65536. */
typedef struct {
  const float* norm_g;
  const float* ada;
  const uint16_t* w_out;
  const float* bias;
  int32_t out_channels;
} dit_head_weights;

/* Last error message of the calling thread ("" if none). Never NULL. */
const char* dit_last_error(void);

/* Library version string. */
const char* dit_version(void);

/* Hit/refresh schedule of a denoise loop ([P1] section 3): step_hit host uint8
 * [n_intervals] receives 1 for each interval that reuses the previous velocity. Pure host
 * work. Returns DIT_ERR_INVALID for a null pointer, n_intervals < 0, ratios outside [0, 1],
 * start > end, refresh_interval < 1 or max_consecutive_reuse < 0; DIT_ERR_UNSUPPORTED for a
 * non-NaN threshold or an unknown mode. */
int dit_cache_schedule(const dit_cache_policy* policy, int32_t n_intervals, uint8_t* step_hit);

/* Workspace needed by dit_block_forward (n_blocks = 0) or denoise_loop (n_blocks >= 1), and
 * the offsets of its parts. Returns the size in bytes, or 0 with dit_last_error() set if the
 * dims/layout are invalid or unsupported. map may be NULL. */
size_t dit_workspace_size(const dit_dims* dims, const dit_layout* layout, int32_t n_blocks,
                          dit_workspace_map* map);

/* One joint audio-video DiT block ([P1] section 2; [P3] "Changes Made"):
 *   E = ada + temb; h = RMSNorm(x) g1 (1 + E[m,1]) + E[m,0];
 *   q,k,v = h Wqkv^T; q,k <- RoPE_neox(RMSNorm_head(q,k) g_{q,k});
 *   o = softmax(q k^T / sqrt(head_dim)) v over the valid rows only;
 *   x1 = x + E[m,2] (o Wo^T); h2 = RMSNorm(x1) g2 (1 + E[m,4]) + E[m,3];
 *   x_out = x1 + E[m,5] ((silu(h2 Wg^T) * (h2 Wu^T)) Wd^T); tail rows of x_out are 0.
 * temb: dev fp32 [n_mod, 6, D] timestep embedding. x_in, x_out: dev bf16 [seq_pad, D]; they
 * may not alias each other or the workspace. attn_mode: DIT_ATTN_VALID_ONLY (work bounded by
 * n_valid) or DIT_ATTN_FIXED_VALID (the whole padded length with a key mask); both give
 * bitwise-identical outputs ([P1] section 5: the lossless modes are bit-exact).
 * ws: dev workspace of at least dit_workspace_size(dims, layout, 0, NULL) bytes, 256-byte
 * aligned; its contents on entry do not matter. stream: hipStream_t. */
int dit_block_forward(const dit_dims* dims, const dit_layout* layout,
                      const dit_block_weights* weights, const float* temb,
                      const uint16_t* x_in, uint16_t* x_out, int32_t attn_mode, void* ws,
                      size_t ws_bytes, void* stream);

/* dit_block_forward without a workspace argument, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation). The block's intermediates live in a device array built into the library, one
 * copy per GPU of DIT_NOALLOC_SCRATCH_BYTES (128 MiB), held from the first call on that GPU
 * (its address is looked up once per device, on the device current at the call) until the
 * process ends. The call allocates nothing and runs the same kernels as dit_block_forward,
 * with the same result bit for bit. A block whose dit_workspace_size(dims, layout, 0) exceeds
 * DIT_NOALLOC_SCRATCH_BYTES is rejected with DIT_ERR_UNSUPPORTED before any device call.
 * Every call on one GPU shares that GPU's array: calls that overlap in time on one GPU (other
 * streams, other threads) race and must be serialised by the caller. Other arguments, errors
 * and aliasing rules as dit_block_forward; a failed scratch lookup is DIT_ERR_DEVICE. */
#define DIT_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
int dit_block_forward_noalloc(const dit_dims* dims, const dit_layout* layout,
                              const dit_block_weights* weights, const float* temb,
                              const uint16_t* x_in, uint16_t* x_out, int32_t attn_mode,
                              void* stream);

/* Workspace for dit_block_forward_batched: the workspace of one block over all batch * seq_pad
 * rows, and its map. Returns 0 with dit_last_error() set for invalid dims or layouts. */
size_t dit_workspace_size_batched(const dit_dims* dims, const dit_layout* layouts, int32_t batch,
                                  dit_workspace_map* map);

/* One block over a batch of requests in a single call: every launch covers all requests, the
 * GEMMs skip the row tiles past each request's valid length, and attention runs per (request,
 * head) over that request's valid keys only ([P1] section 2: valid-only work over each zero
 * tail; [P2] "Purpose": requests are independent). layouts: host [batch] (batch <= 64), each
 * request's n_video, n_audio and positions; all share seq_pad, a multiple of 256 when batch > 1
 * (DIT_ERR_UNSUPPORTED otherwise). Row b * seq_pad + i of x_in / x_out (dev bf16 [batch * seq_pad,
 * D]) is row i of request b; temb: dev fp32 [batch, n_mod, 6, D], request b's table at
 * b * n_mod * 6 * D. Each request's output equals its own dit_block_forward output bit for
 * bit. Workspace from dit_workspace_size_batched; aliasing rules and errors as
 * dit_block_forward. */
int dit_block_forward_batched(const dit_dims* dims, const dit_layout* layouts, int32_t batch,
                              const dit_block_weights* weights, const float* temb,
                              const uint16_t* x_in, uint16_t* x_out, int32_t attn_mode, void* ws,
                              size_t ws_bytes, void* stream);

/* The same block with an fp32 residual stream ([P2] "Test Plan" and "Test Result": the
 * FP32-residual runs): x_in and x_out are dev fp32 [seq_pad, D], 16-byte aligned. RMSNorm 1 reads
 * the fp32 input and both gated residuals (x1 = x + E[m,2] (o Wo^T), x_out = x1 + E[m,5] (...))
 * read and write fp32; the matrix operands h, q/k/v, o, h2 and the SwiGLU output stay bf16.
 * Arguments, workspace, aliasing rules and errors as dit_block_forward. */
int dit_block_forward_f32(const dit_dims* dims, const dit_layout* layout,
                          const dit_block_weights* weights, const float* temb, const float* x_in,
                          float* x_out, int32_t attn_mode, void* ws, size_t ws_bytes,
                          void* stream);

/* Flow-matching Euler update of the fp32 latent ([P3] "Changes Made": optimized scheduler
 * updates with independent modality schedules): for valid rows of modality m,
 * x += dt_m * v; x_bf16 = bf16(x) (the next DiT input). Tail rows of x and x_bf16 are set
 * to 0. x: dev fp32 [seq_pad, hidden] in/out; v: dev bf16 [seq_pad, hidden]; x_bf16: dev
 * bf16 [seq_pad, hidden], or NULL to skip the copy. hidden must be a multiple of 8. */
int step_update(float* x, const uint16_t* v, uint16_t* x_bf16, const dit_layout* layout,
                int32_t hidden, float dt_video, float dt_audio, void* stream);

/* Cached denoise loop ([P1] sections 1 and 3): for each interval i the schedule of
 * dit_cache_schedule decides refresh or reuse; on a refresh the n_blocks-block stack runs on
 * bf16(x_i) with temb_steps[i] and its output is retained as the velocity (both modalities);
 * on a reuse the retained velocity is used and no block runs; then
 * x_{i+1} = x_i + (sigma_m[i+1] - sigma_m[i]) v per row modality.
 *   blocks: host array [n_blocks] of dev weights; sigmas_video, sigmas_audio: host fp32
 *   [n_intervals + 1]; temb_steps: dev fp32 [n_intervals, n_mod, 6, D];
 *   x_latent: dev fp32 [seq_pad, D] in/out (tail rows are zero on return);
 *   stats: host, filled from the schedule (may be NULL).
 * Enqueues every step without a device-to-host synchronization. The per-request cache state
 * (retained velocity, reuse counter) lives only in the workspace and in this call, and is
 * gone when it returns, on success or error ([P2] "Purpose"). */
int denoise_loop(const dit_dims* dims, const dit_layout* layout,
                 const dit_block_weights* blocks, int32_t n_blocks, int32_t n_intervals,
                 const float* sigmas_video, const float* sigmas_audio,
                 const float* temb_steps, const dit_cache_policy* policy, float* x_latent,
                 int32_t attn_mode, dit_loop_stats* stats, void* ws, size_t ws_bytes,
                 void* stream);

/* The cached denoise loop with an fp32 residual stream ([P2] "Test Plan" and "Test Result":
 * FP32 residuals): on a refresh the stack runs on the fp32 latent x_i itself (no bf16
 * conversion), the blocks chain through fp32 rows (dit_block_forward_f32) and the retained
 * velocity is the fp32 output of the last block; the Euler step then uses that fp32 velocity.
 * The sigma arrays may hold any schedule, a different one per modality ([P3] "Motivation":
 * independent schedulers). Arguments, workspace (dit_workspace_size with n_blocks >= 1),
 * request-scoped state and errors as denoise_loop. */
int denoise_loop_f32(const dit_dims* dims, const dit_layout* layout,
                     const dit_block_weights* blocks, int32_t n_blocks, int32_t n_intervals,
                     const float* sigmas_video, const float* sigmas_audio,
                     const float* temb_steps, const dit_cache_policy* policy, float* x_latent,
                     int32_t attn_mode, dit_loop_stats* stats, void* ws, size_t ws_bytes,
                     void* stream);

/* Workspace of dit_velocity_head and dit_velocity_head_f32 for out_channels output channels:
 * the final table folded per modality, fp32 mul [2, D] and cst [2, out_channels] (see
 * dit_velocity_head); independent of seq_pad. Returns 0 with dit_last_error() set for invalid
 * dims, layout or out_channels. */
size_t dit_head_workspace_size(const dit_dims* dims, const dit_layout* layout,
                               int32_t out_channels);

/* Velocity head ([P2] "Test Result", final AdaLN layer; [P1] section 1): for a valid row l of
 * modality m, h = x_l / sqrt(mean(x_l^2) + norm_eps) * norm_g * (1 + E[m][1]) + E[m][0] with
 * E = head->ada + temb (the same fused RMSNorm with indexed modulation as the block), then
 * v_l = h W_m^T + b_m in fp32. Evaluated in one pass over x as
 * v_l = r_l ((x_l * mul_m) W_m^T) + cst_m with r_l = 1 / sqrt(mean(x_l^2) + norm_eps),
 * mul_m = norm_g * (1 + E[m][1]) and cst_m = E[m][0] W_m^T + b_m (fp32): x_l * mul_m is rounded
 * to bf16 for the product, everything else stays fp32. Tail rows of v are 0.
 *   x: dev bf16 [seq_pad, D], the stack output, 16-byte aligned;
 *   temb: dev fp32 [n_mod, 2, D], the timestep part of the final table;
 *   v: dev fp32 [seq_pad, out_channels], 16-byte aligned.
 * x, v and the workspace must not overlap (DIT_ERR_INVALID). Other errors as
 * dit_block_forward. */
int dit_velocity_head(const dit_dims* dims, const dit_layout* layout,
                      const dit_head_weights* head, const float* temb, const uint16_t* x,
                      float* v, void* ws, size_t ws_bytes, void* stream);

/* The same head on an fp32 stack output (the fp32 residual stream): x dev fp32 [seq_pad, D],
 * 16-byte aligned. Everything else as dit_velocity_head. */
int dit_velocity_head_f32(const dit_dims* dims, const dit_layout* layout,
                          const dit_head_weights* head, const float* temb, const float* x,
                          float* v, void* ws, size_t ws_bytes, void* stream);

/* Batched valid-only / fixed-valid attention ([P1] section 2). For request b, head h and
 * query row i < valid_lens[b]: o = softmax_j(q_i . k_j / sqrt(head_dim)) v_j over
 * j < valid_lens[b]; rows i >= valid_lens[b] of o are 0. q, k, v, o: dev bf16; element
 * (b, i, h, d) is at ptr[b * batch_stride + i * row_stride + h * head_dim + d] (strides in
 * elements, row_stride a multiple of 8; q, k, v share strides, o has its own). For the
 * block's qkv buffer, q = qkv, k = qkv + D, v = qkv + 2D with row_stride 3D.
 * valid_lens: host int32 [batch], each in [0, seq_pad]; batch <= 64; head_dim 64 or 128.
 * q_gain, k_gain: dev fp32 [head_dim] or both NULL. When given, q and k must be outputs of the
 * per-head Q/K RMSNorm with these gains ([P3] "Changes Made": fused Q/K RMSNorm), which bounds
 * every logit by max|q_gain| max|k_gain| sqrt(head_dim); when that bound is small the kernel
 * needs no running row maximum (it shifts by the bound, or for bounds up to 30 in log2 units
 * not at all; same result up to rounding). Passing gains for q, k that did not come out of
 * such a norm is undefined. */
int dit_attention_forward(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                          uint16_t* o, int32_t batch, int32_t seq_pad, int32_t heads,
                          int32_t head_dim, int64_t batch_stride, int64_t row_stride,
                          int64_t o_batch_stride, int64_t o_row_stride,
                          const int32_t* valid_lens, const float* q_gain, const float* k_gain,
                          int32_t attn_mode, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* AVDIT_H */
