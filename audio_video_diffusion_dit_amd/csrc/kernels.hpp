// Launch interfaces of the gfx950 kernels. Host code fills these argument structs after
// validating shapes; each launcher checks the structural preconditions its kernel relies on
// (alignment, tile coverage) and returns hipErrorInvalidValue instead of launching if one
// fails, so a kernel never sees a shape it was not written for.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace avdit {

// Rows of the packed sequence: [0, n_video) video, [n_video, n_valid) audio, then the tail.
// A batch of requests (batch > 1) stacks batch sequences of seq_pad rows each, request b with its
// own req_video[b] and req_valid[b]; n_video and n_valid then play no part.
enum { MAX_REQUESTS = 64 };
struct RowLayout {
  int32_t n_video;
  int32_t n_valid;
  int32_t seq_pad;   // rows per request
  int32_t batch;     // 0 or 1: one request; otherwise the number of requests
  int32_t req_video[MAX_REQUESTS];
  int32_t req_valid[MAX_REQUESTS];
};

__host__ __device__ inline int32_t total_rows(const RowLayout& r) {
  return r.batch > 1 ? r.batch * r.seq_pad : r.seq_pad;
}

struct RowInfo {
  int32_t req;    // request
  int32_t idx;    // row inside the request
  bool valid;
  int32_t mod;    // 0 video, 1 audio (valid rows)
};

__host__ __device__ inline RowInfo row_info(const RowLayout& r, int32_t row) {
  if (r.batch <= 1) return RowInfo{0, row, row < r.n_valid, row < r.n_video ? 0 : 1};
  const int32_t b = row / r.seq_pad;
  const int32_t i = row - b * r.seq_pad;
  return RowInfo{b, i, i < r.req_valid[b], i < r.req_video[b] ? 0 : 1};
}

// Whether rows [row0, row0 + n) hold a valid row; for a batch, n divides seq_pad (so the rows
// belong to one request).
__host__ __device__ inline bool rows_have_valid(const RowLayout& r, int32_t row0) {
  if (r.batch <= 1) return row0 < r.n_valid;
  const int32_t b = row0 / r.seq_pad;
  return row0 - b * r.seq_pad < r.req_valid[b];
}

// h = RMSNorm(x) * g * (1 + E[m][scale_chunk]) + E[m][shift_chunk], E = ada + temb.
struct NormModArgs {
  const void* x;      // [seq_pad, D] bf16, or fp32 when x_f32
  uint16_t* h;        // [seq_pad, D] bf16
  const float* gain;  // [D]
  const float* ada;   // [2, table_rows, D]
  const float* temb;  // [2, table_rows, D]
  RowLayout rows;
  int32_t D;
  int32_t shift_chunk, scale_chunk;
  float eps;
  int32_t x_f32;      // 1: x is fp32
  int64_t temb_stride;  // elements between the temb tables of successive requests (batch)
  int32_t table_rows = 6;  // rows per modality of ada/temb (6 in a block)
};
hipError_t launch_norm_mod(const NormModArgs& a, hipStream_t s);

// Per-head RMSNorm + NeoX RoPE of the q and k column blocks of qkv [seq_pad, 3D], in place.
struct QkNormRopeArgs {
  uint16_t* qkv;
  const float* q_gain;     // [Dh]
  const float* k_gain;     // [Dh]
  const int32_t* positions;  // [seq_pad] or null (position = row)
  const int32_t* req_positions[MAX_REQUESTS];  // batch: per-request [seq_pad] or null
  RowLayout rows;
  int32_t heads, head_dim;
  int64_t row_stride;      // elements between rows (3D)
  float eps;
  float inv_freq[64];      // base^(-2i/Dh), i < Dh/2, rounded once from float64
};
hipError_t launch_qk_norm_rope(const QkNormRopeArgs& a, hipStream_t s);

// x += dt_m * u (skipped when v and v_f32 are null), x_bf16 = bf16(x) (skipped when null); tail
// rows set to 0. u = v (bf16, or v_f32 fp32), or, when an older velocity v_prev / v_prev_f32 is
// given, the extrapolation u = v + lambda (v - v_prev).
struct StepArgs {
  float* x;
  const uint16_t* v;
  const float* v_f32;
  const uint16_t* v_prev;
  const float* v_prev_f32;
  float lambda;
  uint16_t* x_bf16;
  RowLayout rows;
  int32_t D;
  float dt_video, dt_audio;
};
hipError_t launch_step_update(const StepArgs& a, hipStream_t s);

// C[m][n] = sum_k A[m][k] * W[n][k] with a fused epilogue.
enum GemmEpilogue : int32_t {
  EPI_STORE = 0,        // out (bf16) = acc
  EPI_GATED_TO_F32 = 1, // out (fp32) = resid (bf16) + (ada + temb)[mod(m)][chunk][n] * acc
  EPI_SWIGLU = 2,       // out (bf16) = silu(acc_gate) * acc_up, gate row n, up row up_offset + n
  EPI_GATED_F32_IN = 3, // out (bf16) = resid (fp32) + (ada + temb)[mod(m)][chunk][n] * acc
  EPI_GATED_F32_TO_F32 = 4, // out (fp32) = resid (fp32) + (ada + temb)[mod(m)][chunk][n] * acc
};
struct GemmArgs {
  const uint16_t* A;  // [rows, K] activations, row stride lda
  const uint16_t* W;  // [N_w, K] weights, row stride ldw
  void* C;            // [rows, N] output (bf16, or fp32 for the *_TO_F32 epilogues), row stride ldc
  int64_t lda, ldw, ldc;
  int32_t N, K;       // output features, reduction length
  RowLayout rows;     // rows >= n_valid of C are written 0; rows >= seq_pad untouched
  int32_t epilogue;
  const void* resid;      // gated epilogues: [rows, N] (bf16 or fp32), row stride ldr
  int64_t ldr;
  const float* ada;       // gated epilogues: [2, 6, N]
  const float* temb;      // gated epilogues: [2, 6, N]
  int32_t chunk;          // gated epilogues: modulation chunk of the gate
  int32_t up_offset;      // EPI_SWIGLU: first up row of W (= F)
  int64_t temb_stride;    // gated epilogues: elements between successive requests' temb tables
};
hipError_t launch_gemm(const GemmArgs& a, hipStream_t s);

// Velocity head (k_head.hip). k_head_prep folds the final table of both modalities:
// mul[m][d] = gain[d] (1 + ada[m][1][d] + temb[m][1][d]) and
// cst[m][c] = sum_d (ada[m][0][d] + temb[m][0][d]) w[m][c][d] + bias[m][c].
struct HeadPrepArgs {
  const float* gain;   // [D]
  const float* ada;    // [2, 2, D]: row 0 shift, row 1 scale
  const float* temb;   // [2, 2, D]
  const uint16_t* w;   // [2, C, D] bf16
  const float* bias;   // [2, C] or null
  float* mul;          // out [2, D], 16-byte aligned
  float* cst;          // out [2, C], 16-byte aligned
  int32_t D, C;
};
hipError_t launch_head_prep(const HeadPrepArgs& a, hipStream_t s);
// k_head_proj, both modalities in one launch (m = 0 video, 1 audio): for each, over its own
// rows, v[r] = rsqrt(mean(x[r]^2) + eps) ((x[r] * mul) w^T) + cst for r < valid, 0 for
// valid <= r < rows; x * mul rounded to bf16 for the product.
struct HeadProjArgs {
  const void* x[2];       // [rows, D] bf16 (or fp32 with x_f32), row stride D, 16-byte aligned
  float* v[2];            // [rows, C] fp32, row stride ldv, 16-byte aligned
  const uint16_t* w[2];   // [C, D] bf16
  const float* mul[2];    // [D], 16-byte aligned
  const float* cst[2];    // [C], 16-byte aligned
  int32_t rows[2], valid[2];
  int32_t D, C;           // D a multiple of 64, at most 8192; C a multiple of 8
  int64_t ldv;
  float eps;
  int32_t x_f32;
  int32_t tiles0 = 0;     // set by the launcher: row tiles of modality 0
};
hipError_t launch_head_proj(const HeadProjArgs& a, hipStream_t s);

// Flash-style attention over packed requests; element (b, i, h, d) of q/k/v at
// b * batch_stride + i * row_stride + h * head_dim + d.
enum { ATTN_MAX_BATCH = 64 };
struct AttnArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  int64_t batch_stride, row_stride, o_batch_stride, o_row_stride;
  int32_t batch, seq_pad, heads, head_dim;
  int32_t fixed_valid;  // 1: sweep the whole padded length with a key mask
  float scale_log2;     // log2(e) / sqrt(head_dim)
  // Optional per-dimension gains [head_dim] of the Q/K RMSNorm that produced q and k (both or
  // neither). With them the kernel bounds every logit and, when the bound is small enough,
  // needs no running row maximum: it shifts by the bound, or not at all (softmax is shift and
  // scale invariant).
  const float* q_gain;
  const float* k_gain;
  int32_t valid[ATTN_MAX_BATCH];
};
hipError_t launch_attention(const AttnArgs& a, hipStream_t s);

// Sets the calling thread's dit_last_error() message and returns code (host code of the
// library's entry points outside abi.cpp).
int set_last_error(int code, const char* msg);

}  // namespace avdit
