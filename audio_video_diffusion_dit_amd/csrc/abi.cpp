// C-ABI of the joint audio-video DiT denoising step: argument validation, the host-side cache
// schedule, the block composer and the denoise loop. Everything here is host code; every step
// of the math runs in the HIP kernels declared in kernels.hpp.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/avdit.h"
#include "kernels.hpp"

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

}  // namespace

int avdit::set_last_error(int code, const char* msg) {
  g_err = msg;
  return code;
}

namespace {

constexpr size_t kAlign = 256;
constexpr int32_t kMaxSeq = 1 << 20;
constexpr int32_t kMaxHidden = 8192;
constexpr int32_t kMaxFfn = 65536;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

int check_dims(const dit_dims* d) {
  if (!d) return fail(DIT_ERR_INVALID, "dims is null");
  if (d->hidden <= 0 || d->heads <= 0 || d->head_dim <= 0 || d->ffn <= 0)
    return fail(DIT_ERR_INVALID, "dims must be positive (hidden %d, heads %d, head_dim %d, ffn %d)",
                d->hidden, d->heads, d->head_dim, d->ffn);
  if (d->head_dim != 64 && d->head_dim != 128)
    return fail(DIT_ERR_UNSUPPORTED, "head_dim %d is not supported (64 or 128)", d->head_dim);
  if ((int64_t)d->heads * d->head_dim != d->hidden)
    return fail(DIT_ERR_INVALID, "hidden %d != heads %d * head_dim %d", d->hidden, d->heads,
                d->head_dim);
  if (d->hidden > kMaxHidden)
    return fail(DIT_ERR_UNSUPPORTED, "hidden %d exceeds %d", d->hidden, kMaxHidden);
  if (d->ffn > kMaxFfn) return fail(DIT_ERR_UNSUPPORTED, "ffn %d exceeds %d", d->ffn, kMaxFfn);
  if (d->n_mod != 2)
    return fail(DIT_ERR_UNSUPPORTED, "n_mod %d is not supported (video + audio = 2)", d->n_mod);
  if (!(d->norm_eps >= 0.0f) || !std::isfinite(d->norm_eps) || !(d->qk_eps >= 0.0f) ||
      !std::isfinite(d->qk_eps))
    return fail(DIT_ERR_INVALID, "epsilons must be finite and >= 0");
  if (!(d->rope_base > 0.0f) || !std::isfinite(d->rope_base))
    return fail(DIT_ERR_INVALID, "rope_base must be finite and > 0");
  return DIT_OK;
}

int check_layout(const dit_layout* l) {
  if (!l) return fail(DIT_ERR_INVALID, "layout is null");
  if (l->n_video < 0 || l->n_audio < 0 || l->seq_pad < 0)
    return fail(DIT_ERR_INVALID, "layout counts must be >= 0");
  if ((int64_t)l->n_video + l->n_audio > l->seq_pad)
    return fail(DIT_ERR_INVALID, "seq_pad %d < n_video %d + n_audio %d", l->seq_pad, l->n_video,
                l->n_audio);
  if (l->seq_pad > kMaxSeq) return fail(DIT_ERR_UNSUPPORTED, "seq_pad %d exceeds %d", l->seq_pad, kMaxSeq);
  return DIT_OK;
}

int check_policy(const dit_cache_policy* p) {
  if (!p) return fail(DIT_ERR_INVALID, "policy is null");
  if (p->mode != DIT_CACHE_OFF && p->mode != DIT_CACHE_VELOCITY && p->mode != DIT_CACHE_EXTRAPOLATE)
    return fail(DIT_ERR_UNSUPPORTED, "cache mode %d is not supported", p->mode);
  if (!(p->start_ratio >= 0.0 && p->start_ratio <= 1.0) ||
      !(p->end_ratio >= 0.0 && p->end_ratio <= 1.0))
    return fail(DIT_ERR_INVALID, "cache ratios must lie in [0, 1]");
  if (p->start_ratio > p->end_ratio) return fail(DIT_ERR_INVALID, "start_ratio > end_ratio");
  if (p->refresh_interval < 1) return fail(DIT_ERR_INVALID, "refresh_interval must be >= 1");
  if (p->max_consecutive_reuse < 0)
    return fail(DIT_ERR_INVALID, "max_consecutive_reuse must be >= 0");
  if (!std::isnan(p->threshold))
    return fail(DIT_ERR_UNSUPPORTED, "a reuse threshold is not supported (only None)");
  return DIT_OK;
}

// Greedy reuse rule of MiniMaxH3DiTCacheConfig (TeleFuser PR #38, section 3): interval i at
// progress i/N reuses when a velocity exists, i/N lies in [start, end) and fewer than
// min(max_consecutive_reuse, refresh_interval - 1) reuses happened since the last refresh.
void schedule(const dit_cache_policy* p, int32_t n, uint8_t* hit) {
  if (p->mode == DIT_CACHE_OFF) {
    if (n > 0) std::memset(hit, 0, (size_t)n);
    return;
  }
  const int32_t cap = p->max_consecutive_reuse < p->refresh_interval - 1 ? p->max_consecutive_reuse
                                                                         : p->refresh_interval - 1;
  bool have = false;
  int32_t run = 0;
  for (int32_t i = 0; i < n; ++i) {
    const double progress = (double)i / (double)n;
    const bool in_window = progress >= p->start_ratio && progress < p->end_ratio;
    if (have && in_window && run < cap) {
      hit[i] = 1;
      ++run;
    } else {
      hit[i] = 0;
      have = true;
      run = 0;
    }
  }
}

int64_t ffn_ld(const dit_dims* d) { return ((int64_t)d->ffn + 7) / 8 * 8; }

void build_map(const dit_dims* d, const dit_layout* l, int32_t n_blocks, dit_workspace_map* m) {
  const size_t L = (size_t)l->seq_pad, D = (size_t)d->hidden;
  const size_t row_d = align_up(L * D * 2);
  size_t off = 0;
  m->h = off; off += row_d;
  m->qkv = off; off += align_up(L * 3 * D * 2);
  m->attn_out = off; off += row_d;
  m->x1 = off; off += align_up(L * D * 4);
  m->h2 = off; off += row_d;
  m->ffn_ld = ffn_ld(d);
  m->act = off; off += align_up(L * (size_t)m->ffn_ld * 2);
  if (n_blocks >= 1) {
    // ping, pong and velocity hold bf16 rows in the bf16-residual loop and fp32 rows in the
    // fp32-residual loop: sized for fp32
    const size_t row_f = align_up(L * D * 4);
    m->x_bf16 = off; off += row_d;
    m->ping = off; off += row_f;
    m->pong = off; off += row_f;
    m->velocity = off; off += row_f;
    m->velocity_prev = off; off += row_f;
  } else {
    m->x_bf16 = m->ping = m->pong = m->velocity = m->velocity_prev = 0;
  }
  m->total = off < kAlign ? kAlign : off;
}

int check_weight_alignment(const dit_block_weights* w, int idx);

int check_weights(const dit_block_weights* w, int idx) {
  if (!w) return fail(DIT_ERR_INVALID, "block %d weights are null", idx);
  if (!w->w_qkv || !w->w_o || !w->w_gate_up || !w->w_down || !w->norm1_g || !w->norm2_g ||
      !w->q_g || !w->k_g || !w->ada)
    return fail(DIT_ERR_INVALID, "block %d has a null weight pointer", idx);
  return check_weight_alignment(w, idx);
}

// The kernels address their large operands through buffer resources with 32-bit byte offsets,
// so each operand must span less than 2 GiB. Checked before anything is enqueued.
constexpr int64_t kMaxSpan = (int64_t)1 << 31;

int check_span(int64_t bytes, const char* what) {
  if (bytes >= kMaxSpan)
    return fail(DIT_ERR_UNSUPPORTED,
                "%s spans %lld bytes; the kernels address at most 2 GiB - 1 per operand", what,
                (long long)bytes);
  return DIT_OK;
}

// Operand spans of one block over rows_total rows (a batch: all requests), seq_pad rows per
// request: the projection weights, the activations the GEMMs read, and one request's q/k/v rows
// that attention reads.
int check_block_spans(const dit_dims* d, int64_t rows_total, int64_t seq_pad) {
  const int64_t D = d->hidden, F = d->ffn;
  int st;
  if ((st = check_span(3 * D * D * 2, "the qkv weight [3D, D]")) != DIT_OK) return st;
  if ((st = check_span(2 * F * D * 2, "the gate/up weight [2F, D]")) != DIT_OK) return st;
  if ((st = check_span(D * F * 2, "the down weight [D, F]")) != DIT_OK) return st;
  if ((st = check_span(rows_total * D * 2, "the block activations [rows, D]")) != DIT_OK) return st;
  if ((st = check_span(rows_total * ffn_ld(d) * 2, "the SwiGLU activations [rows, F]")) != DIT_OK)
    return st;
  if ((st = check_span(seq_pad * 3 * D * 2, "one request's q/k/v rows [seq_pad, 3D]")) != DIT_OK)
    return st;
  return DIT_OK;
}

// Pointers the kernels read or write with 16-byte vector accesses.
int check_aligned16(const void* p, const char* what) {
  if (((uintptr_t)p & 15) != 0) return fail(DIT_ERR_INVALID, "%s must be 16-byte aligned", what);
  return DIT_OK;
}

int check_weight_alignment(const dit_block_weights* w, int idx) {
  const void* ptrs[] = {w->norm1_g, w->norm2_g, w->q_g, w->k_g, w->ada};
  const char* names[] = {"norm1_g", "norm2_g", "q_g", "k_g", "ada"};
  for (int i = 0; i < 5; ++i)
    if (((uintptr_t)ptrs[i] & 15) != 0)
      return fail(DIT_ERR_INVALID, "block %d: %s must be 16-byte aligned", idx, names[i]);
  return DIT_OK;
}

int device_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return DIT_OK;
  return fail(DIT_ERR_DEVICE, "%s launch failed: %s", what, hipGetErrorString(e));
}

bool ranges_overlap(const void* a, size_t an, const void* b, size_t bn) {
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + bn && b0 < a0 + an;
}

// Rows of a block call: one request (from its dit_layout) or a batch of requests that share
// seq_pad, with per-request rotary positions and timestep tables (temb_stride elements apart).
struct BlockRows {
  avdit::RowLayout rows{};
  const int32_t* positions = nullptr;
  const int32_t* req_positions[avdit::MAX_REQUESTS] = {};
  int64_t temb_stride = 0;
};

BlockRows single_rows(const dit_layout* l) {
  BlockRows r;
  r.rows = avdit::RowLayout{l->n_video, l->n_video + l->n_audio, l->seq_pad};
  r.positions = l->positions;
  return r;
}

// Enqueue one block on `s`: eight launches, no host synchronisation. x_in and x_out are bf16
// rows, or fp32 rows when f32 (the fp32 residual stream: norm1 reads fp32, both gated
// residual epilogues read and write fp32).
int enqueue_block(const dit_dims* d, const BlockRows& br, const dit_block_weights* w,
                  const float* temb, const void* x_in, void* x_out, int32_t attn_mode,
                  char* ws, const dit_workspace_map& m, hipStream_t s, bool f32 = false) {
  using namespace avdit;
  const int32_t D = d->hidden, F = d->ffn, L = br.rows.seq_pad;
  const RowLayout& rows = br.rows;
  const int32_t batch = rows.batch > 1 ? rows.batch : 1;
  uint16_t* h = reinterpret_cast<uint16_t*>(ws + m.h);
  uint16_t* qkv = reinterpret_cast<uint16_t*>(ws + m.qkv);
  uint16_t* att = reinterpret_cast<uint16_t*>(ws + m.attn_out);
  float* x1 = reinterpret_cast<float*>(ws + m.x1);
  uint16_t* h2 = reinterpret_cast<uint16_t*>(ws + m.h2);
  uint16_t* act = reinterpret_cast<uint16_t*>(ws + m.act);
  int st;

  NormModArgs n1{};
  n1.x = x_in; n1.h = h; n1.gain = w->norm1_g; n1.ada = w->ada; n1.temb = temb;
  n1.rows = rows; n1.D = D; n1.shift_chunk = 0; n1.scale_chunk = 1; n1.eps = d->norm_eps;
  n1.x_f32 = f32 ? 1 : 0; n1.temb_stride = br.temb_stride;
  if ((st = device_status(launch_norm_mod(n1, s), "norm1+modulation")) != DIT_OK) return st;

  GemmArgs g{};
  g.A = h; g.W = w->w_qkv; g.C = qkv; g.lda = D; g.ldw = D; g.ldc = 3 * D;
  g.N = 3 * D; g.K = D; g.rows = rows; g.epilogue = EPI_STORE;
  if ((st = device_status(launch_gemm(g, s), "qkv projection")) != DIT_OK) return st;

  QkNormRopeArgs r{};
  r.qkv = qkv; r.q_gain = w->q_g; r.k_gain = w->k_g; r.positions = br.positions; r.rows = rows;
  for (int b = 0; b < MAX_REQUESTS; ++b) r.req_positions[b] = br.req_positions[b];
  r.heads = d->heads; r.head_dim = d->head_dim; r.row_stride = 3 * D; r.eps = d->qk_eps;
  for (int i = 0; i < d->head_dim / 2; ++i)
    r.inv_freq[i] = (float)std::pow((double)d->rope_base, -2.0 * i / (double)d->head_dim);
  if ((st = device_status(launch_qk_norm_rope(r, s), "q/k norm+rope")) != DIT_OK) return st;

  AttnArgs at{};
  at.q = qkv; at.k = qkv + D; at.v = qkv + 2 * D; at.o = att;
  at.batch_stride = (int64_t)L * 3 * D; at.row_stride = 3 * D;
  at.o_batch_stride = (int64_t)L * D; at.o_row_stride = D;
  at.batch = batch; at.seq_pad = L; at.heads = d->heads; at.head_dim = d->head_dim;
  at.fixed_valid = attn_mode == DIT_ATTN_FIXED_VALID ? 1 : 0;
  at.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)d->head_dim));
  for (int b = 0; b < batch; ++b) at.valid[b] = rows.batch > 1 ? rows.req_valid[b] : rows.n_valid;
  at.q_gain = w->q_g; at.k_gain = w->k_g;  // q, k come out of the Q/K RMSNorm with these gains
  if ((st = device_status(launch_attention(at, s), "attention")) != DIT_OK) return st;

  GemmArgs go{};
  go.A = att; go.W = w->w_o; go.C = x1; go.lda = D; go.ldw = D; go.ldc = D; go.N = D; go.K = D;
  go.rows = rows; go.epilogue = f32 ? EPI_GATED_F32_TO_F32 : EPI_GATED_TO_F32; go.resid = x_in;
  go.ldr = D; go.ada = w->ada; go.temb_stride = br.temb_stride;
  go.temb = temb; go.chunk = 2;
  if ((st = device_status(launch_gemm(go, s), "out projection")) != DIT_OK) return st;

  NormModArgs n2{};
  n2.x = x1; n2.h = h2; n2.gain = w->norm2_g; n2.ada = w->ada; n2.temb = temb;
  n2.rows = rows; n2.D = D; n2.shift_chunk = 3; n2.scale_chunk = 4; n2.eps = d->norm_eps;
  n2.x_f32 = 1; n2.temb_stride = br.temb_stride;
  if ((st = device_status(launch_norm_mod(n2, s), "norm2+modulation")) != DIT_OK) return st;

  GemmArgs gu{};
  gu.A = h2; gu.W = w->w_gate_up; gu.C = act; gu.lda = D; gu.ldw = D; gu.ldc = m.ffn_ld;
  gu.N = F; gu.K = D; gu.rows = rows; gu.epilogue = EPI_SWIGLU; gu.up_offset = F;
  if ((st = device_status(launch_gemm(gu, s), "gate/up projection")) != DIT_OK) return st;

  GemmArgs gd{};
  gd.A = act; gd.W = w->w_down; gd.C = x_out; gd.lda = m.ffn_ld; gd.ldw = F; gd.ldc = D;
  gd.N = D; gd.K = F; gd.rows = rows; gd.epilogue = f32 ? EPI_GATED_F32_TO_F32 : EPI_GATED_F32_IN;
  gd.resid = x1; gd.ldr = D; gd.temb_stride = br.temb_stride;
  gd.ada = w->ada; gd.temb = temb; gd.chunk = 5;
  if ((st = device_status(launch_gemm(gd, s), "down projection")) != DIT_OK) return st;
  return DIT_OK;
}

int check_ws(void* ws, size_t ws_bytes, size_t need) {
  if (!ws) return fail(DIT_ERR_INVALID, "workspace is null");
  if (((uintptr_t)ws & (kAlign - 1)) != 0)
    return fail(DIT_ERR_INVALID, "workspace must be %zu-byte aligned", kAlign);
  if (ws_bytes < need)
    return fail(DIT_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu needed", ws_bytes,
                need);
  return DIT_OK;
}

}  // namespace

extern "C" {

const char* dit_last_error(void) { return g_err.c_str(); }

const char* dit_version(void) { return "avdit 0.1 (gfx950)"; }

int dit_cache_schedule(const dit_cache_policy* policy, int32_t n_intervals, uint8_t* step_hit) {
  g_err.clear();
  int st = check_policy(policy);
  if (st != DIT_OK) return st;
  if (n_intervals < 0) return fail(DIT_ERR_INVALID, "n_intervals must be >= 0");
  if (n_intervals > 0 && !step_hit) return fail(DIT_ERR_INVALID, "step_hit is null");
  schedule(policy, n_intervals, step_hit);
  return DIT_OK;
}

size_t dit_workspace_size(const dit_dims* dims, const dit_layout* layout, int32_t n_blocks,
                          dit_workspace_map* map) {
  g_err.clear();
  if (check_dims(dims) != DIT_OK || check_layout(layout) != DIT_OK) return 0;
  if (n_blocks < 0) {
    fail(DIT_ERR_INVALID, "n_blocks must be >= 0");
    return 0;
  }
  if (check_block_spans(dims, layout->seq_pad, layout->seq_pad) != DIT_OK) return 0;
  dit_workspace_map m;
  build_map(dims, layout, n_blocks, &m);
  if (map) *map = m;
  return m.total;
}

}  // extern "C"

namespace {

int block_forward_impl(const dit_dims* dims, const dit_layout* layout,
                       const dit_block_weights* weights, const float* temb, const void* x_in,
                       void* x_out, int32_t attn_mode, void* ws, size_t ws_bytes, void* stream,
                       bool f32) {
  g_err.clear();
  int st;
  if ((st = check_dims(dims)) != DIT_OK) return st;
  if ((st = check_layout(layout)) != DIT_OK) return st;
  if ((st = check_weights(weights, 0)) != DIT_OK) return st;
  if (!temb || !x_in || !x_out) return fail(DIT_ERR_INVALID, "temb, x_in and x_out must be non-null");
  if (attn_mode != DIT_ATTN_VALID_ONLY && attn_mode != DIT_ATTN_FIXED_VALID)
    return fail(DIT_ERR_INVALID, "attn_mode %d is not 0 (valid-only) or 1 (fixed-valid)", attn_mode);
  if ((st = check_aligned16(x_in, "x_in")) != DIT_OK) return st;
  if ((st = check_aligned16(x_out, "x_out")) != DIT_OK) return st;
  if ((st = check_aligned16(temb, "temb")) != DIT_OK) return st;
  if ((st = check_block_spans(dims, layout->seq_pad, layout->seq_pad)) != DIT_OK) return st;
  dit_workspace_map m;
  build_map(dims, layout, 0, &m);
  if ((st = check_ws(ws, ws_bytes, m.total)) != DIT_OK) return st;
  const size_t act_bytes = (size_t)layout->seq_pad * dims->hidden * (f32 ? 4 : 2);
  if (ranges_overlap(x_in, act_bytes, x_out, act_bytes) && act_bytes > 0)
    return fail(DIT_ERR_INVALID, "x_in and x_out overlap");
  if (act_bytes > 0 && (ranges_overlap(x_in, act_bytes, ws, m.total) ||
                        ranges_overlap(x_out, act_bytes, ws, m.total)))
    return fail(DIT_ERR_INVALID, "x_in or x_out overlaps the workspace");
  if (layout->seq_pad == 0) return DIT_OK;
  (void)hipGetLastError();
  return enqueue_block(dims, single_rows(layout), weights, temb, x_in, x_out, attn_mode,
                       static_cast<char*>(ws), m, static_cast<hipStream_t>(stream), f32);
}

}  // namespace

extern "C" {

int dit_block_forward(const dit_dims* dims, const dit_layout* layout,
                      const dit_block_weights* weights, const float* temb,
                      const uint16_t* x_in, uint16_t* x_out, int32_t attn_mode, void* ws,
                      size_t ws_bytes, void* stream) {
  return block_forward_impl(dims, layout, weights, temb, x_in, x_out, attn_mode, ws, ws_bytes,
                            stream, false);
}

int dit_block_forward_f32(const dit_dims* dims, const dit_layout* layout,
                          const dit_block_weights* weights, const float* temb, const float* x_in,
                          float* x_out, int32_t attn_mode, void* ws, size_t ws_bytes,
                          void* stream) {
  return block_forward_impl(dims, layout, weights, temb, x_in, x_out, attn_mode, ws, ws_bytes,
                            stream, true);
}

int step_update(float* x, const uint16_t* v, uint16_t* x_bf16, const dit_layout* layout,
                int32_t hidden, float dt_video, float dt_audio, void* stream) {
  g_err.clear();
  int st;
  if ((st = check_layout(layout)) != DIT_OK) return st;
  if (!x || !v) return fail(DIT_ERR_INVALID, "x and v must be non-null");
  if (hidden <= 0 || (hidden & 7) != 0)
    return fail(DIT_ERR_INVALID, "hidden %d must be a positive multiple of 8", hidden);
  if (!std::isfinite(dt_video) || !std::isfinite(dt_audio))
    return fail(DIT_ERR_INVALID, "step sizes must be finite");
  if ((((uintptr_t)x) & 15) || (((uintptr_t)v) & 15) || (((uintptr_t)x_bf16) & 15))
    return fail(DIT_ERR_INVALID, "x, v and x_bf16 must be 16-byte aligned");
  avdit::StepArgs a{};
  a.x = x; a.v = v; a.x_bf16 = x_bf16;
  a.rows = avdit::RowLayout{layout->n_video, layout->n_video + layout->n_audio, layout->seq_pad};
  a.D = hidden; a.dt_video = dt_video; a.dt_audio = dt_audio;
  (void)hipGetLastError();
  return device_status(avdit::launch_step_update(a, static_cast<hipStream_t>(stream)), "step update");
}

}  // extern "C"

namespace {

int loop_impl(const dit_dims* dims, const dit_layout* layout, const dit_block_weights* blocks,
              int32_t n_blocks, int32_t n_intervals, const float* sigmas_video,
              const float* sigmas_audio, const float* temb_steps, const dit_cache_policy* policy,
              float* x_latent, int32_t attn_mode, dit_loop_stats* stats, void* ws,
              size_t ws_bytes, void* stream, bool f32) {
  g_err.clear();
  int st;
  if ((st = check_dims(dims)) != DIT_OK) return st;
  if ((st = check_layout(layout)) != DIT_OK) return st;
  if ((st = check_policy(policy)) != DIT_OK) return st;
  if (n_blocks < 1) return fail(DIT_ERR_INVALID, "n_blocks must be >= 1");
  if (!blocks) return fail(DIT_ERR_INVALID, "blocks is null");
  for (int b = 0; b < n_blocks; ++b)
    if ((st = check_weights(&blocks[b], b)) != DIT_OK) return st;
  if (n_intervals < 0) return fail(DIT_ERR_INVALID, "n_intervals must be >= 0");
  if (n_intervals > 0 && (!sigmas_video || !sigmas_audio || !temb_steps))
    return fail(DIT_ERR_INVALID, "sigmas and temb_steps must be non-null");
  if (!x_latent) return fail(DIT_ERR_INVALID, "x_latent is null");
  if (((uintptr_t)x_latent) & 15) return fail(DIT_ERR_INVALID, "x_latent must be 16-byte aligned");
  if ((st = check_aligned16(temb_steps, "temb_steps")) != DIT_OK) return st;
  if ((st = check_block_spans(dims, layout->seq_pad, layout->seq_pad)) != DIT_OK) return st;
  if (attn_mode != DIT_ATTN_VALID_ONLY && attn_mode != DIT_ATTN_FIXED_VALID)
    return fail(DIT_ERR_INVALID, "attn_mode %d is not 0 (valid-only) or 1 (fixed-valid)", attn_mode);
  for (int i = 0; i <= n_intervals && n_intervals > 0; ++i)
    if (!std::isfinite(sigmas_video[i]) || !std::isfinite(sigmas_audio[i]))
      return fail(DIT_ERR_INVALID, "sigma %d is not finite", i);
  dit_workspace_map m;
  build_map(dims, layout, n_blocks, &m);
  if ((st = check_ws(ws, ws_bytes, m.total)) != DIT_OK) return st;
  const size_t lat_bytes = (size_t)layout->seq_pad * dims->hidden * 4;
  if (lat_bytes > 0 && ranges_overlap(x_latent, lat_bytes, ws, m.total))
    return fail(DIT_ERR_INVALID, "x_latent overlaps the workspace");

  // Request-scoped cache state: the schedule and the retained velocity live only here.
  std::vector<uint8_t> hits((size_t)n_intervals);
  schedule(policy, n_intervals, hits.data());
  int32_t n_hits = 0;
  for (uint8_t h : hits) n_hits += h;

  if (layout->seq_pad > 0 && n_intervals > 0) {
    (void)hipGetLastError();
    hipStream_t s = static_cast<hipStream_t>(stream);
    char* base = static_cast<char*>(ws);
    uint16_t* x_bf16 = reinterpret_cast<uint16_t*>(base + m.x_bf16);
    // the velocity of the last refresh lives in vel_buf[cur]; with extrapolation the one before
    // it is kept in the other buffer (request-scoped state, gone when this call returns)
    void* vel_buf[2] = {base + m.velocity, base + m.velocity_prev};
    int cur = 0;
    int32_t r_last = -1, r_prev = -1;
    const bool extrap = policy->mode == DIT_CACHE_EXTRAPOLATE;
    void* pp[2] = {base + m.ping, base + m.pong};
    const avdit::RowLayout rows{layout->n_video, layout->n_video + layout->n_audio, layout->seq_pad};
    const BlockRows brows = single_rows(layout);
    const size_t temb_step = (size_t)dims->n_mod * 6 * dims->hidden;

    // zero the latent's tail rows; the bf16 loop also takes the bf16 copy of x_0 (its DiT input)
    avdit::StepArgs first{};
    first.x = x_latent; first.x_bf16 = f32 ? nullptr : x_bf16; first.rows = rows;
    first.D = dims->hidden;
    if ((st = device_status(avdit::launch_step_update(first, s), "latent conversion")) != DIT_OK)
      return st;
    for (int32_t i = 0; i < n_intervals; ++i) {
      if (!hits[i]) {
        if (extrap && r_last >= 0) cur ^= 1;   // keep the previous refresh's velocity
        r_prev = r_last;
        r_last = i;
        void* vel = vel_buf[cur];
        const float* temb_i = temb_steps + (size_t)i * temb_step;
        for (int32_t b = 0; b < n_blocks; ++b) {
          // the fp32 loop feeds the latent itself to the first block
          const void* in = b > 0 ? pp[(b - 1) & 1] : (f32 ? (const void*)x_latent : (const void*)x_bf16);
          void* out = b == n_blocks - 1 ? vel : pp[b & 1];
          if ((st = enqueue_block(dims, brows, &blocks[b], temb_i, in, out, attn_mode, base, m, s,
                                  f32)) != DIT_OK)
            return st;
        }
      }
      avdit::StepArgs a{};
      a.x = x_latent;
      if (f32)
        a.v_f32 = static_cast<const float*>(vel_buf[cur]);
      else
        a.v = static_cast<const uint16_t*>(vel_buf[cur]);
      if (hits[i] && extrap && r_prev >= 0) {
        // first-order extrapolation in the interval index from refreshes r_prev < r_last
        a.lambda = (float)((double)(i - r_last) / (double)(r_last - r_prev));
        if (f32)
          a.v_prev_f32 = static_cast<const float*>(vel_buf[cur ^ 1]);
        else
          a.v_prev = static_cast<const uint16_t*>(vel_buf[cur ^ 1]);
      }
      a.x_bf16 = (!f32 && i + 1 < n_intervals) ? x_bf16 : nullptr;
      a.rows = rows; a.D = dims->hidden;
      a.dt_video = sigmas_video[i + 1] - sigmas_video[i];
      a.dt_audio = sigmas_audio[i + 1] - sigmas_audio[i];
      if ((st = device_status(avdit::launch_step_update(a, s), "step update")) != DIT_OK) return st;
    }
  }
  if (stats) {
    const int32_t calls = n_intervals - n_hits;
    const double V = (double)layout->n_video + layout->n_audio;
    const double D = dims->hidden, F = dims->ffn;
    stats->dit_calls = calls;
    stats->cache_hits = n_hits;
    stats->executed_blocks = (int64_t)calls * n_blocks;
    stats->skipped_blocks = (int64_t)n_hits * n_blocks;
    stats->useful_flops = (double)calls * n_blocks * (8 * V * D * D + 6 * V * D * F + 4 * V * V * D);
    if (stats->step_hit && n_intervals > 0) std::memcpy(stats->step_hit, hits.data(), hits.size());
  }
  return DIT_OK;
}

}  // namespace

extern "C" {

int denoise_loop(const dit_dims* dims, const dit_layout* layout,
                 const dit_block_weights* blocks, int32_t n_blocks, int32_t n_intervals,
                 const float* sigmas_video, const float* sigmas_audio,
                 const float* temb_steps, const dit_cache_policy* policy, float* x_latent,
                 int32_t attn_mode, dit_loop_stats* stats, void* ws, size_t ws_bytes,
                 void* stream) {
  return loop_impl(dims, layout, blocks, n_blocks, n_intervals, sigmas_video, sigmas_audio,
                   temb_steps, policy, x_latent, attn_mode, stats, ws, ws_bytes, stream, false);
}

int denoise_loop_f32(const dit_dims* dims, const dit_layout* layout,
                     const dit_block_weights* blocks, int32_t n_blocks, int32_t n_intervals,
                     const float* sigmas_video, const float* sigmas_audio,
                     const float* temb_steps, const dit_cache_policy* policy, float* x_latent,
                     int32_t attn_mode, dit_loop_stats* stats, void* ws, size_t ws_bytes,
                     void* stream) {
  return loop_impl(dims, layout, blocks, n_blocks, n_intervals, sigmas_video, sigmas_audio,
                   temb_steps, policy, x_latent, attn_mode, stats, ws, ws_bytes, stream, true);
}

}  // extern "C"

namespace {

// Validates a batch of request layouts and describes its rows; the combined layout has
// batch * seq_pad rows.
int batch_rows(const dit_layout* layouts, int32_t batch, BlockRows* out, dit_layout* combined) {
  if (!layouts) return fail(DIT_ERR_INVALID, "layouts is null");
  if (batch < 1 || batch > avdit::MAX_REQUESTS)
    return fail(DIT_ERR_INVALID, "batch %d outside [1, %d]", batch, (int)avdit::MAX_REQUESTS);
  int st;
  for (int b = 0; b < batch; ++b) {
    if ((st = check_layout(&layouts[b])) != DIT_OK) return st;
    if (layouts[b].seq_pad != layouts[0].seq_pad)
      return fail(DIT_ERR_INVALID, "request %d has seq_pad %d, request 0 has %d", b,
                  layouts[b].seq_pad, layouts[0].seq_pad);
  }
  const int32_t L = layouts[0].seq_pad;
  if (batch > 1 && L % 256 != 0)
    return fail(DIT_ERR_UNSUPPORTED, "a batch of requests needs seq_pad a multiple of 256 (got %d)", L);
  if ((int64_t)batch * L > kMaxSeq)
    return fail(DIT_ERR_INVALID, "batch x seq_pad = %lld rows is too many", (long long)batch * L);
  if (batch == 1) {
    *out = single_rows(&layouts[0]);
  } else {
    *out = BlockRows{};
    out->rows.seq_pad = L;
    out->rows.batch = batch;
    for (int b = 0; b < batch; ++b) {
      out->rows.req_video[b] = layouts[b].n_video;
      out->rows.req_valid[b] = layouts[b].n_video + layouts[b].n_audio;
      out->req_positions[b] = layouts[b].positions;
    }
  }
  *combined = dit_layout{0, 0, (int32_t)((int64_t)batch * L), nullptr};
  return DIT_OK;
}

}  // namespace

extern "C" {

size_t dit_workspace_size_batched(const dit_dims* dims, const dit_layout* layouts, int32_t batch,
                                  dit_workspace_map* map) {
  g_err.clear();
  BlockRows br;
  dit_layout all;
  if (check_dims(dims) != DIT_OK || batch_rows(layouts, batch, &br, &all) != DIT_OK) return 0;
  if (check_block_spans(dims, all.seq_pad, br.rows.seq_pad) != DIT_OK) return 0;
  dit_workspace_map m;
  build_map(dims, &all, 0, &m);
  if (map) *map = m;
  return m.total;
}

int dit_block_forward_batched(const dit_dims* dims, const dit_layout* layouts, int32_t batch,
                              const dit_block_weights* weights, const float* temb,
                              const uint16_t* x_in, uint16_t* x_out, int32_t attn_mode, void* ws,
                              size_t ws_bytes, void* stream) {
  g_err.clear();
  int st;
  BlockRows br;
  dit_layout all;
  if ((st = check_dims(dims)) != DIT_OK) return st;
  if ((st = batch_rows(layouts, batch, &br, &all)) != DIT_OK) return st;
  if ((st = check_weights(weights, 0)) != DIT_OK) return st;
  if (!temb || !x_in || !x_out) return fail(DIT_ERR_INVALID, "temb, x_in and x_out must be non-null");
  if (attn_mode != DIT_ATTN_VALID_ONLY && attn_mode != DIT_ATTN_FIXED_VALID)
    return fail(DIT_ERR_INVALID, "attn_mode %d is not 0 (valid-only) or 1 (fixed-valid)", attn_mode);
  if ((st = check_aligned16(x_in, "x_in")) != DIT_OK) return st;
  if ((st = check_aligned16(x_out, "x_out")) != DIT_OK) return st;
  if ((st = check_aligned16(temb, "temb")) != DIT_OK) return st;
  if ((st = check_block_spans(dims, all.seq_pad, br.rows.seq_pad)) != DIT_OK) return st;
  dit_workspace_map m;
  build_map(dims, &all, 0, &m);
  if ((st = check_ws(ws, ws_bytes, m.total)) != DIT_OK) return st;
  const size_t act_bytes = (size_t)all.seq_pad * dims->hidden * 2;
  if (act_bytes > 0 && ranges_overlap(x_in, act_bytes, x_out, act_bytes))
    return fail(DIT_ERR_INVALID, "x_in and x_out overlap");
  if (act_bytes > 0 && (ranges_overlap(x_in, act_bytes, ws, m.total) ||
                        ranges_overlap(x_out, act_bytes, ws, m.total)))
    return fail(DIT_ERR_INVALID, "x_in or x_out overlaps the workspace");
  if (all.seq_pad == 0) return DIT_OK;
  br.temb_stride = (int64_t)dims->n_mod * 6 * dims->hidden;
  (void)hipGetLastError();
  return enqueue_block(dims, br, weights, temb, x_in, x_out, attn_mode, static_cast<char*>(ws), m,
                       static_cast<hipStream_t>(stream));
}

int dit_attention_forward(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o,
                          int32_t batch, int32_t seq_pad, int32_t heads, int32_t head_dim,
                          int64_t batch_stride, int64_t row_stride, int64_t o_batch_stride,
                          int64_t o_row_stride, const int32_t* valid_lens, const float* q_gain,
                          const float* k_gain, int32_t attn_mode, void* stream) {
  g_err.clear();
  if (!q || !k || !v || !o || !valid_lens) return fail(DIT_ERR_INVALID, "null pointer argument");
  if ((q_gain == nullptr) != (k_gain == nullptr))
    return fail(DIT_ERR_INVALID, "q_gain and k_gain must both be given or both be NULL");
  if (batch < 1 || batch > avdit::ATTN_MAX_BATCH)
    return fail(DIT_ERR_INVALID, "batch %d outside [1, %d]", batch, (int)avdit::ATTN_MAX_BATCH);
  if (seq_pad < 0 || seq_pad > kMaxSeq) return fail(DIT_ERR_INVALID, "seq_pad %d out of range", seq_pad);
  if (heads < 1) return fail(DIT_ERR_INVALID, "heads must be >= 1");
  if (head_dim != 64 && head_dim != 128)
    return fail(DIT_ERR_UNSUPPORTED, "head_dim %d is not supported (64 or 128)", head_dim);
  const int64_t width = (int64_t)heads * head_dim;
  if (row_stride < width || o_row_stride < width || (row_stride & 7) || (o_row_stride & 7))
    return fail(DIT_ERR_INVALID, "row strides must be >= heads*head_dim and multiples of 8");
  if (batch > 1 && (batch_stride < (int64_t)seq_pad * row_stride ||
                    o_batch_stride < (int64_t)seq_pad * o_row_stride))
    return fail(DIT_ERR_INVALID, "batch strides must cover seq_pad rows");
  if ((batch_stride & 7) || (o_batch_stride & 7))
    return fail(DIT_ERR_INVALID, "batch strides must be multiples of 8");
  if ((((uintptr_t)q) | ((uintptr_t)k) | ((uintptr_t)v) | ((uintptr_t)o)) & 15)
    return fail(DIT_ERR_INVALID, "q, k, v and o must be 16-byte aligned");
  if ((((uintptr_t)q_gain) | ((uintptr_t)k_gain)) & 15)
    return fail(DIT_ERR_INVALID, "q_gain and k_gain must be 16-byte aligned");
  {
    const int st = check_span((int64_t)seq_pad * row_stride * 2, "one request's q/k/v rows");
    if (st != DIT_OK) return st;
  }
  if (attn_mode != DIT_ATTN_VALID_ONLY && attn_mode != DIT_ATTN_FIXED_VALID)
    return fail(DIT_ERR_INVALID, "attn_mode %d is not 0 (valid-only) or 1 (fixed-valid)", attn_mode);
  avdit::AttnArgs a{};
  for (int b = 0; b < batch; ++b) {
    if (valid_lens[b] < 0 || valid_lens[b] > seq_pad)
      return fail(DIT_ERR_INVALID, "valid_lens[%d] = %d outside [0, %d]", b, valid_lens[b], seq_pad);
    a.valid[b] = valid_lens[b];
  }
  a.q = q; a.k = k; a.v = v; a.o = o;
  a.batch_stride = batch_stride; a.row_stride = row_stride;
  a.o_batch_stride = o_batch_stride; a.o_row_stride = o_row_stride;
  a.batch = batch; a.seq_pad = seq_pad; a.heads = heads; a.head_dim = head_dim;
  a.fixed_valid = attn_mode == DIT_ATTN_FIXED_VALID ? 1 : 0;
  a.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)head_dim));
  a.q_gain = q_gain; a.k_gain = k_gain;
  (void)hipGetLastError();
  return device_status(avdit::launch_attention(a, static_cast<hipStream_t>(stream)), "attention");
}

}  // extern "C"

// ---------------------------------------------------------------------------------------
// Velocity head: final RMSNorm with the two-row indexed modulation, then one output
// projection per modality with an fp32 bias epilogue.
// ---------------------------------------------------------------------------------------
namespace {

constexpr int32_t kMaxOutChannels = 1 << 16;
// A projection to few channels carries little matrix work per k-tile, so one workgroup's walk
// over the reduction is a chain of load latencies: for C <= 256 the reduction is split four
// ways (fp32 partials in the workspace, summed in order by one reduction pass).
// workspace: the folded table, mul [2, D] then cst [2, C] (fp32)
size_t head_ws_bytes(const dit_dims* d, int32_t C) {
  return align_up((size_t)2 * d->hidden * 4) + align_up((size_t)2 * C * 4);
}

int head_impl(const dit_dims* dims, const dit_layout* layout, const dit_head_weights* hw,
              const float* temb, const void* x, float* v, void* ws, size_t ws_bytes,
              void* stream, bool f32) {
  using namespace avdit;
  g_err.clear();
  int st;
  if ((st = check_dims(dims)) != DIT_OK) return st;
  if ((st = check_layout(layout)) != DIT_OK) return st;
  if (!hw) return fail(DIT_ERR_INVALID, "head weights are null");
  if (!hw->norm_g || !hw->ada || !hw->w_out)
    return fail(DIT_ERR_INVALID, "the head has a null weight pointer");
  const int32_t C = hw->out_channels;
  if (C <= 0 || (C & 7) != 0 || C > kMaxOutChannels)
    return fail(DIT_ERR_INVALID, "out_channels %d must be a positive multiple of 8, at most %d", C,
                kMaxOutChannels);
  if (((uintptr_t)hw->bias & 15) != 0) return fail(DIT_ERR_INVALID, "bias must be 16-byte aligned");
  if (!temb || !x || !v) return fail(DIT_ERR_INVALID, "temb, x and v must be non-null");
  if ((((uintptr_t)x) & 15) || (((uintptr_t)v) & 15))
    return fail(DIT_ERR_INVALID, "x and v must be 16-byte aligned");
  if ((st = check_aligned16(temb, "temb")) != DIT_OK) return st;
  if ((st = check_aligned16(hw->norm_g, "norm_g")) != DIT_OK) return st;
  if ((st = check_aligned16(hw->ada, "ada")) != DIT_OK) return st;
  if ((st = check_aligned16(hw->w_out, "w_out")) != DIT_OK) return st;
  const size_t need = head_ws_bytes(dims, C);
  if ((st = check_ws(ws, ws_bytes, need)) != DIT_OK) return st;
  const int32_t D = dims->hidden, L = layout->seq_pad;
  const int32_t nv = layout->n_video, V = layout->n_video + layout->n_audio;
  const size_t xb = (size_t)L * D * (f32 ? 4 : 2), vb = (size_t)L * C * 4;
  if (L > 0 && (ranges_overlap(x, xb, v, vb) || ranges_overlap(x, xb, ws, need) ||
                ranges_overlap(v, vb, ws, need)))
    return fail(DIT_ERR_INVALID, "x, v and the workspace must not overlap");
  if (L == 0) return DIT_OK;
  (void)hipGetLastError();
  hipStream_t s = static_cast<hipStream_t>(stream);
  float* mul = static_cast<float*>(ws);
  float* cst = reinterpret_cast<float*>(static_cast<char*>(ws) + align_up((size_t)2 * D * 4));

  HeadPrepArgs p{};
  p.gain = hw->norm_g; p.ada = hw->ada; p.temb = temb; p.w = hw->w_out; p.bias = hw->bias;
  p.mul = mul; p.cst = cst; p.D = D; p.C = C;
  if ((st = device_status(launch_head_prep(p, s), "head table fold")) != DIT_OK) return st;

  // Both modalities in one launch, each over its own rows; the audio rows include the zero tail.
  HeadProjArgs a{};
  for (int m = 0; m < 2; ++m) {
    const int32_t r0 = m == 0 ? 0 : nv;
    a.x[m] = static_cast<const char*>(x) + (size_t)r0 * D * (f32 ? 4 : 2);
    a.v[m] = v + (size_t)r0 * C;
    a.w[m] = hw->w_out + (size_t)m * C * D;
    a.mul[m] = mul + (size_t)m * D;
    a.cst[m] = cst + (size_t)m * C;
    a.rows[m] = m == 0 ? nv : L - nv;
    a.valid[m] = m == 0 ? nv : V - nv;
  }
  a.D = D; a.C = C; a.ldv = C; a.eps = dims->norm_eps; a.x_f32 = f32 ? 1 : 0;
  if ((st = device_status(launch_head_proj(a, s), "head projection")) != DIT_OK) return st;
  return DIT_OK;
}

}  // namespace

extern "C" {

size_t dit_head_workspace_size(const dit_dims* dims, const dit_layout* layout,
                               int32_t out_channels) {
  g_err.clear();
  if (check_dims(dims) != DIT_OK || check_layout(layout) != DIT_OK) return 0;
  if (out_channels <= 0 || (out_channels & 7) != 0 || out_channels > kMaxOutChannels) {
    fail(DIT_ERR_INVALID, "out_channels %d must be a positive multiple of 8, at most %d",
         out_channels, kMaxOutChannels);
    return 0;
  }
  return head_ws_bytes(dims, out_channels);
}

int dit_velocity_head(const dit_dims* dims, const dit_layout* layout,
                      const dit_head_weights* head, const float* temb, const uint16_t* x,
                      float* v, void* ws, size_t ws_bytes, void* stream) {
  return head_impl(dims, layout, head, temb, x, v, ws, ws_bytes, stream, false);
}

int dit_velocity_head_f32(const dit_dims* dims, const dit_layout* layout,
                          const dit_head_weights* head, const float* temb, const float* x,
                          float* v, void* ws, size_t ws_bytes, void* stream) {
  return head_impl(dims, layout, head, temb, x, v, ws, ws_bytes, stream, true);
}

}  // extern "C"
