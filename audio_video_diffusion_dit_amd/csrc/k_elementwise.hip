// HBM-bound kernels of the block and the loop: RMSNorm + indexed AdaLN modulation,
// per-head Q/K RMSNorm + NeoX RoPE, and the per-modality Euler update.
//
// Each is a single pass with 16-byte coalesced accesses and wavefront (or lane-group)
// reductions; all arithmetic is fp32 and every stored bf16 is rounded once.
#include "common.hpp"
#include "kernels.hpp"

namespace avdit {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------------------
// RMSNorm fused with indexed AdaLN modulation (TeleFuser PR #38, section 2; TeleFuser PR #23,
// "Changes Made": indexed modulation). The input is the bf16 block input (norm1) or the fp32
// mid-block residual (norm2). One wave owns a run of up to 8 consecutive rows and keeps the
// next row's loads (fp32 rows: the next two rows') in flight while it reduces the current one;
// the modulation of the current modality, folded to mul = g * (1 + scale) and add = shift,
// stays in registers and is reloaded only when the run crosses the video/audio boundary, so the
// tables cost little cache traffic per row. Shorter runs at short sequences keep enough waves in
// flight (a wave's rows are a chain of memory round trips).
// ---------------------------------------------------------------------------------------
// Rows per wave: 8, or fewer when 8 would leave under kNormWaves waves. Measured on the
// hidden-1024 block (4,608 rows): 3 rows per wave 9.0 us against 13.5 us for 8 (norm1); on
// the hidden-3072 block of 13,568 rows, 7 rows per wave was 1-4% faster than 8 and 4 rows
// 12-19% slower (every wave first loads its modulation rows, 60 KB at hidden 3072).
constexpr int kNormRowsPerWave = 8;
constexpr int kNormWaves = 2048;

// Row data as loaded: 8 elements per chunk, bf16 (one 16-byte word) or fp32 (two).
template <bool F32IN>
struct RowChunk {
  uint4 w[F32IN ? 2 : 1];
};

template <int CPL, bool F32IN>
__device__ __forceinline__ void load_row(const NormModArgs& a, int row, int lane, int nchunk,
                                         RowChunk<F32IN> (&r)[CPL]) {
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    const int c = lane + 64 * i;
#pragma unroll
    for (int h = 0; h < (F32IN ? 2 : 1); ++h) r[i].w[h] = zero4();
    if (c < nchunk) {
      if (F32IN) {
        const uint4* in = reinterpret_cast<const uint4*>(static_cast<const float*>(a.x) + (size_t)row * a.D);
        r[i].w[0] = in[2 * c];
        r[i].w[F32IN ? 1 : 0] = in[2 * c + 1];
      } else {
        const uint4* in = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.x) + (size_t)row * a.D);
        r[i].w[0] = in[c];
      }
    }
  }
}

template <bool F32IN>
__device__ __forceinline__ void unpack_chunk(const RowChunk<F32IN>& r, float (&x)[8]) {
  if (F32IN) {
    const uint32_t w[8] = {r.w[0].x, r.w[0].y, r.w[0].z, r.w[0].w,
                           r.w[F32IN ? 1 : 0].x, r.w[F32IN ? 1 : 0].y, r.w[F32IN ? 1 : 0].z, r.w[F32IN ? 1 : 0].w};
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = __uint_as_float(w[e]);
  } else {
    const uint32_t w[4] = {r.w[0].x, r.w[0].y, r.w[0].z, r.w[0].w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[2 * j] = bf_lo(w[j]);
      x[2 * j + 1] = bf_hi(w[j]);
    }
  }
}

template <int CPL, bool F32IN>  // CPL: 8-element chunks per lane, ceil(D / 512)
__global__ __launch_bounds__(256) void k_norm_mod(NormModArgs a, int rpw) {
  const int lane = threadIdx.x & 63;
  // wave-uniform (readfirstlane): the per-request lookups of a batch then become scalar loads,
  // whose wait does not drain the rows prefetched with vector loads
  const int wave = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (threadIdx.x >> 6));
  const int D = a.D;
  const int nchunk = D >> 3;
  const float inv_d = 1.0f / (float)D;
  float mul[CPL][8];
  float add[CPL][8];
  int cur = -1;   // (request, modality) whose modulation the registers hold
  const int rows_total = total_rows(a.rows);
  const int row0 = wave * rpw;
  if (row0 >= rows_total) return;

  // software pipeline: the next row's loads are in flight while the current row is reduced
  // (fp32 rows: two rows ahead, which measured 4% faster on the 32k-token block; bf16 rows: one)
  constexpr int AHEAD = F32IN ? 2 : 1;
  RowChunk<F32IN> buf[CPL], nxt[CPL], nx2[CPL];
  if (row_info(a.rows, row0).valid) load_row<CPL, F32IN>(a, row0, lane, nchunk, buf);
  if constexpr (AHEAD == 2) {
    if (row0 + 1 < rows_total && row_info(a.rows, row0 + 1).valid)
      load_row<CPL, F32IN>(a, row0 + 1, lane, nchunk, nxt);
  }
  for (int rr = 0; rr < rpw; ++rr) {
    const int row = row0 + rr;
    if (row >= rows_total) return;
    const RowInfo ri = row_info(a.rows, row);
    if (rr + AHEAD < rpw && row + AHEAD < rows_total &&
        row_info(a.rows, row + AHEAD).valid)
      load_row<CPL, F32IN>(a, row + AHEAD, lane, nchunk, AHEAD == 2 ? nx2 : nxt);
    uint4* out = reinterpret_cast<uint4*>(a.h + (size_t)row * D);
    if (!ri.valid) {
#pragma unroll
      for (int i = 0; i < CPL; ++i) {
        const int c = lane + 64 * i;
        if (c < nchunk) out[c] = zero4();
      }
    } else {
      const int m = ri.mod;
      if (ri.req * 2 + m != cur) {
        cur = ri.req * 2 + m;
        const float* A = a.ada + (size_t)m * a.table_rows * D;
        const float* T = a.temb + ri.req * a.temb_stride + (size_t)m * a.table_rows * D;
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
          const int c = lane + 64 * i;
          if (c < nchunk) {
            const int d0 = c * 8;
#pragma unroll
            for (int e = 0; e < 8; e += 4) {
              const float4 g = *reinterpret_cast<const float4*>(a.gain + d0 + e);
              const float4 sa = *reinterpret_cast<const float4*>(A + a.scale_chunk * D + d0 + e);
              const float4 st = *reinterpret_cast<const float4*>(T + a.scale_chunk * D + d0 + e);
              const float4 ha = *reinterpret_cast<const float4*>(A + a.shift_chunk * D + d0 + e);
              const float4 ht = *reinterpret_cast<const float4*>(T + a.shift_chunk * D + d0 + e);
              mul[i][e + 0] = g.x * (1.0f + (sa.x + st.x));
              mul[i][e + 1] = g.y * (1.0f + (sa.y + st.y));
              mul[i][e + 2] = g.z * (1.0f + (sa.z + st.z));
              mul[i][e + 3] = g.w * (1.0f + (sa.w + st.w));
              add[i][e + 0] = ha.x + ht.x;
              add[i][e + 1] = ha.y + ht.y;
              add[i][e + 2] = ha.z + ht.z;
              add[i][e + 3] = ha.w + ht.w;
            }
          }
        }
      }
      float ss = 0.0f;
#pragma unroll
      for (int i = 0; i < CPL; ++i) {
        float x[8];
        unpack_chunk<F32IN>(buf[i], x);
#pragma unroll
        for (int e = 0; e < 8; ++e) ss = fmaf(x[e], x[e], ss);
      }
      ss = wave_sum(ss);
      const float r = rsqrtf(ss * inv_d + a.eps);
#pragma unroll
      for (int i = 0; i < CPL; ++i) {
        const int c = lane + 64 * i;
        if (c < nchunk) {
          float x[8];
          unpack_chunk<F32IN>(buf[i], x);
          uint32_t o[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float y0 = fmaf(x[2 * j] * r, mul[i][2 * j], add[i][2 * j]);
            const float y1 = fmaf(x[2 * j + 1] * r, mul[i][2 * j + 1], add[i][2 * j + 1]);
            o[j] = pack_bf16x2(y0, y1);
          }
          out[c] = make_uint4(o[0], o[1], o[2], o[3]);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      buf[i] = nxt[i];
      if constexpr (AHEAD == 2) nxt[i] = nx2[i];
    }
  }
}

template <int CPL>
static hipError_t norm_mod_instance(const NormModArgs& a, hipStream_t s) {
  const int rows = total_rows(a.rows);
  // rows per wave: up to 8, fewer when that leaves under kNormWaves waves
  int rpw = (rows + kNormWaves - 1) / kNormWaves;
  rpw = rpw < 1 ? 1 : (rpw > kNormRowsPerWave ? kNormRowsPerWave : rpw);
  const int waves = (rows + rpw - 1) / rpw;
  const int blocks = (waves + 3) / 4;
  if (blocks == 0) return hipSuccess;
  if (a.x_f32)
    hipLaunchKernelGGL((k_norm_mod<CPL, true>), dim3(blocks), dim3(256), 0, s, a, rpw);
  else
    hipLaunchKernelGGL((k_norm_mod<CPL, false>), dim3(blocks), dim3(256), 0, s, a, rpw);
  return hipGetLastError();
}

hipError_t launch_norm_mod(const NormModArgs& a, hipStream_t s) {
  if (a.D <= 0 || (a.D & 7) != 0) return hipErrorInvalidValue;
  const int cpl = (a.D / 8 + 63) / 64;
  if (cpl <= 1) return norm_mod_instance<1>(a, s);
  if (cpl <= 2) return norm_mod_instance<2>(a, s);
  if (cpl <= 4) return norm_mod_instance<4>(a, s);
  if (cpl <= 6) return norm_mod_instance<6>(a, s);
  if (cpl <= 8) return norm_mod_instance<8>(a, s);
  if (cpl <= 12) return norm_mod_instance<12>(a, s);
  if (cpl <= 16) return norm_mod_instance<16>(a, s);
  return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------------------
// Per-head Q/K RMSNorm + NeoX rotary embedding (TeleFuser PR #38, section 2; TeleFuser
// PR #23, "Changes Made"). A group of head_dim/8 lanes owns one token: lane j holds
// elements 8j..8j+7 of a head vector, so the rotate-half partner of lane j is lane
// j ^ (group/2). The token's rotation angles are computed once (one sincos per element
// slot) and reused for all 2H vectors (q heads then k heads, contiguous in qkv); at short
// sequences the vectors of a token are split over gridDim.y lane groups (each computing the
// angles again) so that enough waves are in flight.
// ---------------------------------------------------------------------------------------
template <int DH>
__global__ __launch_bounds__(256) void k_qk_norm_rope(QkNormRopeArgs a) {
  constexpr int G = DH / 8;         // lanes per head vector
  constexpr int HALF_G = G / 2;
  constexpr int TPB = 256 / G;      // tokens per block
  const int gl = threadIdx.x % G;
  const int token = blockIdx.x * TPB + threadIdx.x / G;
  if (token >= total_rows(a.rows)) return;
  const RowInfo ri = row_info(a.rows, token);
  if (!ri.valid) return;

  const int32_t* positions = a.rows.batch > 1 ? a.req_positions[ri.req] : a.positions;
  const float pos = positions ? (float)positions[ri.idx] : (float)ri.idx;
  const int gg = gl % HALF_G;       // frequency block of this lane: i = 8 * gg + e
  float inv[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) inv[e] = 0.0f;
#pragma unroll
  for (int b = 0; b < HALF_G; ++b) {
#pragma unroll
    for (int e = 0; e < 8; ++e) inv[e] = (gg == b) ? a.inv_freq[8 * b + e] : inv[e];
  }
  float cs[8], sn[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) sincosf(pos * inv[e], &sn[e], &cs[e]);

  float gq[8], gk[8];
#pragma unroll
  for (int e = 0; e < 8; e += 4) {
    const float4 q4 = *reinterpret_cast<const float4*>(a.q_gain + gl * 8 + e);
    const float4 k4 = *reinterpret_cast<const float4*>(a.k_gain + gl * 8 + e);
    gq[e] = q4.x; gq[e + 1] = q4.y; gq[e + 2] = q4.z; gq[e + 3] = q4.w;
    gk[e] = k4.x; gk[e + 1] = k4.y; gk[e + 2] = k4.z; gk[e + 3] = k4.w;
  }
  const bool first_half = gl < HALF_G;
  const float inv_dh = 1.0f / (float)DH;
  uint16_t* base = a.qkv + (size_t)token * a.row_stride + gl * 8;
  const int nvec = 2 * a.heads;

  constexpr int U = 8;
  // this lane group's vectors: a contiguous share of whole U-vector chunks
  const int chunks = (nvec + U - 1) / U;
  const int per = (chunks + (int)gridDim.y - 1) / (int)gridDim.y;
  const int v_begin = (int)blockIdx.y * per * U;
  const int v_end = v_begin + per * U < nvec ? v_begin + per * U : nvec;
  for (int v0 = v_begin; v0 < v_end; v0 += U) {
    uint4 raw[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
      raw[u] = (v0 + u < v_end) ? *reinterpret_cast<const uint4*>(base + (size_t)(v0 + u) * DH)
                                : zero4();
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int vec = v0 + u;
      const uint32_t w[4] = {raw[u].x, raw[u].y, raw[u].z, raw[u].w};
      float x[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        x[2 * j] = bf_lo(w[j]);
        x[2 * j + 1] = bf_hi(w[j]);
      }
      float ss = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) ss = fmaf(x[e], x[e], ss);
      ss = group_sum<G>(ss);
      const float r = rsqrtf(ss * inv_dh + a.eps);
      const bool is_q = vec < a.heads;
      float y[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) y[e] = x[e] * r * (is_q ? gq[e] : gk[e]);
      uint32_t o[4];
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const float p0 = __shfl_xor(y[e], HALF_G, 64);
        const float p1 = __shfl_xor(y[e + 1], HALF_G, 64);
        const float r0 = first_half ? fmaf(y[e], cs[e], -p0 * sn[e]) : fmaf(y[e], cs[e], p0 * sn[e]);
        const float r1 = first_half ? fmaf(y[e + 1], cs[e + 1], -p1 * sn[e + 1])
                                    : fmaf(y[e + 1], cs[e + 1], p1 * sn[e + 1]);
        o[e / 2] = pack_bf16x2(r0, r1);
      }
      if (vec < v_end)
        *reinterpret_cast<uint4*>(base + (size_t)vec * DH) = make_uint4(o[0], o[1], o[2], o[3]);
    }
  }
}

// Lane groups per token: enough to reach kQkWaves waves, at most one per 8-vector chunk
// (measured: 15.2 -> 13.0 us at 4,608 tokens x 16 vectors, 64.5 -> 57.2 us at 13,440 x 48;
// the 32k-token launch already has 8192 waves and keeps one group per token).
constexpr int kQkWaves = 8192;

hipError_t launch_qk_norm_rope(const QkNormRopeArgs& a, hipStream_t s) {
  if ((a.row_stride & 7) != 0) return hipErrorInvalidValue;
  // one request: the valid rows; a batch: every row (invalid ones return at once)
  const int n = a.rows.batch > 1 ? total_rows(a.rows) : a.rows.n_valid;
  if (n <= 0) return hipSuccess;
  if (a.head_dim != 128 && a.head_dim != 64) return hipErrorInvalidValue;
  const int tpb = 256 / (a.head_dim / 8);  // tokens per block
  const int blocks = (n + tpb - 1) / tpb;
  // split a token's 8-vector chunks over more lane groups while the grid has fewer than
  // kQkWaves waves
  const int chunks = (2 * a.heads + 7) / 8;
  int split = (kQkWaves + 4 * blocks - 1) / (4 * blocks);
  split = split < 1 ? 1 : (split > chunks ? chunks : split);
  const dim3 grid(blocks, split);
  if (a.head_dim == 128)
    hipLaunchKernelGGL(k_qk_norm_rope<128>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(k_qk_norm_rope<64>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------
// Flow-matching Euler update with per-modality step sizes (TeleFuser PR #23, "Motivation"
// and "Changes Made": independent video/audio schedulers, optimized scheduler updates).
// One thread per 8 consecutive elements of a row and one pass over the grid (no grid-stride
// loop), with non-temporal loads and stores: this streaming pattern measured 6.1-6.3 TB/s on
// a plain copy against 4.7-4.9 TB/s for a grid-stride loop. The bf16 copy is the next DiT input
// of the bf16-residual loop; the fp32-residual loop takes an fp32 velocity and no copy.
// ---------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_step_update(StepArgs a) {
  const int per_row = a.D >> 3;
  const long total = (long)a.rows.seq_pad * per_row;
  const long idx = (long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= total) return;
  const int row = (int)(idx / per_row);
  const int c = (int)(idx - (long)row * per_row);
  f32x4* xp = reinterpret_cast<f32x4*>(a.x + (size_t)row * a.D + 8 * c);
  u32x4* bp = a.x_bf16 ? reinterpret_cast<u32x4*>(a.x_bf16 + (size_t)row * a.D + 8 * c) : nullptr;
  if (row >= a.rows.n_valid) {
    __builtin_nontemporal_store(f32x4{0.f, 0.f, 0.f, 0.f}, xp);
    __builtin_nontemporal_store(f32x4{0.f, 0.f, 0.f, 0.f}, xp + 1);
    if (bp) __builtin_nontemporal_store(u32x4{0u, 0u, 0u, 0u}, bp);
    return;
  }
  f32x4 x0 = __builtin_nontemporal_load(xp), x1 = __builtin_nontemporal_load(xp + 1);
  if (a.v || a.v_f32) {
    const float dt = row < a.rows.n_video ? a.dt_video : a.dt_audio;
    f32x4 v0, v1;
    if (a.v) {
      const u32x4 vv = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4*>(a.v + (size_t)row * a.D + 8 * c));
      v0 = f32x4{bf_lo(vv.x), bf_hi(vv.x), bf_lo(vv.y), bf_hi(vv.y)};
      v1 = f32x4{bf_lo(vv.z), bf_hi(vv.z), bf_lo(vv.w), bf_hi(vv.w)};
    } else {
      const f32x4* vp = reinterpret_cast<const f32x4*>(a.v_f32 + (size_t)row * a.D + 8 * c);
      v0 = __builtin_nontemporal_load(vp);
      v1 = __builtin_nontemporal_load(vp + 1);
    }
    if (a.v_prev || a.v_prev_f32) {
      // first-order extrapolation from the last two refreshes: u = v + lambda (v - v_prev)
      f32x4 p0, p1;
      if (a.v_prev) {
        const u32x4 pp = __builtin_nontemporal_load(
            reinterpret_cast<const u32x4*>(a.v_prev + (size_t)row * a.D + 8 * c));
        p0 = f32x4{bf_lo(pp.x), bf_hi(pp.x), bf_lo(pp.y), bf_hi(pp.y)};
        p1 = f32x4{bf_lo(pp.z), bf_hi(pp.z), bf_lo(pp.w), bf_hi(pp.w)};
      } else {
        const f32x4* pq = reinterpret_cast<const f32x4*>(a.v_prev_f32 + (size_t)row * a.D + 8 * c);
        p0 = __builtin_nontemporal_load(pq);
        p1 = __builtin_nontemporal_load(pq + 1);
      }
      const float l = a.lambda;
      v0 = f32x4{fmaf(l, v0.x - p0.x, v0.x), fmaf(l, v0.y - p0.y, v0.y),
                 fmaf(l, v0.z - p0.z, v0.z), fmaf(l, v0.w - p0.w, v0.w)};
      v1 = f32x4{fmaf(l, v1.x - p1.x, v1.x), fmaf(l, v1.y - p1.y, v1.y),
                 fmaf(l, v1.z - p1.z, v1.z), fmaf(l, v1.w - p1.w, v1.w)};
    }
    x0.x = fmaf(dt, v0.x, x0.x);
    x0.y = fmaf(dt, v0.y, x0.y);
    x0.z = fmaf(dt, v0.z, x0.z);
    x0.w = fmaf(dt, v0.w, x0.w);
    x1.x = fmaf(dt, v1.x, x1.x);
    x1.y = fmaf(dt, v1.y, x1.y);
    x1.z = fmaf(dt, v1.z, x1.z);
    x1.w = fmaf(dt, v1.w, x1.w);
    __builtin_nontemporal_store(x0, xp);
    __builtin_nontemporal_store(x1, xp + 1);
  }
  if (bp)
    __builtin_nontemporal_store(u32x4{pack_bf16x2(x0.x, x0.y), pack_bf16x2(x0.z, x0.w),
                                      pack_bf16x2(x1.x, x1.y), pack_bf16x2(x1.z, x1.w)}, bp);
}

hipError_t launch_step_update(const StepArgs& a, hipStream_t s) {
  if (a.D <= 0 || (a.D & 7) != 0) return hipErrorInvalidValue;
  const long total = (long)a.rows.seq_pad * (a.D >> 3);
  if (total == 0) return hipSuccess;
  const long blocks = (total + 255) / 256;
  if (blocks > 0x7FFFFFFFL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_step_update, dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace avdit
