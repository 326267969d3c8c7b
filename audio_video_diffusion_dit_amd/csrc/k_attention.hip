// Flash-style softmax attention over the valid prefix of each packed request (TeleFuser PR #38,
// section 2: fixed-valid and valid-only attention modes, valid-only gather fused with the
// zero-tail merge).
//
// Design for gfx950:
//  * A workgroup (4 wave64s) owns 128 queries of one (request, head); each wave owns 32 queries
//    and keeps its Q fragments in registers for the whole key sweep.
//  * Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16 (K tile from
//    LDS as the A operand, Q as the B operand): each lane then holds 32 of the 64 scores of
//    one query per key tile, so the running max and sum need only one cross-lane exchange
//    (lanes l and l^32).
//  * O^T = V^T P^T reuses the score registers directly as the B operand: the k index of that
//    MFMA is mapped onto keys in the order the score layout already has, and V is written to
//    LDS transposed and in that same key order, so both operands are single 16-byte reads.
//  * K/V tiles of 64 keys are double buffered in LDS with one barrier per tile; the next
//    tile's global loads are in flight during the current tile's math.
//  * Valid-only mode bounds the key sweep by the request's valid length and query tiles that
//    lie wholly in the tail only write zeros. Fixed-valid mode sweeps the whole padded
//    length with a key mask. Keys at or past the valid length are loaded as zero and scored
//    -inf, so a fully masked tile leaves the running max, the sum and the accumulator
//    unchanged bit for bit: the two modes give identical outputs.
#include <math.h>

#include "common.hpp"
#include "kernels.hpp"

namespace avdit {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kQB = 128;  // queries per workgroup
constexpr int kKB = 64;   // keys per tile

// XOR swizzle of the 16-byte chunk index of a V^T row (row = head-dim index d).
__device__ __forceinline__ int vt_swz(int d) { return (d ^ (d >> 3)) & 7; }

// Position of key group g4 (keys 4 g4 .. 4 g4 + 3 of a 64-key tile) inside a V^T row: within
// each 16 keys the order is [0-3, 8-11, 4-7, 12-15], the order in which one score lane-half
// holds keys for the P V product.
__device__ __forceinline__ int vt_pos(int g4) {
  const int q4 = g4 & 3;
  return (g4 >> 2) * 16 + (((q4 & 1) << 1) | (q4 >> 1)) * 4;
}

template <int DH>
__global__ __launch_bounds__(256, 2) void k_attn(AttnArgs a) {
  constexpr int NC = DH / 8;        // 16-byte chunks per q/k row
  constexpr int QS = DH / 16;       // k-steps of the score MFMA
  constexpr int DT = DH / 32;       // 32-row tiles of O^T
  constexpr int KCH = kKB * NC;     // chunks in a K tile
  constexpr int KPT = KCH / 256;    // K chunks staged per thread
  constexpr int VIT = (16 * NC + 255) / 256;  // (key group, d chunk) items per thread

  __shared__ u32x4 ks[2][KCH];
  __shared__ u32x4 vts[2][DH * 8];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hh = lane >> 5;
  const int wave = tid >> 6;
  const int bq = blockIdx.z;
  const int head = blockIdx.y;
  const int q0 = blockIdx.x * kQB;
  const int V = a.valid[bq];
  const int L = a.seq_pad;

  const uint16_t* Q = a.q + (int64_t)bq * a.batch_stride + head * DH;
  const uint16_t* K = a.k + (int64_t)bq * a.batch_stride + head * DH;
  const uint16_t* Vp = a.v + (int64_t)bq * a.batch_stride + head * DH;
  uint16_t* O = a.o + (int64_t)bq * a.o_batch_stride + head * DH;

  if (V <= 0 || (!a.fixed_valid && q0 >= V)) {
    // nothing to attend: the whole query tile is tail
    for (int i = tid; i < kQB * NC; i += 256) {
      const int r = q0 + i / NC;
      if (r < L) *reinterpret_cast<u32x4*>(O + (int64_t)r * a.o_row_stride + (i % NC) * 8) =
          u32x4{0u, 0u, 0u, 0u};
    }
    return;
  }

  const int my_q = q0 + wave * 32 + l32;
  bf16x8 qf[QS];
#pragma unroll
  for (int s = 0; s < QS; ++s) {
    u32x4 w = u32x4{0u, 0u, 0u, 0u};
    if (my_q < V) w = *reinterpret_cast<const u32x4*>(Q + (int64_t)my_q * a.row_stride + (2 * s + hh) * 8);
    qf[s] = __builtin_bit_cast(bf16x8, w);
  }

  const int key_end = a.fixed_valid ? L : V;
  const int nkt = (key_end + kKB - 1) / kKB;

  u32x4 kst[KPT];
  u32x4 vst[VIT][4];
  auto load_tile = [&](int kt) {
    const int kv0 = kt * kKB;
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int q = tid + 256 * i;
      const int key = kv0 + q / NC;
      kst[i] = (key < V) ? *reinterpret_cast<const u32x4*>(K + (int64_t)key * a.row_stride + (q % NC) * 8)
                         : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int it = 0; it < VIT; ++it) {
      const int idx = tid + 256 * it;
      const int g4 = idx / NC, dc = idx % NC;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = kv0 + 4 * g4 + r;
        vst[it][r] = (idx < 16 * NC && key < V)
                         ? *reinterpret_cast<const u32x4*>(Vp + (int64_t)key * a.row_stride + dc * 8)
                         : u32x4{0u, 0u, 0u, 0u};
      }
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int q = tid + 256 * i;
      const int row = q / NC, c = q % NC;
      ks[buf][row * NC + (c ^ (row & (NC - 1)))] = kst[i];
    }
#pragma unroll
    for (int it = 0; it < VIT; ++it) {
      const int idx = tid + 256 * it;
      if (idx < 16 * NC) {
        const int g4 = idx / NC, dc = idx % NC;
        const int p = vt_pos(g4);
        u32x2* vt2 = reinterpret_cast<u32x2*>(vts[buf]);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          // element e of the 8-wide d chunk, for the 4 keys of the group
          const int wsel = e >> 1;
          const bool hi = e & 1;
          uint32_t k4[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const uint32_t w = vst[it][r][wsel];
            k4[r] = hi ? (w >> 16) : (w & 0xFFFFu);
          }
          const int d = dc * 8 + e;
          const int chunk = (p >> 3) ^ vt_swz(d);
          vt2[d * 16 + chunk * 2 + ((p & 7) >> 2)] = u32x2{k4[0] | (k4[1] << 16), k4[2] | (k4[3] << 16)};
        }
      }
    }
  };

  f32x16 oacc[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[t][e] = 0.0f;
  float m_run = -INFINITY;
  float l_run = 0.0f;
  const float c = a.scale_log2;

  load_tile(0);
  store_tile(0);
  __syncthreads();
  for (int kt = 0; kt < nkt; ++kt) {
    const int cur = kt & 1;
    const int kv0 = kt * kKB;
    if (kt + 1 < nkt) load_tile(kt + 1);

    // ---- S^T = K Q^T for 64 keys x 32 queries ----
    f32x16 sacc[2];
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
#pragma unroll
      for (int e = 0; e < 16; ++e) sacc[h2][e] = 0.0f;
#pragma unroll
      for (int s = 0; s < QS; ++s) {
        const int row = h2 * 32 + l32;
        const int ch = (2 * s + hh) ^ (row & (NC - 1));
        const bf16x8 kf = __builtin_bit_cast(bf16x8, ks[cur][row * NC + ch]);
        sacc[h2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[s], sacc[h2], 0, 0, 0);
      }
    }
    // element (j, i) of sacc[h2] is key kv0 + 32 h2 + 8 j + 4 hh + i
    if (kv0 + kKB > V) {
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int key = kv0 + h2 * 32 + (e >> 2) * 8 + 4 * hh + (e & 3);
          if (key >= V) sacc[h2][e] = -INFINITY;
        }
    }

    // ---- online softmax (base 2, scale folded into c) ----
    float mx = sacc[0][0];
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sacc[h2][e]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
    const float alpha = __builtin_amdgcn_exp2f((m_run - m_use) * c);
    m_run = m_new;
    const float mc = m_use * c;
    float psum = 0.0f;
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float p = __builtin_amdgcn_exp2f(fmaf(sacc[h2][e], c, -mc));
        sacc[h2][e] = p;
        psum += p;
      }
    l_run = fmaf(l_run, alpha, psum);
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int e = 0; e < 16; ++e) oacc[t][e] *= alpha;

    // ---- O^T += V^T P^T, 4 k-steps of 16 keys ----
#pragma unroll
    for (int ps = 0; ps < 4; ++ps) {
      const int h2 = ps >> 1;
      const int j0 = 2 * (ps & 1);
      const uint32_t p0 = pack_bf16x2(sacc[h2][4 * j0 + 0], sacc[h2][4 * j0 + 1]);
      const uint32_t p1 = pack_bf16x2(sacc[h2][4 * j0 + 2], sacc[h2][4 * j0 + 3]);
      const uint32_t p2 = pack_bf16x2(sacc[h2][4 * j0 + 4], sacc[h2][4 * j0 + 5]);
      const uint32_t p3 = pack_bf16x2(sacc[h2][4 * j0 + 6], sacc[h2][4 * j0 + 7]);
      const bf16x8 pf = __builtin_bit_cast(bf16x8, u32x4{p0, p1, p2, p3});
#pragma unroll
      for (int t = 0; t < DT; ++t) {
        const int d = t * 32 + l32;
        const int ch = (2 * ps + hh) ^ vt_swz(d);
        const bf16x8 vf = __builtin_bit_cast(bf16x8, vts[cur][d * 8 + ch]);
        oacc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf, oacc[t], 0, 0, 0);
      }
    }

    if (kt + 1 < nkt) store_tile(cur ^ 1);
    __syncthreads();
  }

  // ---- normalise and store: element (j, i) of oacc[t] is d = 32 t + 8 j + 4 hh + i ----
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const float inv_l = 1.0f / l_tot;
  if (my_q < L) {
    uint16_t* orow = O + (int64_t)my_q * a.o_row_stride;
    const bool valid = my_q < V;
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d = t * 32 + 8 * j + 4 * hh;
        u32x2 w = u32x2{0u, 0u};
        if (valid)
          w = u32x2{pack_bf16x2(oacc[t][4 * j] * inv_l, oacc[t][4 * j + 1] * inv_l),
                    pack_bf16x2(oacc[t][4 * j + 2] * inv_l, oacc[t][4 * j + 3] * inv_l)};
        *reinterpret_cast<u32x2*>(orow + d) = w;
      }
  }
}

hipError_t launch_attention(const AttnArgs& a, hipStream_t s) {
  if (a.batch <= 0 || a.batch > ATTN_MAX_BATCH || a.seq_pad < 0) return hipErrorInvalidValue;
  if ((a.row_stride & 7) != 0 || (a.o_row_stride & 7) != 0 || (a.batch_stride & 7) != 0 ||
      (a.o_batch_stride & 7) != 0)
    return hipErrorInvalidValue;
  if (a.seq_pad == 0) return hipSuccess;
  const dim3 grid((a.seq_pad + kQB - 1) / kQB, a.heads, a.batch);
  if (a.head_dim == 128) {
    hipLaunchKernelGGL(k_attn<128>, grid, dim3(256), 0, s, a);
  } else if (a.head_dim == 64) {
    hipLaunchKernelGGL(k_attn<64>, grid, dim3(256), 0, s, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace avdit
