// Flash-style softmax attention over the valid prefix of each packed request (TeleFuser PR #38,
// section 2: fixed-valid and valid-only attention modes, valid-only gather fused with the
// zero-tail merge).
//
// Design for gfx950:
//  * A workgroup (8 wave64s, one per CU, two waves per SIMD) owns 256 queries of one (request,
//    head); workgroups are remapped so that the query tiles of one head run on one XCD (K/V
//    fetched once per head). Each wave owns 32 queries and keeps its Q fragments in registers
//    for the whole key sweep; each K/V tile is staged into LDS once for all 256 queries (two
//    workgroups of 128 queries per CU staged every tile twice: 5.6% slower).
//  * Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16 (K tile from
//    LDS as the A operand, Q as the B operand): each lane then holds 32 of the 64 scores of
//    one query per key tile, so the running max needs one cross-lane exchange (lanes l, l^32: one v_permlane32_swap).
//  * O^T = V^T P^T reuses the score registers directly as the B operand: the k index of that
//    MFMA is mapped onto keys in the order the score layout already has. V stays row-major in
//    LDS, like K, and its A-operand fragments are assembled by the LDS transpose read
//    (ds_read_b64_tr_b16): within 16 lanes it turns four 4-element row pieces into four
//    4-key columns, so V needs no transposition work on the way in.
//  * K/V tiles of 64 keys go straight from memory into LDS (buffer loads with the LDS
//    destination, no staging registers); the resource range ends at the request's valid
//    length, so keys past it read as zero. Tiles are double buffered with one barrier per
//    tile, and the next tile's loads are in flight during the current tile's math. The key
//    loop is unrolled by two so that both LDS buffers are addressed with immediate offsets.
//    The first tiles are issued before the Q fragments and the gains are loaded, so that the
//    prologue waits for memory once rather than once per operand.
//  * Only the last partial tile (and, in fixed-valid mode, the tiles past the valid length)
//    run the masking code.
//  * Softmax shift: q and k of the DiT block come out of the per-head Q/K RMSNorm, so every
//    logit is bounded by max|gq| max|gk| sqrt(Dh) (a normalised head vector has norm below
//    sqrt(Dh)). When the caller passes the gains and that bound B, in log2 units, is small, no
//    running row maximum is needed: for 30 < B <= 60 the probabilities are exp2(s c - B), within
//    [2^-121, 1]; for B <= 30 no shift is needed at all (softmax is scale invariant): the factor
//    c = log2(e)/sqrt(Dh) is folded into the Q fragments once per wave, so the score MFMAs yield
//    log2-unit logits and a probability is a bare exp2 of the score, within [2^-31, 2^31]. The
//    extra bf16 rounding of q c moves a logit by under 0.005 in log2 units at such bounds (it
//    grows with the logits, which is why larger bounds keep c in fp32). Either way the per-tile
//    max reduction, cross-lane exchange and rescale disappear, and the row sum is taken from the
//    bf16 probabilities the P V product uses (v_dot2c_f32_bf16). Otherwise the exact running
//    maximum is kept, with the accumulator rescale run only on tiles where some row's maximum
//    grew.
//  * Valid-only mode bounds the key sweep by the request's valid length and query tiles that
//    lie wholly in the tail only write zeros. Fixed-valid mode sweeps the whole padded
//    length with a key mask. A fully masked tile leaves the running max, the sum and the
//    accumulator unchanged bit for bit, so the two modes give identical outputs.
#include <math.h>

#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace avdit {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) char lds_char;

constexpr int kQB = 256;                    // queries per workgroup
constexpr int kNW = kQB / 32;               // waves per workgroup
constexpr int kKB = 64;                     // keys per tile
constexpr int kKPF = 4;                     // K fragments read ahead in the score phase
constexpr int kVPF = 4;                     // V fragments read ahead in the P V phase
constexpr int32_t kAttnRsrcWord3 = 0x00020000;

// 16-byte-chunk XOR swizzle of a K row: 16 consecutive rows read at one logical chunk hit
// distinct banks (rows are 256 bytes at head_dim 128, 128 bytes at 64).
template <int DH>
__device__ __forceinline__ int kswz(int row) {
  return DH == 128 ? (row & 15) : ((row ^ (row >> 3)) & 7);
}
// Swizzle of a V row for the transpose reads: the 4 key rows x 32 bytes that one pair of
// 16-lane groups reads land on 16 distinct 16-byte bank groups.
template <int DH>
__device__ __forceinline__ int vswz(int key) {
  return DH == 128 ? 4 * (key & 3) : 4 * ((key >> 1) & 1);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t attn_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes,
                                           kAttnRsrcWord3);
}

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

// Raw buffer resource as four SGPR words: base, range in bytes, 32-bit-element format.
__device__ __forceinline__ i32x4 attn_rsrc_words(const void* p, uint32_t bytes) {
  const uint64_t ad = reinterpret_cast<uint64_t>(p);
  return i32x4{(int32_t)(uint32_t)ad, (int32_t)(uint32_t)(ad >> 32), (int32_t)bytes, kAttnRsrcWord3};
}

// One 16-byte-per-lane buffer load written straight into LDS: lane l's chunk lands at LDS byte
// address lds_base + 16 l (lds_base uniform across the wave). Offsets past the resource range
// read as zero. Issued as inline assembly so that the compiler does not serialise later LDS
// reads behind it; completion is awaited explicitly with s_waitcnt vmcnt before the barrier
// that publishes the tile.
__device__ __forceinline__ void dma_b128(uint32_t lds_base, uint32_t voffset, i32x4 rsrc) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(lds_base), "v"(voffset), "s"(rsrc)
               : "memory", "m0");
}

// Max and sum of the values of lanes l and l ^ 32, from one v_permlane32_swap (no LDS round
// trip): the swap leaves lanes l and l + 32 holding {x[l], x[l + 32]} in its two results.
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int DH>
__global__ __launch_bounds__(64 * kNW, 1) void k_attn(AttnArgs a) {
  constexpr int NC = DH / 8;          // 16-byte chunks per K/V row
  constexpr int QS = DH / 16;         // k-steps of the score MFMA
  constexpr int DT = DH / 32;         // 32-row tiles of O^T
  constexpr int TILE = kKB * NC;      // 16-byte chunks per K (or V) tile
  constexpr int LPT = TILE / (64 * kNW);  // chunks each thread stages per operand per tile
  constexpr int VOFF = TILE * 16;     // byte offset of the V tile inside a buffer
  constexpr int BUFB = 2 * TILE * 16; // bytes per buffer

  __shared__ u32x4 smem[2 * 2 * TILE];  // [buffer][K tile | V tile]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hh = lane >> 5;
  const int wave = tid >> 6;
  // Workgroup ids are dealt round-robin over the 8 XCDs; remap them so that each XCD receives a
  // contiguous range of (head, request, query-tile) triples, query tile fastest: the query
  // tiles of one (request, head) then run on one XCD and share its K/V tiles in that XCD's L2,
  // and with the request varying faster than the head each XCD's range mixes the requests of a
  // ragged batch, so short and long requests spread evenly over the XCDs.
  const int n_qt = gridDim.x;
  const int total = gridDim.x * gridDim.y * gridDim.z;
  const int b_lin = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
  const int xcd = b_lin & 7, local = b_lin >> 3;
  const int per = total >> 3, rem = total & 7;
  const int logical = xcd * per + (xcd < rem ? xcd : rem) + local;
  const int qt = logical % n_qt;
  const int pair = logical / n_qt;
  const int bq = pair % gridDim.z;
  const int head = pair / gridDim.z;
  const int q0 = qt * kQB;
  const int V = a.valid[bq];
  const int L = a.seq_pad;

  const uint16_t* Q = a.q + (int64_t)bq * a.batch_stride + head * DH;
  const uint16_t* K = a.k + (int64_t)bq * a.batch_stride + head * DH;
  const uint16_t* Vp = a.v + (int64_t)bq * a.batch_stride + head * DH;
  uint16_t* O = a.o + (int64_t)bq * a.o_batch_stride + head * DH;

  if (V <= 0 || (!a.fixed_valid && q0 >= V)) {
    // nothing to attend: the whole query tile is tail
    for (int i = tid; i < kQB * NC; i += 64 * kNW) {
      const int r = q0 + i / NC;
      if (r < L) *reinterpret_cast<u32x4*>(O + (int64_t)r * a.o_row_stride + (i % NC) * 8) =
          u32x4{0u, 0u, 0u, 0u};
    }
    return;
  }

  // ---- global -> LDS staging: wave w's i-th load fills 16-byte slots (kNW i + w) * 64 + lane of
  // a tile, i.e. row p / NC and physical chunk p % NC of slot p; the lane fetches the logical
  // chunk that the swizzle places there. Keys >= V read as zero (resource range). ----
  const uint32_t span = (uint32_t)((int64_t)V * a.row_stride * 2);
  const i32x4 rs_k = attn_rsrc_words(K, span);
  const i32x4 rs_v = attn_rsrc_words(Vp, span);
  const uint32_t tile_bytes = (uint32_t)(kKB * a.row_stride * 2);
  // At head_dim 128 successive loads of a wave are 32 rows apart and both swizzles have period
  // 16 in the row, so one offset per operand plus a uniform stride covers them.
  constexpr int GK = (DH == 128) ? 1 : LPT;
  uint32_t goff_k[GK], goff_v[GK];
#pragma unroll
  for (int i = 0; i < GK; ++i) {
    const int p = (kNW * i + wave) * 64 + lane;
    const int row = p / NC, pc = p % NC;
    goff_k[i] = (uint32_t)(row * a.row_stride * 2 + (pc ^ kswz<DH>(row)) * 16);
    goff_v[i] = (uint32_t)(row * a.row_stride * 2 + (pc ^ vswz<DH>(row)) * 16);
  }
  const uint32_t gstep = (uint32_t)(kNW * 64 / NC * a.row_stride * 2);  // rows between loads
  lds_char* lds = (lds_char*)(smem);  // __shared__ array viewed in the LDS address space
  const uint32_t lds0 = (uint32_t)__builtin_amdgcn_readfirstlane(
      (int)(uint32_t)(uintptr_t)lds + wave * 1024);
  auto load_tile = [&](int kt, int buf) {
    const uint32_t g = (uint32_t)kt * tile_bytes;
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const uint32_t ok = (DH == 128) ? goff_k[0] + i * gstep : goff_k[i % GK];
      const uint32_t ov = (DH == 128) ? goff_v[0] + i * gstep : goff_v[i % GK];
      dma_b128(lds0 + buf * BUFB + i * (kNW * 1024), g + ok, rs_k);
      dma_b128(lds0 + buf * BUFB + VOFF + i * (kNW * 1024), g + ov, rs_v);
    }
  };
  auto load_k = [&](int kt, int buf) __attribute__((always_inline)) {
    const uint32_t g = (uint32_t)kt * tile_bytes;
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const uint32_t ok = (DH == 128) ? goff_k[0] + i * gstep : goff_k[i % GK];
      dma_b128(lds0 + buf * BUFB + i * (kNW * 1024), g + ok, rs_k);
    }
  };
  auto load_v = [&](int kt, int buf) __attribute__((always_inline)) {
    const uint32_t g = (uint32_t)kt * tile_bytes;
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const uint32_t ov = (DH == 128) ? goff_v[0] + i * gstep : goff_v[i % GK];
      dma_b128(lds0 + buf * BUFB + VOFF + i * (kNW * 1024), g + ov, rs_v);
    }
  };

  const int key_end = a.fixed_valid ? L : V;
  const int nkt = (key_end + kKB - 1) / kKB;
  const int n_full = V / kKB;  // tiles whose 64 keys are all valid

  // Prologue in one memory round trip: the first K and V tiles and the next K tile are issued
  // into their buffers before the Q fragments and the gains are loaded; the compiler's wait for
  // those (before the key loop) then also covers the tiles, since loads complete in issue order.
  // (The paths with a running or fixed shift load K and V of tile 1 again at their first tile:
  // the same bytes into the same place, before any wave reads them.)
  load_tile(0, 0);
  if (nkt > 1) load_k(1, 1);
  // the Q/K RMSNorm gains (for the logit bound below), lane-strided
  const bool has_gains = a.q_gain != nullptr && a.k_gain != nullptr;
  float graw[2][DH / 64] = {};
  if (has_gains) {
#pragma unroll
    for (int r = 0; r < DH / 64; ++r) {
      graw[0][r] = a.q_gain[lane + 64 * r];
      graw[1][r] = a.k_gain[lane + 64 * r];
    }
  }
  const int my_q = q0 + wave * 32 + l32;
  const float c = a.scale_log2;
  bf16x8 qf[QS];
#pragma unroll
  for (int s = 0; s < QS; ++s) {
    u32x4 w = u32x4{0u, 0u, 0u, 0u};
    if (my_q < V) w = *reinterpret_cast<const u32x4*>(Q + (int64_t)my_q * a.row_stride + (2 * s + hh) * 8);
    qf[s] = __builtin_bit_cast(bf16x8, w);
  }
  // Consume the Q fragments and the gains once here: the compiler then places its wait for these
  // loads here, where it also covers the tiles issued before them, instead of at their first use
  // inside the key loop, where the same counter would also wait for the K/V prefetch in flight
  // (the LDS-destination loads are invisible to it).
#pragma unroll
  for (int s = 0; s < QS; ++s) asm volatile("" ::"v"(qf[s]));
#pragma unroll
  for (int r = 0; r < DH / 64; ++r) asm volatile("" ::"v"(graw[0][r]), "v"(graw[1][r]));


  // Logit bound from the Q/K RMSNorm gains: a normalised head vector has norm below sqrt(Dh),
  // so |q.k| < max|gq| max|gk| Dh; the factor 1 + 2^-6 covers the bf16 roundings of q, k and
  // q c. In log2 units (times c): up to 30, every probability exp2(s c) lies in [2^-31, 2^31]
  // (P V sums stay far from fp32 overflow); up to 60, exp2(s c - bound) lies in [2^-121, 1].
  // Both are normal in fp32 and bf16, and no running maximum is needed.
  float bound = INFINITY;
  if (has_gains) {
    float gq = 0.0f, gk = 0.0f;
#pragma unroll
    for (int r = 0; r < DH / 64; ++r) {
      gq = fmaxf(gq, fabsf(graw[0][r]));
      gk = fmaxf(gk, fabsf(graw[1][r]));
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      gq = fmaxf(gq, __shfl_xor(gq, o, 64));
      gk = fmaxf(gk, __shfl_xor(gk, o, 64));
    }
    bound = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(
        int, gq * gk * (float)DH * c * (1.0f + 1.0f / 64.0f))));
  }
  // 2: no shift, 1: shift by the bound, 0: online maximum (also for an infinite or NaN bound)
  const int shift_mode = bound <= 30.0f ? 2 : (bound <= 60.0f ? 1 : 0);
  if (shift_mode == 2) {
    // fold c into the Q fragments: the score MFMAs then yield logits in log2 units
#pragma unroll
    for (int s = 0; s < QS; ++s) {
      bf16x8 scaled;
#pragma unroll
      for (int e = 0; e < 8; ++e) scaled[e] = (__bf16)((float)qf[s][e] * c);
      qf[s] = scaled;
    }
  }
  // ---- per-lane LDS read addresses (byte offsets inside buffer 0) ----
  // K fragment of score k-step s, key half h2: row 32 h2 + l32, logical chunk 2 s + hh. At
  // head_dim 128 the swizzle ignores h2, which then only adds 32 rows.
  constexpr int KH = (DH == 128) ? 1 : 2;
  int kaddr[KH][QS];
#pragma unroll
  for (int h2 = 0; h2 < KH; ++h2)
#pragma unroll
    for (int s = 0; s < QS; ++s) {
      const int row = h2 * 32 + l32;
      kaddr[h2][s] = (row * NC + ((2 * s + hh) ^ kswz<DH>(row))) * 16;
    }
  auto kaddr_of = [&](int h2, int s) {
    return (DH == 128) ? kaddr[0][s] + h2 * 32 * NC * 16 : kaddr[h2 % KH][s];
  };
  // V^T fragment of d-tile dt: lane group g = lane / 16 supplies rows key0 + (lane & 15) / 4 and
  // columns 32 dt + 16 (g & 1) + 4 (lane & 3); key0 = 16 ps + 8 r + 4 (g >> 1) is added per read.
  int vaddr[DT];
  {
    const int g = lane >> 4, s16 = lane & 15;
    const int key = 4 * (g >> 1) + (s16 >> 2);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const int d = dt * 32 + 16 * (g & 1) + 4 * (s16 & 3);
      vaddr[dt] = VOFF + key * NC * 16 + (((d >> 3) ^ vswz<DH>(key)) * 16) + (d & 7) * 2;
    }
  }

  f32x16 oacc[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[t][e] = 0.0f;
  float m_run = -INFINITY;
  float l_run = 0.0f;

  const bf16x2 ones2 = {(__bf16)1.0f, (__bf16)1.0f};

  auto tile = [&](auto mode_c, auto masked_c, auto buf_c, int kt) __attribute__((always_inline)) {
    constexpr int MODE = decltype(mode_c)::value;
    constexpr bool FIXED = MODE != 0;
    constexpr bool MASKED = decltype(masked_c)::value;
    constexpr int BUF = decltype(buf_c)::value;
    const bool more = kt + 1 < nkt;
    if (more) load_tile(kt + 1, BUF ^ 1);

    // ---- S^T = K Q^T for 64 keys x 32 queries ----
    f32x16 sacc[2];
    {
      // K fragments are read kKPF MFMAs ahead of their use through a ring of registers, and the
      // issue order is pinned (left alone, the scheduler moves each read next to its MFMA and
      // the LDS latency lands in front of every MFMA of the first chain)
      constexpr int NS = 2 * QS;
      bf16x8 kr[kKPF];
      auto kread = [&](int i) __attribute__((always_inline)) {
        return __builtin_bit_cast(bf16x8, *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(
                                              lds + BUF * BUFB + kaddr_of(i / QS, i % QS)));
      };
#pragma unroll
      for (int i = 0; i < kKPF; ++i) kr[i] = kread(i);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        sacc[0][e] = 0.0f;
        sacc[1][e] = 0.0f;
      }
#pragma unroll
      for (int i = 0; i < NS; ++i) {
        const bf16x8 kf = kr[i % kKPF];
        if (i + kKPF < NS) kr[i % kKPF] = kread(i + kKPF);
        sacc[i / QS] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[i % QS], sacc[i / QS], 0, 0, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, kKPF, 0);  // kKPF LDS reads
#pragma unroll
      for (int i = 0; i + kKPF < NS; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // the next LDS read
      }
      __builtin_amdgcn_sched_group_barrier(0x008, kKPF, 0);  // the last kKPF MFMAs
    }
    // element (j, i) of sacc[h2] is key kt * 64 + 32 h2 + 8 j + 4 hh + i
    if (MASKED) {
      const int kv0 = kt * kKB;
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int key = kv0 + h2 * 32 + (e >> 2) * 8 + 4 * hh + (e & 3);
          if (key >= V) sacc[h2][e] = -INFINITY;
        }
    }

    // ---- softmax in base 2 (mode 2: the scores are already in log2 units) ----
    float mc;
    if (FIXED) {
      mc = bound;
    } else {
      // Online: the running max is exact (the largest probability of a row is exactly 1).
      // The accumulator rescale is skipped when no lane's max grew: alpha would be exactly 1.
      float mx = sacc[0][0];
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sacc[h2][e]);
      mx = pair_max(mx);
      const float m_new = fmaxf(m_run, mx);
      const bool grow = m_new > m_run;  // false for a fully masked tile (mx = -inf)
      if (__builtin_amdgcn_ballot_w64(grow) != 0) {
        const float alpha = grow ? __builtin_amdgcn_exp2f((m_run - m_new) * c) : 1.0f;
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int t = 0; t < DT; ++t)
#pragma unroll
          for (int e = 0; e < 16; ++e) oacc[t][e] *= alpha;
      }
      mc = (m_run == -INFINITY) ? 0.0f : m_run * c;
    }
    float psum = 0.0f;
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float p = (MODE == 2) ? __builtin_amdgcn_exp2f(sacc[h2][e])
                                    : __builtin_amdgcn_exp2f(fmaf(sacc[h2][e], c, -mc));
        sacc[h2][e] = p;
        if (!FIXED) psum += p;
      }
    if (!FIXED) l_run += psum;

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
      if (FIXED) {
        // row sum of the probabilities exactly as rounded for the P V product
        l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, p0), ones2, l_run, false);
        l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, p1), ones2, l_run, false);
        l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, p2), ones2, l_run, false);
        l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, p3), ones2, l_run, false);
      }
#pragma unroll
      for (int t = 0; t < DT; ++t) {
        lds_char* base = lds + BUF * BUFB + vaddr[t] + (16 * ps) * NC * 16;
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(reinterpret_cast<lds_s16x4*>(base));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(reinterpret_cast<lds_s16x4*>(base + 8 * NC * 16));
        const s16x8 v8 = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        oacc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, v8), pf,
                                                          oacc[t], 0, 0, 0);
      }
    }

    if (more) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  };

  auto sweep = [&](auto mode_c) __attribute__((always_inline)) {
    int kt = 0;
    for (; kt + 2 <= n_full; kt += 2) {
      tile(mode_c, std::false_type{}, std::integral_constant<int, 0>{}, kt);
      tile(mode_c, std::false_type{}, std::integral_constant<int, 1>{}, kt + 1);
    }
    for (; kt < nkt; ++kt) {
      if (kt & 1)
        tile(mode_c, std::true_type{}, std::integral_constant<int, 1>{}, kt);
      else
        tile(mode_c, std::true_type{}, std::integral_constant<int, 0>{}, kt);
    }
  };
  // ---- shift-free path, software pipelined inside the wave: iteration j issues the score MFMAs
  // of key tile j in the same instruction stream as the softmax and P V product of tile j - 1,
  // laid out slot by slot so that every MFMA has two VALU operations beside it. K and V are
  // staged one tile apart: while iteration j runs, K(j + 1) and V(j) are in flight into the
  // halves of the double buffer that iteration j - 1 finished reading (K(t) and V(t) live in
  // buffer t & 1). ----
  constexpr int NS = 2 * QS;            // score MFMAs per tile
  constexpr int NP = 4 * DT;            // P V MFMAs per tile
  // 64 VALU operations per tile (32 exps, 16 packs, 16 row-sum dots): 4 before the first slot,
  // the rest spread evenly over the NS + NP MFMA slots
  constexpr int kOpsPerSlot = (60 + NS + NP - 1) / (NS + NP);
  // every pack (op 3p + 2 of pair p) runs in an earlier slot than the P V MFMA that reads it
  // (slot NS + DT (p / 4))
  static_assert([] {
    for (int p = 0; p < 16; ++p) {
      const int op = 3 * p + 2;
      const int slot = op < 4 ? -1 : (op - 4) / kOpsPerSlot;
      if (slot >= NS + DT * (p / 4)) return false;
    }
    return true;
  }(), "softmax packs must precede their P V MFMAs");
  auto kread = [&](int kb, int i) __attribute__((always_inline)) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(
                                          lds + kb * BUFB + kaddr_of(i / QS, i % QS)));
  };
  // K fragment of score MFMA i of the pipelined path: the two 32-key halves alternate (key half
  // i & 1, k-step i >> 1), so consecutive MFMAs accumulate into different registers
  auto kread2 = [&](int kb, int i) __attribute__((always_inline)) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(
                                          lds + kb * BUFB + kaddr_of(i & 1, i >> 1)));
  };
  auto vread = [&](int vb, int m) __attribute__((always_inline)) {
    const int ps = m / DT, t = m % DT;
    lds_char* base = lds + vb * BUFB + vaddr[t] + (16 * ps) * NC * 16;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(reinterpret_cast<lds_s16x4*>(base));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(reinterpret_cast<lds_s16x4*>(base + 8 * NC * 16));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  // the first tile's scores and the last tile's P V run on their own, without the slot layout
  auto s_only = [&](int kb, f32x16 (&sn)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int e = 0; e < 16; ++e) { sn[0][e] = 0.0f; sn[1][e] = 0.0f; }
#pragma unroll
    for (int i = 0; i < NS; ++i)
      sn[i / QS] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kread(kb, i), qf[i % QS], sn[i / QS], 0, 0, 0);
  };
  auto pv_only = [&](int vb, f32x16 (&sp)[2]) __attribute__((always_inline)) {
    uint32_t pk[16];
#pragma unroll
    for (int p = 0; p < 16; ++p) {
      const float e0 = __builtin_amdgcn_exp2f(sp[p / 8][(2 * p) % 16]);
      const float e1 = __builtin_amdgcn_exp2f(sp[p / 8][(2 * p + 1) % 16]);
      pk[p] = pack_bf16x2(e0, e1);
      l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk[p]), ones2, l_run, false);
    }
#pragma unroll
    for (int m = 0; m < NP; ++m) {
      const int ps = m / DT;
      const bf16x8 pf = __builtin_bit_cast(bf16x8, u32x4{pk[4 * ps], pk[4 * ps + 1], pk[4 * ps + 2], pk[4 * ps + 3]});
      oacc[m % DT] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vread(vb, m), pf, oacc[m % DT], 0, 0, 0);
    }
  };
  // One pipelined iteration: scores of the K tile in buffer kb into sn, and softmax + P V of sp
  // with the V tile in buffer kb ^ 1, laid out slot by slot: slot k holds MFMA k (score MFMAs
  // first, then P V), the LDS reads for later slots and two VALU operations of the softmax.
  auto pipe = [&](auto kb_c, f32x16 (&sn)[2], f32x16 (&sp)[2]) __attribute__((always_inline)) {
    constexpr int kb = decltype(kb_c)::value;
    constexpr int vb = kb ^ 1;
    uint32_t pk[16];
    bf16x8 kr[kKPF];
    bf16x8 vr[kVPF];
    // VALU operation n of the iteration (0..63): exps e0..e31 (element idx of sp), packs of pairs,
    // row-sum dots; ordered so every pack is ready before its P V MFMA.
    float ex[32];
    // ops 0..47: exp, exp, pack for pairs 0..15 (pack of pair p at op 3p + 2, slot 3p/2 - 1 at
    // the latest, before the P V MFMA of its key group at slot 16 + 4 (p / 4)); ops 48..63: the
    // row-sum dots, which no MFMA waits for
    auto valu = [&](int n) __attribute__((always_inline)) {
      if (n < 48) {
        const int pair = n / 3, r = n % 3;
        if (r == 0) ex[2 * pair] = __builtin_amdgcn_exp2f(sp[(2 * pair) / 16][(2 * pair) % 16]);
        else if (r == 1) ex[2 * pair + 1] = __builtin_amdgcn_exp2f(sp[(2 * pair + 1) / 16][(2 * pair + 1) % 16]);
        else pk[pair] = pack_bf16x2(ex[2 * pair], ex[2 * pair + 1]);
      } else {
        l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk[n - 48]), ones2, l_run, false);
      }
    };
#pragma unroll
    for (int e = 0; e < 16; ++e) { sn[0][e] = 0.0f; sn[1][e] = 0.0f; }
#pragma unroll
    for (int i = 0; i < kKPF; ++i) kr[i] = kread2(kb, i);
    valu(0); valu(1); valu(2); valu(3);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 0; k < NS + NP; ++k) {
      if (k < NS) {
        const bf16x8 kf = kr[k % kKPF];
        if (k + kKPF < NS) kr[k % kKPF] = kread2(kb, k + kKPF);
        sn[k & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[k >> 1], sn[k & 1], 0, 0, 0);
        if (k >= NS - kVPF) vr[k - (NS - kVPF)] = vread(vb, k - (NS - kVPF));
      } else {
        const int m = k - NS;
        const int ps = m / DT;
        const bf16x8 vf = vr[m % kVPF];
        if (m + kVPF < NP) vr[m % kVPF] = vread(vb, m + kVPF);
        const bf16x8 pf = __builtin_bit_cast(bf16x8, u32x4{pk[4 * ps], pk[4 * ps + 1], pk[4 * ps + 2], pk[4 * ps + 3]});
        oacc[m % DT] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf, oacc[m % DT], 0, 0, 0);
      }
      // two VALU operations per slot (ops 4..63 over slots 0..29)
#pragma unroll
      for (int r = 0; r < kOpsPerSlot; ++r)
        if (4 + kOpsPerSlot * k + r < 64) valu(4 + kOpsPerSlot * k + r);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto mask_tile = [&](f32x16 (&sn)[2], int kt) __attribute__((always_inline)) {
    const int kv0 = kt * kKB;
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int key = kv0 + h2 * 32 + (e >> 2) * 8 + 4 * hh + (e & 3);
        if (key >= V) sn[h2][e] = -INFINITY;
      }
  };
  auto step = [&](auto kb_c, auto masked_c, f32x16 (&sn)[2], f32x16 (&sp)[2], int j)
      __attribute__((always_inline)) {
    constexpr int KB = decltype(kb_c)::value;
    if (j + 1 < nkt) load_k(j + 1, KB ^ 1);
    load_v(j, KB);
    pipe(kb_c, sn, sp);
    if constexpr (decltype(masked_c)::value) mask_tile(sn, j);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  };
  auto sweep_pipelined = [&]() __attribute__((always_inline)) {
    f32x16 sA[2], sB[2];
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    s_only(0, sA);
    if (0 >= n_full) mask_tile(sA, 0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    // steps j < n_full compute unmasked score tiles; the rest (at most the last partial tile,
    // plus the tail tiles in fixed-valid mode) mask theirs
    int j = 1;
    for (; j + 2 <= nkt && j + 1 < n_full; j += 2) {
      step(std::integral_constant<int, 1>{}, std::false_type{}, sB, sA, j);
      step(std::integral_constant<int, 0>{}, std::false_type{}, sA, sB, j + 1);
    }
    for (; j + 2 <= nkt; j += 2) {
      step(std::integral_constant<int, 1>{}, std::true_type{}, sB, sA, j);
      step(std::integral_constant<int, 0>{}, std::true_type{}, sA, sB, j + 1);
    }
    if (j < nkt) {
      step(std::integral_constant<int, 1>{}, std::true_type{}, sB, sA, j);
      pv_only(1, sB);
    } else {
      pv_only(0, sA);
    }
  };

  if (shift_mode == 2) {
    sweep_pipelined();
  } else {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (shift_mode == 1)
      sweep(std::integral_constant<int, 1>{});
    else
      sweep(std::integral_constant<int, 0>{});
  }

  // ---- normalise and store: element (j, i) of oacc[t] is d = 32 t + 8 j + 4 hh + i ----
  const float l_tot = pair_sum(l_run);
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
  // buffer offsets are 32-bit: one request's rows must span less than 2 GiB
  if ((int64_t)a.seq_pad * a.row_stride * 2 >= (int64_t)0x80000000) return hipErrorInvalidValue;
  if (a.seq_pad == 0) return hipSuccess;
  const dim3 grid((a.seq_pad + kQB - 1) / kQB, a.heads, a.batch);
  if (a.head_dim == 128) {
    hipLaunchKernelGGL(k_attn<128>, grid, dim3(64 * kNW), 0, s, a);
  } else if (a.head_dim == 64) {
    hipLaunchKernelGGL(k_attn<64>, grid, dim3(64 * kNW), 0, s, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace avdit
