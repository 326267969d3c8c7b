// bf16 MFMA GEMM for the block's projections: C[m][n] = sum_k A[m][k] * W[n][k], both operands
// contiguous along k (activations [tokens, K], weights [out, in]), fp32 accumulation, with the
// epilogue fused: plain store (QKV), gated residual (out-projection into the fp32 mid-block
// residual, down-projection from it), or SwiGLU over interleaved gate/up weight rows (gate/up
// projection; TeleFuser PR #23, "Changes Made": fused SwiGLU).
//
// Design for gfx950:
//  * WM x WN wave64s per workgroup (128 x 128 or 64 x 128 token x feature tiles, or the
//    256 x 256 direct-to-LDS kernel below); each wave owns a (BN/WN features) x (BM/WM tokens)
//    accumulator block of 32x32 tiles of v_mfma_f32_32x32x16_bf16. The weight tile is the MFMA
//    A operand and the token tile the B operand, so every lane ends up holding 4 consecutive
//    output features of one token; the epilogue turns that layout row-major through the LDS
//    (see store_tile_staged) so that its loads and stores cover whole row segments.
//  * k-tiles of 64 staged global -> registers -> LDS, double buffered, one barrier per k-tile.
//    Global loads are raw buffer loads: rows past the valid range or past K read as zero from
//    the hardware's range check, so the loop has no branches. The next tile's loads are issued
//    at the top of the current tile and written to the other LDS buffer after the current
//    tile's last MFMAs have been issued.
//  * MFMA fragments are double buffered in registers: the fragments of k-substep s+1 are read
//    from LDS while the MFMAs of substep s run, so LDS latency hides under matrix work.
//  * LDS rows are 128 bytes with the 16-byte chunk index XOR-swizzled by (r ^ r >> 3) & 7,
//    which keeps both the 16-byte fragment reads (32 rows, same chunk) and the loader's writes
//    free of bank conflicts.
//  * Workgroup ids are remapped so that each XCD (ids are dealt round-robin over the 8 XCDs)
//    receives a contiguous range of tiles, ordered in groups of token-tiles, so the workgroups
//    resident on one XCD share operand panels in that XCD's L2; the tiles that hold valid rows
//    are shared evenly over the XCDs before the tail tiles (see select_tile).
//  * Rows at or beyond n_valid are never multiplied: their loads read zero and a tile that lies
//    entirely in the tail only writes zeros (the zero-tail merge of TeleFuser PR #38, section 2).
#include "common.hpp"
#include "kernels.hpp"

namespace avdit {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) char lds_char_t;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4_t;

constexpr int kBK = 64;                      // k-tile; 8 chunks of 8 bf16 per LDS row
constexpr uint32_t kOob = 0x80000000u;       // buffer offset past every range: reads zero
constexpr int32_t kRsrcWord3 = 0x00020000;   // raw buffer resource, 32-bit elements

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, kRsrcWord3);
}

// Element-wise load of 8 bf16 at (row, k) for operands whose rows are not 16-byte aligned.
__device__ __forceinline__ u32x4 load_chunk_slow(const uint16_t* __restrict__ base, int64_t ld,
                                                 int row, bool row_ok, int k, int K) {
  if (!row_ok || k >= K) return u32x4{0u, 0u, 0u, 0u};
  const uint16_t* p = base + (int64_t)row * ld + k;
  uint32_t w[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t lo = (k + 2 * j < K) ? p[2 * j] : 0u;
    const uint32_t hi = (k + 2 * j + 1 < K) ? p[2 * j + 1] : 0u;
    w[j] = lo | (hi << 16);
  }
  return u32x4{w[0], w[1], w[2], w[3]};
}

// XOR swizzle of the 16-byte chunk index inside a 128-byte LDS row. Sixteen consecutive rows
// read at one logical chunk land on distinct banks whether the LDS serves 8 or 16 lanes of a
// 16-byte read per cycle: f is a permutation on every 8 aligned rows, and injective on the even
// and on the odd rows of every 16.
__device__ __forceinline__ int swz(int r) { return (r ^ (r >> 3)) & 7; }

__device__ __forceinline__ float silu_mul(float g, float u) {
  return g / (1.0f + __expf(-g)) * u;
}

// Token-tiles of bm rows that hold a valid row ("work" tiles) and those wholly in a tail (which
// only write zeros), counted over the requests of a batch (bm divides a request's rows).
__device__ __forceinline__ int work_mtiles(const RowLayout& r, int bm, int tiles_m) {
  if (r.batch <= 1) {
    const int v = (r.n_valid + bm - 1) / bm;
    return v < tiles_m ? v : tiles_m;
  }
  const int tpr = r.seq_pad / bm;
  int n = 0;
  for (int b = 0; b < r.batch; ++b) {
    const int v = (r.req_valid[b] + bm - 1) / bm;
    n += v < tpr ? v : tpr;
  }
  return n;
}
// Index of the j-th work token-tile (work) or the j-th tail token-tile (!work), in row order.
__device__ __forceinline__ int nth_mtile(const RowLayout& r, int bm, int tiles_m, int j, bool work) {
  if (r.batch <= 1) {
    const int v = work_mtiles(r, bm, tiles_m);
    return work ? j : v + j;
  }
  const int tpr = r.seq_pad / bm;
  for (int b = 0; b < r.batch; ++b) {
    int v = (r.req_valid[b] + bm - 1) / bm;
    v = v < tpr ? v : tpr;
    const int c = work ? v : tpr - v;
    if (j < c) return b * tpr + (work ? j : v + j);
    j -= c;
  }
  return tiles_m - 1;  // not reached: j is below the count of its kind
}

// Tile selection: workgroup ids are dealt round-robin over the 8 XCDs, so XCD x runs the ids
// b = x (mod 8), in order. Each XCD receives an equal contiguous share of the work tiles first,
// then an equal share of the tail tiles, so that a ragged batch (whose short requests leave
// whole token-tiles in their tails) loads the XCDs evenly; with the tail tiles ordered after
// the work tiles an XCD holding short requests would otherwise finish long before one holding
// full ones. Work tiles are ordered in groups of GM token-tiles, so that the workgroups
// resident on one XCD share operand panels in its L2. GM is 6, or 3 for a long reduction
// (K >= 2 N: the down projection), chosen by the launcher from kernel-trace sweeps of
// GM = 2, 3, 4, 6 (8 and 16 were slower) on the 32k-token and 13,440-token blocks: the down
// projection ran 3-5% faster with 3, the other three projections fastest with 6 or within 1%
// of it. The map from ids to tiles is a bijection for any counts (each XCD's share of work
// tiles never exceeds its share of ids).
__device__ __forceinline__ void select_tile(const RowLayout& rows, int bm, int tiles_m,
                                            int tiles_n, int& tile_m, int& tile_n, int GM = 6) {
  const int nt = tiles_m * tiles_n;
  const int b = blockIdx.x;
  const int xcd = b & 7, local = b >> 3;
  const int mw = work_mtiles(rows, bm, tiles_m);
  const int wt = mw * tiles_n;
  const int per_t = nt >> 3, rem_t = nt & 7;
  const int per_w = wt >> 3, rem_w = wt & 7;
  const int base_w = xcd * per_w + (xcd < rem_w ? xcd : rem_w);
  const int w_x = per_w + (xcd < rem_w ? 1 : 0);
  if (local < w_x) {
    const int logical = base_w + local;
    const int group = logical / (GM * tiles_n);
    const int first_m = group * GM;
    const int gm = (mw - first_m) < GM ? (mw - first_m) : GM;
    const int in_group = logical - group * GM * tiles_n;
    tile_m = nth_mtile(rows, bm, tiles_m, first_m + in_group % gm, true);
    tile_n = in_group / gm;
  } else {
    const int base_t = xcd * per_t + (xcd < rem_t ? xcd : rem_t);
    const int z = base_t - base_w + (local - w_x);
    tile_m = nth_mtile(rows, bm, tiles_m, z / tiles_n, false);
    tile_n = z % tiles_n;
  }
}

typedef __attribute__((address_space(3))) f32x4 lds_f32x4_t;

// Fused epilogue, staged through the LDS (free once every wave has passed the barrier at its
// top). In the MFMA layout lane (l32, hh) holds features 32 f + 8 j + 4 hh .. + 3 of token
// 32 t + l32 of its wave's block in acc[f][t][4 j .. 4 j + 3] (SwiGLU pairs gate sub-tile 0 with
// up sub-tile 1), so a store instruction straight from the accumulators would write 8 or 16
// bytes into each of 32 token rows. Instead each wave writes its 32 MT tokens x 64 features of
// fp32 accumulators into a private 16 KB region of the LDS (as many tokens per pass as fit) and
// reads them back row-major, 16 lanes per token row (8 for SwiGLU's 32 output features), so that
// every global load and store instruction covers whole 128- or 256-byte row segments of 4 or 8
// rows. The gated epilogues issue all their residual and gate loads before the first store:
// loads and stores share one completion counter, so a load issued after a store would be
// waited for together with that store. Values: acc (fp32), then silu(g) u, or
// resid + gate acc (fmaf), or the plain value, rounded once to the output type. Invalid rows
// (at or past a request's valid length) are written 0, rows past the last request are not
// written.
// LDS bytes of one wave's staging region: as many 32-token blocks per pass as fit in 16 KB.
template <int EPI, int MT>
constexpr int staged_region_bytes() {
  constexpr int OF = (EPI == EPI_SWIGLU) ? 32 : 64;  // output features of the wave
  constexpr int TP = (128 / OF) < MT ? (128 / OF) : MT;
  return TP * 32 * OF * 4;
}

template <int EPI, int MT>
__device__ __forceinline__ void store_tile_staged(const GemmArgs& a, f32x16 (&acc)[2][MT], int m0,
                                                  int n0, int wm, int wn, int lane,
                                                  lds_char_t* region) {
  constexpr int TM = 32 * MT;                              // tokens per wave
  constexpr bool GATED = (EPI == EPI_GATED_TO_F32) || (EPI == EPI_GATED_F32_IN) ||
                         (EPI == EPI_GATED_F32_TO_F32);
  constexpr bool OUT_F32 = (EPI == EPI_GATED_TO_F32) || (EPI == EPI_GATED_F32_TO_F32);
  constexpr bool RESID_F32 = (EPI == EPI_GATED_F32_IN) || (EPI == EPI_GATED_F32_TO_F32);
  constexpr int OUT_T = (EPI == EPI_SWIGLU) ? 1 : 2;      // 32-feature output sub-tiles
  constexpr int OF = OUT_T * 32;                           // output features of the wave
  constexpr int LR = OF / 4;                               // lanes per token row
  constexpr int RI = 64 / LR;                              // token rows per step
  constexpr int TP = (128 / OF) < MT ? (128 / OF) : MT;    // 32-row blocks per pass (<= 16 KB)
  constexpr int NP = MT / TP;                              // passes
  static_assert(MT % TP == 0, "whole passes");
  static_assert(TP * 32 * OF * 4 == staged_region_bytes<EPI, MT>(), "region size");
  constexpr int RB = OF * 4;                               // bytes per staged row
  constexpr int SPP = TP * 32 / RI;                        // steps per pass
  const int l32 = lane & 31, hh = lane >> 5;
  const int rsub = lane / LR, q = lane % LR;
  const int rows_total = total_rows(a.rows);
  const int fb = n0 + wn * OF + 4 * q;                     // this lane's 4 output features
  const int tok0 = m0 + wm * TM;
  // A tile never straddles two requests: the request, its first row and its bounds are uniform.
  int req = 0, base = 0, nvalid = a.rows.n_valid, nvideo = a.rows.n_video;
  if (a.rows.batch > 1) {
    req = m0 / a.rows.seq_pad;
    base = req * a.rows.seq_pad;
    nvalid = a.rows.req_valid[req];
    nvideo = a.rows.req_video[req];
  }
  // Bank-conflict-free staging: 16-byte chunk c of row r sits at chunk c ^ sw(r), so that the 8
  // (or 16) lanes that the LDS serves together, consecutive rows at one chunk when writing and
  // the chunks of one or two rows when reading, fall on distinct 16-byte bank groups of 128 (or
  // 256) bytes: sw = r mod 16 for 256-byte rows; for 128-byte rows sw = (r mod 8) ^ (r / 8 mod 2),
  // a permutation on every 8 aligned rows that also separates the even (and the odd) rows of 16.
  auto sw = [](int r) __attribute__((always_inline)) {
    return RB == 256 ? (r & 15) : ((r & 7) ^ ((r >> 3) & 1));
  };

  if constexpr (EPI == EPI_SWIGLU) {
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[0][t][e] = silu_mul(acc[0][t][e], acc[1][t][e]);
  }
  auto stage = [&](int p) __attribute__((always_inline)) {
#pragma unroll
    for (int tt = 0; tt < TP; ++tt) {
      const int row = tt * 32 + l32;
#pragma unroll
      for (int f = 0; f < OUT_T; ++f)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int c = 8 * f + 2 * j + hh;
          const f32x4 v = {acc[f][p * TP + tt][4 * j], acc[f][p * TP + tt][4 * j + 1],
                           acc[f][p * TP + tt][4 * j + 2], acc[f][p * TP + tt][4 * j + 3]};
          *reinterpret_cast<lds_f32x4_t*>(region + row * RB + ((c ^ sw(row)) << 4)) = v;
        }
    }
  };
  __syncthreads();  // every wave is done with the ring's fragments
  stage(0);

  // gated: every residual the wave reads, then the gate terms (ada, temb) of both modalities
  // for the lane's features, all in flight before the first store; the gate sum ada + temb is
  // formed at its first use, so that no wait separates the loads
  f32x4 rv[NP][SPP];
  float4 ga[2], gt[2];
  if constexpr (GATED) {
    const int fc = fb < a.N ? fb : a.N - 4;
#pragma unroll
    for (int p = 0; p < NP; ++p)
#pragma unroll
      for (int st = 0; st < SPP; ++st) {
        int tok = tok0 + p * TP * 32 + st * RI + rsub;
        tok = tok < rows_total ? tok : rows_total - 1;
        if constexpr (RESID_F32) {
          const float4 r4 = *reinterpret_cast<const float4*>(
              static_cast<const float*>(a.resid) + (int64_t)tok * a.ldr + fc);
          rv[p][st] = f32x4{r4.x, r4.y, r4.z, r4.w};
        } else {
          const u32x2 rr = *reinterpret_cast<const u32x2*>(
              static_cast<const uint16_t*>(a.resid) + (int64_t)tok * a.ldr + fc);
          rv[p][st] = f32x4{bf_lo(rr.x), bf_hi(rr.x), bf_lo(rr.y), bf_hi(rr.y)};
        }
      }
#pragma unroll
    for (int mod = 0; mod < 2; ++mod) {
      const int64_t goff = ((int64_t)mod * 6 + a.chunk) * a.N + fc;
      ga[mod] = *reinterpret_cast<const float4*>(a.ada + goff);
      gt[mod] = *reinterpret_cast<const float4*>(a.temb + req * a.temb_stride + goff);
    }
  }

#pragma unroll
  for (int p = 0; p < NP; ++p) {
    if (p > 0) stage(p);  // the wave's own reads of pass p - 1 precede these writes (LDS order)
#pragma unroll
    for (int st = 0; st < SPP; ++st) {
      const int row = st * RI + rsub;
      const f32x4 v = *reinterpret_cast<lds_f32x4_t*>(region + row * RB + ((q ^ sw(row)) << 4));
      const int tok = tok0 + p * TP * 32 + row;
      if (tok >= rows_total || fb >= a.N) continue;
      const int i = tok - base;
      float o[4] = {0.0f, 0.0f, 0.0f, 0.0f};
      if (i < nvalid) {
        if constexpr (GATED) {
          const float4 g4 = i < nvideo ? make_float4(ga[0].x + gt[0].x, ga[0].y + gt[0].y,
                                                     ga[0].z + gt[0].z, ga[0].w + gt[0].w)
                                       : make_float4(ga[1].x + gt[1].x, ga[1].y + gt[1].y,
                                                     ga[1].z + gt[1].z, ga[1].w + gt[1].w);
          o[0] = fmaf(g4.x, v[0], rv[p][st][0]);
          o[1] = fmaf(g4.y, v[1], rv[p][st][1]);
          o[2] = fmaf(g4.z, v[2], rv[p][st][2]);
          o[3] = fmaf(g4.w, v[3], rv[p][st][3]);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] = v[e];
        }
      }
      if constexpr (OUT_F32) {
        float* crow = static_cast<float*>(a.C) + (int64_t)tok * a.ldc;
        *reinterpret_cast<float4*>(crow + fb) = make_float4(o[0], o[1], o[2], o[3]);
      } else {
        uint16_t* crow = static_cast<uint16_t*>(a.C) + (int64_t)tok * a.ldc;
        if (fb + 4 <= a.N) {
          *reinterpret_cast<u32x2*>(crow + fb) = u32x2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (fb + e < a.N) crow[fb + e] = to_bf16(o[e]);
        }
      }
    }
  }
}

template <int BM, int BN, int WM, int WN, int EPI, bool ALIGNED>
__global__ __launch_bounds__(64 * WM * WN, 1) void k_gemm(GemmArgs a, int tiles_m, int tiles_n) {
  constexpr int NT = 64 * WM * WN;    // threads
  constexpr int TM = BM / WM;         // tokens per wave
  constexpr int TN = BN / WN;         // weight rows per wave
  constexpr int MT = TM / 32;         // 32-token sub-tiles per wave
  constexpr int FT = TN / 32;         // 32-row weight sub-tiles per wave
  constexpr int ROWS = BM + BN;       // LDS rows per stage (weights first)
  constexpr int PT = ROWS * 8 / NT;   // 16-byte chunks each thread stages per k-tile
  constexpr int RPI = NT / 8;         // LDS rows covered by one staging step
  static_assert(EPI != EPI_SWIGLU || (FT % 2) == 0, "SwiGLU pairs gate/up sub-tiles");
  static_assert(BN % RPI == 0 && BM % RPI == 0, "staging steps must not straddle operands");

  __shared__ u32x4 lds[2][ROWS * 8];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hh = lane >> 5;
  const int wave = tid >> 6;
  const int wm = wave % WM;   // token slice
  const int wn = wave / WM;   // feature slice

  int tile_m, tile_n;
  select_tile(a.rows, BM, tiles_m, tiles_n, tile_m, tile_n);

  const int m0 = tile_m * BM;
  const int rows_total = total_rows(a.rows);
  // first output feature of this tile (SwiGLU tiles cover BN/2 outputs)
  const int n0 = (EPI == EPI_SWIGLU) ? tile_n * (BN / 2) : tile_n * BN;

  f32x16 acc[FT][MT];
#pragma unroll
  for (int f = 0; f < FT; ++f)
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[f][t][e] = 0.0f;

  if (rows_have_valid(a.rows, m0)) {
    const int ck = tid & 7;
    const int w_rows = (EPI == EPI_SWIGLU) ? a.up_offset + a.N : a.N;
    const __amdgpu_buffer_rsrc_t rs_w = make_rsrc(a.W, (uint32_t)((int64_t)w_rows * a.ldw * 2));
    const __amdgpu_buffer_rsrc_t rs_a = make_rsrc(a.A, (uint32_t)((int64_t)rows_total * a.lda * 2));
    // byte offset of each staged row (kOob when the row is masked)
    uint32_t src_off[PT];
    int src_row[PT];
    bool src_ok[PT];
#pragma unroll
    for (int i = 0; i < PT; ++i) {
      const int r = (tid >> 3) + RPI * i;
      if (i < BN / RPI) {
        int wrow, feat;
        if (EPI == EPI_SWIGLU) {
          const int blk = r >> 5;
          feat = n0 + (blk >> 1) * 32 + (r & 31);
          wrow = (blk & 1) ? a.up_offset + feat : feat;
        } else {
          feat = n0 + r;
          wrow = feat;
        }
        src_row[i] = wrow;
        src_ok[i] = feat < a.N;
        src_off[i] = src_ok[i] ? (uint32_t)((int64_t)wrow * a.ldw * 2) : kOob;
      } else {
        const int tok = m0 + (r - BN);
        src_row[i] = tok;
        src_ok[i] = tok < rows_total && row_info(a.rows, tok).valid;
        src_off[i] = src_ok[i] ? (uint32_t)((int64_t)tok * a.lda * 2) : kOob;
      }
    }
    const int nk = (a.K + kBK - 1) / kBK;
    u32x4 stage[PT];
    auto load_stage = [&](int kt) {
      const int k = kt * kBK + ck * 8;
#pragma unroll
      for (int i = 0; i < PT; ++i) {
        // staging step i covers rows RPI*i .. RPI*i + RPI - 1: all weight rows or all token rows
        const bool w_step = i < BN / RPI;
        if (ALIGNED) {
          const uint32_t off = (k < a.K) ? src_off[i] + (uint32_t)(k * 2) : kOob;
          stage[i] = w_step ? __builtin_amdgcn_raw_buffer_load_b128(rs_w, off, 0, 0)
                            : __builtin_amdgcn_raw_buffer_load_b128(rs_a, off, 0, 0);
        } else {
          stage[i] = w_step ? load_chunk_slow(a.W, a.ldw, src_row[i], src_ok[i], k, a.K)
                            : load_chunk_slow(a.A, a.lda, src_row[i], src_ok[i], k, a.K);
        }
      }
    };
    auto store_stage = [&](int buf) {
#pragma unroll
      for (int i = 0; i < PT; ++i) {
        const int r = (tid >> 3) + RPI * i;
        lds[buf][r * 8 + (ck ^ swz(r))] = stage[i];
      }
    };
    bf16x8 af[2][FT], bf[2][MT];
    auto read_frags = [&](int buf, int s, int slot) {
      const int c = 2 * s + hh;
#pragma unroll
      for (int f = 0; f < FT; ++f) {
        const int r = wn * TN + f * 32 + l32;
        af[slot][f] = __builtin_bit_cast(bf16x8, lds[buf][r * 8 + (c ^ swz(r))]);
      }
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        const int r = BN + wm * TM + t * 32 + l32;
        bf[slot][t] = __builtin_bit_cast(bf16x8, lds[buf][r * 8 + (c ^ swz(r))]);
      }
    };

    load_stage(0);
    store_stage(0);
    __syncthreads();
    read_frags(0, 0, 0);
    for (int kt = 0; kt < nk; ++kt) {
      const int cur = kt & 1;
      const bool more = kt + 1 < nk;
      if (more) load_stage(kt + 1);
#pragma unroll
      for (int s = 0; s < kBK / 16; ++s) {
        const int slot = s & 1;
        if (s + 1 < kBK / 16) read_frags(cur, s + 1, slot ^ 1);
#pragma unroll
        for (int f = 0; f < FT; ++f)
#pragma unroll
          for (int t = 0; t < MT; ++t)
            acc[f][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[slot][f], bf[slot][t],
                                                                acc[f][t], 0, 0, 0);
      }
      if (more) store_stage(cur ^ 1);
      __syncthreads();
      if (more) read_frags(cur ^ 1, 0, 0);
    }
  }

  // one staging region per wave inside the (now free) operand buffers
  constexpr int REGION = staged_region_bytes<EPI, MT>();
  static_assert(FT == 2 && (int)sizeof(lds) >= WM * WN * REGION,
                "staged epilogue: 64 features per wave, every wave's region inside the LDS");
  store_tile_staged<EPI, MT>(a, acc, m0, n0, wm, wn, lane, (lds_char_t*)(&lds[0][0]) + wave * REGION);
}

// ---------------------------------------------------------------------------------------------
// Large-problem GEMM: operands go straight from memory into a ring of LDS stages.
//
//  * 256 x 256 tiles (weights x tokens), 8 wave64s of 64 features x 128 tokens, k-tiles of 64.
//  * Buffer loads with the LDS destination (no staging registers, no LDS write instructions):
//    one wave load fills 8 LDS rows of 128 bytes; each lane fetches the 16-byte global chunk
//    that the swizzle places in its slot.
//  * One barrier per k-tile, placed before the last MFMA k-step of k-tile kt: by then every
//    fragment of kt is in registers, so kt's stage receives the loads of k-tile kt + 2 while
//    the barrier publishes k-tile kt + 1, whose first fragments are read under the last
//    k-step's MFMAs. Two 64 KB stages measured faster than four 32 KB ones (half the barriers;
//    deeper prefetch gained nothing).
//  * Waves 0-3 (one on each SIMD) issue all 64 loads of a k-tile, 16 each; waves 4-7 issue
//    none. The loads of a k-tile are accepted by the CU's memory pipeline at a fixed rate, so a
//    wave that issues them stalls for a good part of a k-tile: with every wave loading, both
//    waves of a SIMD stalled together and its MFMA pipe drained; with one loader per SIMD the
//    other wave keeps issuing MFMAs meanwhile (14% fewer cycles per k-tile on the QKV
//    projection, with the loads still landing in time).
// ---------------------------------------------------------------------------------------------
constexpr int kDlBK = 64;                  // k-tile
constexpr int kDlStages = 2;               // LDS ring depth: 2 x 64 KB
constexpr int kDlRows = 512;               // LDS rows per stage: 256 weight rows, 256 token rows
constexpr int kDlRowB = kDlBK * 2;         // bytes per LDS row
constexpr int kDlNch = kDlBK / 8;          // 16-byte chunks per row
constexpr int kDlStageBytes = kDlRows * kDlRowB;

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ i32x4 raw_rsrc(const void* p, uint32_t bytes) {
  const uint64_t ad = reinterpret_cast<uint64_t>(p);
  return i32x4{(int32_t)(uint32_t)ad, (int32_t)(uint32_t)(ad >> 32), (int32_t)bytes, kRsrcWord3};
}
// 16 bytes per lane from memory into LDS at lds_base + 16 lane (lds_base wave-uniform); offsets
// past the resource range read as zero. Completion is awaited with explicit vmcnt waits.
__device__ __forceinline__ void dl_b128(uint32_t lds_base, uint32_t voffset, i32x4 rsrc) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(lds_base), "v"(voffset), "s"(rsrc)
               : "memory", "m0");
}
// Chunk swizzle of a 128-byte LDS row: the 16 rows that one group of lanes reads at a logical
// chunk (8 even and 8 odd rows) land on 16 distinct 16-byte bank groups.
__device__ __forceinline__ int dl_swz(int r) { return (r >> 1) & 7; }

template <int EPI>
__global__ __launch_bounds__(512, 2) void k_gemm_dl(GemmArgs a, int tiles_m, int tiles_n, int gm) {
  constexpr int BM = 256, BN = 256, WM = 2, WN = 4;
  constexpr int STAGES = kDlStages;
  constexpr int NW = WM * WN;
  constexpr int NL = 4;                       // loading waves: one per SIMD
  constexpr int LPW = kDlRows / 8 / NL;       // wave loads per loading wave per stage (16)
  constexpr int RPL = 64 / kDlNch;            // rows per wave load
  constexpr int TM = BM / WM, TN = BN / WN, MT = TM / 32, FT = TN / 32;
  constexpr int KS = kDlBK / 16;              // MFMA k-steps per k-tile
  __shared__ u32x4 lds_ring[STAGES * kDlStageBytes / 16];
  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hh = lane >> 5, wave = tid >> 6;
  const int wm = wave % WM, wn = wave / WM;
  int tile_m, tile_n;
  select_tile(a.rows, BM, tiles_m, tiles_n, tile_m, tile_n, gm);
  const int m0 = tile_m * BM;
  const int rows_total = total_rows(a.rows);
  const int n0 = (EPI == EPI_SWIGLU) ? tile_n * (BN / 2) : tile_n * BN;
  f32x16 acc[FT][MT];
#pragma unroll
  for (int f = 0; f < FT; ++f)
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[f][t][e] = 0.0f;
  if (rows_have_valid(a.rows, m0)) {
    const int w_rows = (EPI == EPI_SWIGLU) ? a.up_offset + a.N : a.N;
    const i32x4 rs_w = raw_rsrc(a.W, (uint32_t)((int64_t)w_rows * a.ldw * 2));
    const i32x4 rs_a = raw_rsrc(a.A, (uint32_t)((int64_t)rows_total * a.lda * 2));
    uint32_t goff[LPW];
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int r = RPL * (NL * i + (wave % NL)) + lane / kDlNch;
      const int kc = (lane % kDlNch) ^ dl_swz(r);
      if (i < LPW / 2) {
        int wrow, feat;
        if (EPI == EPI_SWIGLU) {
          const int blk = r >> 5;
          feat = n0 + (blk >> 1) * 32 + (r & 31);
          wrow = (blk & 1) ? a.up_offset + feat : feat;
        } else {
          feat = n0 + r;
          wrow = feat;
        }
        goff[i] = feat < a.N ? (uint32_t)((int64_t)wrow * a.ldw * 2 + kc * 16) : kOob;
      } else {
        const int tok = m0 + (r - BN);
        goff[i] = (tok < rows_total && row_info(a.rows, tok).valid)
                      ? (uint32_t)((int64_t)tok * a.lda * 2 + kc * 16) : kOob;
      }
    }
    lds_char_t* lds = (lds_char_t*)(lds_ring);
    const uint32_t lbase = (uint32_t)__builtin_amdgcn_readfirstlane(
        (int)(uint32_t)(uintptr_t)lds + (wave % NL) * 1024);
    const bool loader = wave < NL;
    const int nk = a.K / kDlBK;
    auto issue = [&](int kt) __attribute__((always_inline)) {
      const uint32_t sb = lbase + (uint32_t)(kt % STAGES) * kDlStageBytes;
      const uint32_t kb = (uint32_t)kt * (kDlBK * 2);
#pragma unroll
      for (int i = 0; i < LPW; ++i)
        dl_b128(sb + i * NL * 1024, goff[i] + kb, i < LPW / 2 ? rs_w : rs_a);
    };
    const int sw = dl_swz(l32);
    int foff[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) foff[s] = l32 * kDlRowB + ((2 * s + hh) ^ sw) * 16;
    bf16x8 af[2][FT], bf[2][MT];
    auto read_frags = [&](int kt, int s, int slot) __attribute__((always_inline)) {
      lds_char_t* st = lds + (kt % STAGES) * kDlStageBytes + foff[s];
#pragma unroll
      for (int f = 0; f < FT; ++f)
        af[slot][f] = __builtin_bit_cast(bf16x8, *reinterpret_cast<lds_u32x4_t*>(st + (wn * TN + f * 32) * kDlRowB));
#pragma unroll
      for (int t = 0; t < MT; ++t)
        bf[slot][t] = __builtin_bit_cast(bf16x8, *reinterpret_cast<lds_u32x4_t*>(st + (BN + wm * TM + t * 32) * kDlRowB));
    };
    auto mfmas = [&](int slot) __attribute__((always_inline)) {
#pragma unroll
      for (int f = 0; f < FT; ++f)
#pragma unroll
        for (int t = 0; t < MT; ++t)
          acc[f][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[slot][f], bf[slot][t], acc[f][t], 0, 0, 0);
    };
    // wait until at most `ahead` k-tiles of this wave's loads (16 each) are still in flight
    static_assert(LPW == 16 && STAGES == 2, "vmcnt values encode 16 loads per k-tile, 2 stages");
    auto wait_tiles = [&](int ahead) __attribute__((always_inline)) {
      if (ahead >= 1) asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
      else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    };
    // prologue: every stage filled, wait for k-tile 0
    if (loader)
      for (int kt = 0; kt < STAGES && kt < nk; ++kt) issue(kt);
    wait_tiles(min(STAGES - 1, nk - 1));
    __syncthreads();
    read_frags(0, 0, 0);
    for (int kt = 0; kt + 1 < nk; ++kt) {
#pragma unroll
      for (int s = 0; s + 1 < KS; ++s) {
        read_frags(kt, s + 1, (s + 1) & 1);
        __builtin_amdgcn_sched_barrier(0);
        mfmas(s & 1);
      }
      // all fragments of k-tile kt are in registers: its stage takes k-tile kt + STAGES
      wait_tiles(min(STAGES - 2, nk - 2 - kt));
      __syncthreads();
      if (loader && kt + STAGES < nk) issue(kt + STAGES);
      read_frags(kt + 1, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      mfmas((KS - 1) & 1);
    }
#pragma unroll
    for (int s = 0; s + 1 < KS; ++s) {
      read_frags(nk - 1, s + 1, (s + 1) & 1);
      mfmas(s & 1);
    }
    mfmas((KS - 1) & 1);
  }
  static_assert(FT == 2 && MT == 4 && TM == 128 && STAGES * kDlStageBytes == NW * 16384 &&
                    staged_region_bytes<EPI, MT>() == 16384,
                "staged epilogue: 128 x 64 accumulators and 16 KB of the ring per wave");
  store_tile_staged<EPI, MT>(a, acc, m0, n0, wm, wn, lane, (lds_char_t*)(lds_ring) + wave * 16384);
}

template <int BM, int BN, int WM, int WN, int EPI, bool ALIGNED>
static hipError_t gemm_instance(const GemmArgs& a, hipStream_t s) {
  const int out_per_tile = (EPI == EPI_SWIGLU) ? BN / 2 : BN;
  const int tiles_m = (total_rows(a.rows) + BM - 1) / BM;
  const int tiles_n = (a.N + out_per_tile - 1) / out_per_tile;
  const int nt = tiles_m * tiles_n;
  if (nt == 0) return hipSuccess;
  hipLaunchKernelGGL((k_gemm<BM, BN, WM, WN, EPI, ALIGNED>), dim3(nt),
                     dim3(64 * WM * WN), 0, s, a, tiles_m, tiles_n);
  return hipGetLastError();
}

template <int BM, int BN, int WM, int WN, bool ALIGNED>
static hipError_t gemm_dispatch_epi(const GemmArgs& a, hipStream_t s) {
  switch (a.epilogue) {
    case EPI_STORE: return gemm_instance<BM, BN, WM, WN, EPI_STORE, ALIGNED>(a, s);
    case EPI_GATED_TO_F32: return gemm_instance<BM, BN, WM, WN, EPI_GATED_TO_F32, ALIGNED>(a, s);
    case EPI_GATED_F32_IN: return gemm_instance<BM, BN, WM, WN, EPI_GATED_F32_IN, ALIGNED>(a, s);
    case EPI_GATED_F32_TO_F32:
      return gemm_instance<BM, BN, WM, WN, EPI_GATED_F32_TO_F32, ALIGNED>(a, s);
    case EPI_SWIGLU: return gemm_instance<BM, BN, WM, WN, EPI_SWIGLU, ALIGNED>(a, s);
    default: return hipErrorInvalidValue;
  }
}

// Compute units of the current device (queried once; 256 on MI355X).
static long compute_units() {
  static const long n = [] {
    int dev = 0, cu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cu <= 0)
      return 256L;
    return (long)cu;
  }();
  return n;
}

hipError_t launch_gemm(const GemmArgs& a, hipStream_t s) {
  if (a.N <= 0 || a.K <= 0) return hipErrorInvalidValue;
  // Epilogue vectors are 4 features wide and 8-byte aligned.
  if ((a.ldc & 3) != 0) return hipErrorInvalidValue;
  const bool gated = a.epilogue == EPI_GATED_TO_F32 || a.epilogue == EPI_GATED_F32_IN ||
                     a.epilogue == EPI_GATED_F32_TO_F32;
  if (gated && ((a.N & 3) != 0 || (a.ldr & 3) != 0)) return hipErrorInvalidValue;
  // Buffer offsets are 32-bit: both operands must span less than 2 GiB.
  const int64_t w_rows = (a.epilogue == EPI_SWIGLU) ? (int64_t)a.up_offset + a.N : a.N;
  if (w_rows * a.ldw * 2 >= (int64_t)kOob || (int64_t)total_rows(a.rows) * a.lda * 2 >= (int64_t)kOob)
    return hipErrorInvalidValue;
  // a batch of requests: tiles of 256 (or 128) rows must not straddle two requests
  if (a.rows.batch > 1 && (a.rows.seq_pad % 256) != 0) return hipErrorInvalidValue;
  const bool aligned = (a.K % 8 == 0) && (a.lda % 8 == 0) && (a.ldw % 8 == 0) &&
                       ((reinterpret_cast<uintptr_t>(a.A) & 15) == 0) &&
                       ((reinterpret_cast<uintptr_t>(a.W) & 15) == 0);
  const int out_big = (a.epilogue == EPI_SWIGLU) ? 128 : 256;
  long valid_rows = a.rows.n_valid;
  if (a.rows.batch > 1) {
    valid_rows = 0;
    for (int b = 0; b < a.rows.batch; ++b) valid_rows += (a.rows.req_valid[b] + 255) / 256 * 256;
  }
  // Choose the tile shape by the estimated time of its launch: rounds of tiles over the CUs
  // times the time of one tile. A 256 x 256 direct-to-LDS tile (one per CU) does 4x the work of
  // a 128 x 128 register-staged tile (two per CU) and takes about 1.2x as long per round
  // (measured on the hidden-1024 projections: 28.6 us against 23.8 us per round at K = 1024),
  // so few large tiles can still win over twice as many rounds of small ones.
  const long cus = compute_units();
  const long tiles_big = (long)((valid_rows + 255) / 256) * ((a.N + out_big - 1) / out_big);
  const int out_small = (a.epilogue == EPI_SWIGLU) ? 64 : 128;
  const long tiles_small = (long)((valid_rows + 127) / 128) * ((a.N + out_small - 1) / out_small);
  const double t_big = 1.2 * (double)((tiles_big + cus - 1) / cus);
  const double t_small = (double)((tiles_small + 2 * cus - 1) / (2 * cus));
  const bool big = t_big < t_small;
  if (aligned && big && (a.K % kDlBK) == 0) {
    const int tiles_m = (total_rows(a.rows) + 255) / 256;
    const int tiles_n = (a.N + out_big - 1) / out_big;
    const dim3 grid(tiles_m * tiles_n), block(512);
    const int gm = (a.K >= 2 * a.N) ? 3 : 6;  // token-tiles per group (see select_tile)
    switch (a.epilogue) {
      case EPI_STORE: hipLaunchKernelGGL(k_gemm_dl<EPI_STORE>, grid, block, 0, s, a, tiles_m, tiles_n, gm); break;
      case EPI_GATED_TO_F32: hipLaunchKernelGGL(k_gemm_dl<EPI_GATED_TO_F32>, grid, block, 0, s, a, tiles_m, tiles_n, gm); break;
      case EPI_GATED_F32_IN: hipLaunchKernelGGL(k_gemm_dl<EPI_GATED_F32_IN>, grid, block, 0, s, a, tiles_m, tiles_n, gm); break;
      case EPI_GATED_F32_TO_F32: hipLaunchKernelGGL(k_gemm_dl<EPI_GATED_F32_TO_F32>, grid, block, 0, s, a, tiles_m, tiles_n, gm); break;
      case EPI_SWIGLU: hipLaunchKernelGGL(k_gemm_dl<EPI_SWIGLU>, grid, block, 0, s, a, tiles_m, tiles_n, gm); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  // Small problems, reductions that are not a multiple of 64, and unaligned operands. When the
  // 128 x 128 tiles fit in one round (two per CU) the 64 x 128 tiles of the same kernel spread
  // the work over more CUs (up to three per CU): on the hidden-1024 block (4,608 tokens) the
  // out-projection 26.8 -> 24.8 us and the down projection 57.1 -> 54.6 us, the 640-token block
  // 0.127 -> 0.118 ms, bit-identical (each output sums the same products in the same order).
  if (aligned) {
    if (tiles_small <= 2 * cus) return gemm_dispatch_epi<64, 128, 2, 2, true>(a, s);
    return gemm_dispatch_epi<128, 128, 2, 2, true>(a, s);
  }
  return gemm_dispatch_epi<128, 128, 2, 2, false>(a, s);
}

}  // namespace avdit
