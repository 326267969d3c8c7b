// Velocity head in one pass over the stack output (1Cat-vLLM PR #584, "Test Result": the model
// ends in a final AdaLN layer; TeleFuser PR #38, section 1: the DiT predicts the flow-matching
// velocity). For a valid row l of modality m the head computes
//   v_l = (x_l / sqrt(mean(x_l^2) + eps) * g * (1 + scale_m) + shift_m) W_m^T + b_m,
// which is evaluated here as
//   v_l = r_l ((x_l * mul_m) W_m^T) + cst_m,   r_l = 1 / sqrt(mean(x_l^2) + eps),
//   mul_m = g * (1 + scale_m),                  cst_m = shift_m W_m^T + b_m,
// so that x is read once and nothing of size [rows, D] is written back: the product runs on
// MFMA with x * mul_m rounded to bf16 (fp32 multiply, one rounding), while r_l, the shift term
// and the bias stay fp32. k_head_prep folds the table into mul and cst; k_head_proj streams
// x from memory into LDS several k-tiles ahead (the kernel is bound by reading x), rescales and
// rounds it there, takes each row's sum of squares from the same values, and writes
// v = r acc + cst in fp32, zeros for rows past the valid ones.
#include "common.hpp"
#include "kernels.hpp"

namespace avdit {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char_h;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4_h;
typedef __attribute__((address_space(3))) u32x2 lds_u32x2_h;

namespace {

constexpr uint32_t kHeadOob = 0x80000000u;      // buffer offset past every range: reads zero
constexpr int32_t kHeadRsrcWord3 = 0x00020000;  // raw buffer resource, 32-bit elements
constexpr int kHeadBK = 64;                     // k per tile
constexpr int kHeadBN = 128;                    // output channels per workgroup
constexpr int kHeadRowB = kHeadBK * 2;          // bytes of one 64-wide bf16 LDS row
constexpr int kHeadMaxD = 8192;                 // the folded scale of a row lives in LDS

// Raw buffer resource in scalar registers (its words are wave-uniform by construction).
__device__ __forceinline__ i32x4 head_rsrc(const void* p, uint32_t bytes) {
  const uint64_t ad = reinterpret_cast<uint64_t>(p);
  return i32x4{__builtin_amdgcn_readfirstlane((int32_t)(uint32_t)ad),
               __builtin_amdgcn_readfirstlane((int32_t)(uint32_t)(ad >> 32)),
               __builtin_amdgcn_readfirstlane((int32_t)bytes), kHeadRsrcWord3};
}
// 16 bytes per lane from memory straight into LDS at lds_base + 16 lane; offsets past the
// resource range read as zero. Completion is awaited with explicit vmcnt waits.
__device__ __forceinline__ void head_dl_b128(uint32_t lds_base, uint32_t voffset, i32x4 rsrc) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(lds_base), "v"(voffset), "s"(rsrc)
               : "memory", "m0");
}
// Chunk swizzle of a 128-byte LDS row (as in the block GEMMs): the 16 rows read at one logical
// chunk land on 16 distinct 16-byte bank groups.
__device__ __forceinline__ int head_swz(int r) { return (r >> 1) & 7; }

template <int N>
__device__ __forceinline__ void head_wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x70 | 0xF00);
}

}  // namespace

// mul[m][d] = g[d] (1 + (ada[m][1][d] + temb[m][1][d])) for d < D, m < 2; then, one wave per
// (m, c): cst[m][c] = sum_d (ada[m][0][d] + temb[m][0][d]) W[m][c][d] + b[m][c], 8 elements of d
// per lane and step.
__global__ __launch_bounds__(256) void k_head_prep(HeadPrepArgs a) {
  const int D = a.D, C = a.C;
  const int tid = blockIdx.x * blockDim.x + threadIdx.x;
  if (blockIdx.y == 0) {
    for (int i = tid; i < 2 * D; i += gridDim.x * blockDim.x) {
      const int m = i / D, d = i - m * D;
      const float sc = a.ada[(size_t)(2 * m + 1) * D + d] + a.temb[(size_t)(2 * m + 1) * D + d];
      a.mul[i] = a.gain[d] * (1.0f + sc);
    }
    return;
  }
  const int wave = tid >> 6, lane = threadIdx.x & 63;
  if (wave >= 2 * C) return;
  const int m = wave / C, c = wave - m * C;
  const float* sa = a.ada + (size_t)(2 * m) * D;
  const float* st = a.temb + (size_t)(2 * m) * D;
  const uint16_t* w = a.w + ((size_t)m * C + c) * D;
  float s = 0.0f;
  for (int d = lane * 8; d < D; d += 512) {
    const u32x4 wv = *reinterpret_cast<const u32x4*>(w + d);
    const f32x4 a0 = *reinterpret_cast<const f32x4*>(sa + d), a1 = *reinterpret_cast<const f32x4*>(sa + d + 4);
    const f32x4 t0 = *reinterpret_cast<const f32x4*>(st + d), t1 = *reinterpret_cast<const f32x4*>(st + d + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float sh0 = (e < 2 ? a0[2 * e] + t0[2 * e] : a1[2 * e - 4] + t1[2 * e - 4]);
      const float sh1 = (e < 2 ? a0[2 * e + 1] + t0[2 * e + 1] : a1[2 * e - 3] + t1[2 * e - 3]);
      s = fmaf(sh0, bf_lo(wv[e]), s);
      s = fmaf(sh1, bf_hi(wv[e]), s);
    }
  }
  s = wave_sum(s);
  if (lane == 0) a.cst[wave] = s + (a.bias ? a.bias[wave] : 0.0f);
}

// One workgroup: BM rows x 128 channels of v of one modality (workgroups [0, tiles0) take the
// video rows, the rest the audio rows), 4 waves (2 x 2) of (BM / 2) rows x 64 channels.
// Weights are the MFMA A operand (lane = 4 consecutive channels of one row in the result).
// Every operand goes from memory straight into LDS, so that only the explicit waits below track
// the loads in flight:
//   - x tile t lands in ring stage t % XRING. bf16 rows land in the MFMA layout and each lane
//     rescales the 16 bytes it loaded in place (x * mul, rounded to bf16); fp32 rows land as
//     loaded and each lane writes its 4 rescaled values into x-stage t % 2.
//   - weight tile t lands in ring stage t % WS.
// Iteration kt rescales tile kt + 1 while it multiplies tile kt; one barrier then publishes
// tile kt + 1 and frees tile kt's stages, which take x tile kt + XRING and weight tile kt + WS.
// Each lane adds the squares of the x values it rescales to its rows' sums.
template <bool F32IN, int BM>
__global__ __launch_bounds__(256) void k_head_proj(HeadProjArgs a) {
  constexpr int XRING = F32IN ? 3 : 4;           // x tiles resident or in flight
  // weight tiles resident or in flight: two for 64-row bf16 tiles, so that two workgroups fit in
  // a CU's LDS (measured 74-77 -> 71 us on the 32k-token head against one 128-row workgroup per CU)
  constexpr int WS = (!F32IN && BM == 64) ? 2 : 3;
  constexpr int ESZ = F32IN ? 4 : 2;
  constexpr int W_STAGE = kHeadBN * kHeadRowB;   // 16 KB
  constexpr int XRAW = BM * kHeadBK * ESZ;       // one x tile as loaded
  constexpr int XBF = BM * kHeadRowB;            // one x tile in bf16 (fp32 input only)
  constexpr int CPR = kHeadBK * ESZ / 16;        // 16-byte chunks per loaded row: 8 or 16
  constexpr int RPW = 64 / CPR;                  // rows per wave load: 8 or 4
  constexpr int NXL = BM / (RPW * 4);            // x loads per wave per tile
  constexpr int NW = 4;                          // weight loads per wave per tile
  constexpr int WM = 2, WN = 2, TM = BM / WM, TN = kHeadBN / WN, MT = TM / 32, FT = TN / 32;
  static_assert(XRING * XRAW + (F32IN ? 2 * XBF : 0) + WS * W_STAGE + 4 * (BM + kHeadMaxD) <= 160 * 1024,
                "LDS budget");
  static_assert(XRING >= WS, "an x tile is never issued after its weight tile");
  __shared__ u32x4 smem[(XRING * XRAW + (F32IN ? 2 * XBF : 0) + WS * W_STAGE) / 16];
  __shared__ float rsq[BM];
  extern __shared__ f32x4 mul_s[];  // mul of this modality: D floats of dynamic LDS

  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hh = lane >> 5, wave = tid >> 6;
  const int wm = wave % WM, wn = wave / WM;
  const int m = (int)blockIdx.x < a.tiles0 ? 0 : 1;
  const int rows = a.rows[m], valid = a.valid[m];
  const int D = a.D, C = a.C;
  const int r0 = ((int)blockIdx.x - (m ? a.tiles0 : 0)) * BM;  // first row (within the modality)
  const int c0 = blockIdx.y * kHeadBN;                          // first channel
  const int nk = D / kHeadBK;
  const float* mulp = a.mul[m];
  const float* cstp = a.cst[m];

  lds_char_h* lds = (lds_char_h*)(smem);
  lds_char_h* xring = lds;
  lds_char_h* xbf = lds + XRING * XRAW;                       // fp32 input only
  lds_char_h* wring = xbf + (F32IN ? 2 * XBF : 0);

  // ---- weights: wave w's load i fills rows 8 (4 i + w) .. + 7 of the 128-channel tile ----
  const i32x4 rs_w = head_rsrc(a.w[m], (uint32_t)((int64_t)C * D * 2));
  uint32_t woff[NW];
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const int r = 8 * (4 * i + wave) + lane / 8;
    const int kc = (lane % 8) ^ head_swz(r);
    woff[i] = (c0 + r < C) ? (uint32_t)((int64_t)(c0 + r) * D * 2 + kc * 16) : kHeadOob;
  }
  const uint32_t wlds = (uint32_t)__builtin_amdgcn_readfirstlane(
      (int)(uint32_t)(uintptr_t)wring + wave * 1024);
  auto issue_w = [&](int kt) __attribute__((always_inline)) {
    const uint32_t sb = wlds + (uint32_t)(kt % WS) * W_STAGE;
#pragma unroll
    for (int i = 0; i < NW; ++i) head_dl_b128(sb + i * 4 * 1024, woff[i] + (uint32_t)kt * kHeadRowB, rs_w);
  };

  // ---- x: the resource covers only this workgroup's valid rows (rows past them read zero) ----
  const int nvr = max(0, min(BM, valid - r0));
  const i32x4 rs_x = head_rsrc(static_cast<const char*>(a.x[m]) + (size_t)r0 * D * ESZ,
                               (uint32_t)((int64_t)nvr * D * ESZ));
  int xrow[NXL];
  uint32_t xoff[NXL];
#pragma unroll
  for (int i = 0; i < NXL; ++i) {
    xrow[i] = RPW * (4 * i + wave) + lane / CPR;
    const int pc = lane % CPR;
    const int kc = F32IN ? pc : (pc ^ head_swz(xrow[i]));   // bf16 rows land swizzled
    xoff[i] = (uint32_t)((int64_t)xrow[i] * D * ESZ + kc * 16);
  }
  const uint32_t xlds = (uint32_t)__builtin_amdgcn_readfirstlane(
      (int)(uint32_t)(uintptr_t)xring + wave * 1024);
  auto issue_x = [&](int kt) __attribute__((always_inline)) {
    const uint32_t sb = xlds + (uint32_t)(kt % XRING) * XRAW;
#pragma unroll
    for (int i = 0; i < NXL; ++i)
      head_dl_b128(sb + i * 4 * 1024, xoff[i] + (uint32_t)kt * (kHeadBK * ESZ), rs_x);
  };
  float ss[NXL];
#pragma unroll
  for (int i = 0; i < NXL; ++i) ss[i] = 0.0f;
  // x * mul rounded to bf16 for the lane's own chunks of tile kt (after its loads landed)
  auto stage_x = [&](int kt) __attribute__((always_inline)) {
    lds_char_h* raw = xring + (kt % XRING) * XRAW + wave * 1024 + lane * 16;
#pragma unroll
    for (int i = 0; i < NXL; ++i) {
      const u32x4 w = *reinterpret_cast<lds_u32x4_h*>(raw + i * 4 * 1024);
      if (F32IN) {
        const int q = lane % CPR;                  // fp32 chunk: k = 4 q .. 4 q + 3
        const f32x4 mq = mul_s[(kt * kHeadBK) / 4 + q];
        float x[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[e] = __uint_as_float(w[e]);
          ss[i] = fmaf(x[e], x[e], ss[i]);
        }
        const uint32_t lo = pack_bf16x2(x[0] * mq[0], x[1] * mq[1]);
        const uint32_t hi = pack_bf16x2(x[2] * mq[2], x[3] * mq[3]);
        const int row = xrow[i];
        lds_char_h* dst = xbf + (kt & 1) * XBF + row * kHeadRowB +
                          (((q >> 1) ^ head_swz(row)) * 16) + (q & 1) * 8;
        *reinterpret_cast<lds_u32x2_h*>(dst) = u32x2{lo, hi};
      } else {
        const int kc = (lane % CPR) ^ head_swz(xrow[i]);   // logical chunk held by this lane
        const f32x4 m0 = mul_s[(kt * kHeadBK + kc * 8) / 4];
        const f32x4 m1 = mul_s[(kt * kHeadBK + kc * 8) / 4 + 1];
        const float mv[8] = {m0[0], m0[1], m0[2], m0[3], m1[0], m1[1], m1[2], m1[3]};
        u32x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float x0 = bf_lo(w[e]), x1 = bf_hi(w[e]);
          ss[i] = fmaf(x0, x0, ss[i]);
          ss[i] = fmaf(x1, x1, ss[i]);
          o[e] = pack_bf16x2(x0 * mv[2 * e], x1 * mv[2 * e + 1]);
        }
        *reinterpret_cast<lds_u32x4_h*>(raw + i * 4 * 1024) = o;
      }
    }
  };

  // ---- MFMA fragments: k-step s reads logical chunk 2 s + hh of rows l32 + 32 (f or t), one
  // k-step ahead of its MFMAs ----
  const int sw = head_swz(l32);
  int foff[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) foff[s] = l32 * kHeadRowB + ((2 * s + hh) ^ sw) * 16;
  f32x16 acc[FT][MT];
#pragma unroll
  for (int f = 0; f < FT; ++f)
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[f][t][e] = 0.0f;
  auto mma_tile = [&](int kt) __attribute__((always_inline)) {
    lds_char_h* wst = wring + (kt % WS) * W_STAGE;
    lds_char_h* xst = F32IN ? xbf + (kt & 1) * XBF : xring + (kt % XRING) * XRAW;
    bf16x8 af[2][FT], bfr[2][MT];
    auto rd = [&](int s, int slot) __attribute__((always_inline)) {
#pragma unroll
      for (int f = 0; f < FT; ++f)
        af[slot][f] = __builtin_bit_cast(bf16x8, *reinterpret_cast<lds_u32x4_h*>(wst + (wn * TN + f * 32) * kHeadRowB + foff[s]));
#pragma unroll
      for (int t = 0; t < MT; ++t)
        bfr[slot][t] = __builtin_bit_cast(bf16x8, *reinterpret_cast<lds_u32x4_h*>(xst + (wm * TM + t * 32) * kHeadRowB + foff[s]));
    };
    rd(0, 0);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      if (s + 1 < 4) rd(s + 1, (s + 1) & 1);
#pragma unroll
      for (int f = 0; f < FT; ++f)
#pragma unroll
        for (int t = 0; t < MT; ++t)
          acc[f][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[s & 1][f], bfr[s & 1][t], acc[f][t], 0, 0, 0);
    }
  };

  // ---- pipeline. Issue order: x tiles 0 .. XRING - 1 and weight tiles 0 .. WS - 1, then after
  // the barrier of iteration kt: x tile kt + XRING and weight tile kt + WS (each if it exists).
  // Loads complete in issue order and every x tile is issued no later than its weight tile, so
  // tile t has landed once at most the loads issued after weight tile t are in flight; that
  // count is exact below and the wait takes the largest available bound not above it. ----
  for (int t = 0; t < XRING && t < nk; ++t) issue_x(t);
  for (int t = 0; t < WS && t < nk; ++t) issue_w(t);
  // the folded scale into LDS, all loads of it at once (their wait also covers the tiles above)
  {
    constexpr int MPT = kHeadMaxD / 4 / 256;
    f32x4 mv[MPT];
#pragma unroll
    for (int k = 0; k < MPT; ++k)  // unconditional loads (clamped index): one wait for all
      mv[k] = *reinterpret_cast<const f32x4*>(mulp + 4 * min(tid + 256 * k, D / 4 - 1));
#pragma unroll
    for (int k = 0; k < MPT; ++k)
      if (tid + 256 * k < D / 4) mul_s[tid + 256 * k] = mv[k];
  }
  auto wait_tile = [&](int t) __attribute__((always_inline)) {
    int n = 0;  // loads issued after weight tile t
    if (t < WS) {
      n += max(0, min(WS, nk) - (t + 1)) * NW;       // later weight tiles of the prologue
      for (int j = 0; j < t - 1; ++j)                // iterations 0 .. t - 2 (issued before t - 1 waits)
        n += (j + XRING < nk ? NXL : 0) + (j + WS < nk ? NW : 0);
    } else {
      for (int j = t - WS + 1; j < t - 1; ++j)
        n += (j + XRING < nk ? NXL : 0) + (j + WS < nk ? NW : 0);
    }
    constexpr int G = NXL + NW, LO = NXL < NW ? NXL : NW, HI = NXL < NW ? NW : NXL;
    if (n >= 2 * G) head_wait_vm<2 * G>();
    else if (n >= G) head_wait_vm<G>();
    else if (n >= HI) head_wait_vm<HI>();
    else if (n >= LO) head_wait_vm<LO>();
    else head_wait_vm<0>();
  };
  __syncthreads();  // mul_s
  wait_tile(0);
  stage_x(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    if (kt + 1 < nk) {
      wait_tile(kt + 1);
      stage_x(kt + 1);
    }
    mma_tile(kt);
    __syncthreads();  // tile kt + 1 published; tile kt's stages free
    if (kt + XRING < nk) issue_x(kt + XRING);
    if (kt + WS < nk) issue_w(kt + WS);
  }

  // ---- this lane's constants (loaded once, before any store: a load behind the stores would
  // wait for them), then the row scales from the lanes holding each row's chunks ----
  float4 kv[FT][4];
#pragma unroll
  for (int f = 0; f < FT; ++f)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = c0 + wn * TN + f * 32 + 8 * j + 4 * hh;
      kv[f][j] = *reinterpret_cast<const float4*>(cstp + min(c, C - 4));  // clamped: unconditional
    }
  // consumed here, before the first store: the compiler's wait for these loads lands once, here,
  // instead of before every store (behind which it could no longer count on load order)
#pragma unroll
  for (int f = 0; f < FT; ++f)
#pragma unroll
    for (int j = 0; j < 4; ++j) asm volatile("" ::"v"(kv[f][j].x), "v"(kv[f][j].y), "v"(kv[f][j].z), "v"(kv[f][j].w));
#pragma unroll
  for (int i = 0; i < NXL; ++i) {
    float v = ss[i];
#pragma unroll
    for (int o = 1; o < CPR; o <<= 1) v += __shfl_xor(v, o, 64);
    if (lane % CPR == 0) rsq[xrow[i]] = rsqrtf(v / (float)D + a.eps);
  }
  __syncthreads();

  // ---- v = r acc + cst (fp32) for valid rows, 0 for rows past them ----
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const int row = wm * TM + t * 32 + l32;
    const int grow = r0 + row;
    if (grow >= rows) continue;
    const bool ok = grow < valid;
    const float r = rsq[row];
    float* out = a.v[m] + (size_t)grow * a.ldv;
#pragma unroll
    for (int f = 0; f < FT; ++f)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int c = c0 + wn * TN + f * 32 + 8 * j + 4 * hh;
        if (c >= C) continue;
        float4 o = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        if (ok) {
          const float4 k = kv[f][j];
          o.x = fmaf(r, acc[f][t][4 * j + 0], k.x);
          o.y = fmaf(r, acc[f][t][4 * j + 1], k.y);
          o.z = fmaf(r, acc[f][t][4 * j + 2], k.z);
          o.w = fmaf(r, acc[f][t][4 * j + 3], k.w);
        }
        *reinterpret_cast<float4*>(out + c) = o;
      }
  }
}

hipError_t launch_head_prep(const HeadPrepArgs& a, hipStream_t s) {
  if (a.D <= 0 || (a.D & 7) != 0 || a.C <= 0) return hipErrorInvalidValue;
  const int mul_blocks = (2 * a.D + 255) / 256;
  const int cst_blocks = (2 * a.C + 3) / 4;  // 4 waves per block, one wave per (m, c)
  const int gx = mul_blocks > cst_blocks ? mul_blocks : cst_blocks;
  hipLaunchKernelGGL(k_head_prep, dim3(gx, 2), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_head_proj(const HeadProjArgs& a, hipStream_t s) {
  if (a.D <= 0 || (a.D % kHeadBK) != 0 || a.D > kHeadMaxD || a.C <= 0 || (a.C & 7) != 0 ||
      (a.ldv & 3) != 0)
    return hipErrorInvalidValue;
  for (int m = 0; m < 2; ++m)
    if (a.rows[m] < 0 || a.valid[m] < 0 || a.valid[m] > a.rows[m]) return hipErrorInvalidValue;
  const int ny = (a.C + kHeadBN - 1) / kHeadBN;
  // 64-row tiles: for bf16 rows two workgroups share a CU (8 waves streaming x)
  const int bm = 64;
  HeadProjArgs b = a;
  b.tiles0 = (a.rows[0] + bm - 1) / bm;
  const int tiles = b.tiles0 + (a.rows[1] + bm - 1) / bm;
  if (tiles == 0) return hipSuccess;
  const dim3 grid(tiles, ny);
  const size_t dyn = (size_t)a.D * sizeof(float);  // the folded scale of the modality
  if (a.x_f32) hipLaunchKernelGGL((k_head_proj<true, 64>), grid, dim3(256), dyn, s, b);
  else hipLaunchKernelGGL((k_head_proj<false, 64>), grid, dim3(256), dyn, s, b);
  return hipGetLastError();
}

}  // namespace avdit
