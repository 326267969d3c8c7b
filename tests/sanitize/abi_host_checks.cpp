// Host-side checks of the C-ABI's validation, cache schedule, loop sequencing and error state,
// built together with csrc/abi.cpp under AddressSanitizer and UndefinedBehaviorSanitizer by
// tests/test_host_sanitized.py. No GPU is involved: the kernel launchers are replaced by stubs
// that count launches and return a chosen status, so every path of abi.cpp up to and including
// the launch sequence runs on the CPU.
//
// Output: one "S <mode> <start> <end> <refresh> <max_reuse> <n> <flags>" line per schedule (the
// Python side compares them with the oracle), one "FAIL ..." line per failed check, and a final
// "DONE <checks> <failures>" line. Exit status 1 when a check failed.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <string>
#include <thread>
#include <vector>

#include "../../include/avdit.h"
#include "../../audio_video_diffusion_dit_amd/csrc/kernels.hpp"

// ------------------------------------------------------------------ launcher stubs --------
static int g_launches = 0;
static int g_fail_at = -1;  // launch index that reports a failure (-1: none)

static hipError_t stub_launch() {
  const int i = g_launches++;
  return i == g_fail_at ? hipErrorInvalidValue : hipSuccess;
}

namespace avdit {
hipError_t launch_norm_mod(const NormModArgs&, hipStream_t) { return stub_launch(); }
hipError_t launch_qk_norm_rope(const QkNormRopeArgs&, hipStream_t) { return stub_launch(); }
hipError_t launch_step_update(const StepArgs&, hipStream_t) { return stub_launch(); }
hipError_t launch_gemm(const GemmArgs&, hipStream_t) { return stub_launch(); }
hipError_t launch_head_prep(const HeadPrepArgs&, hipStream_t) { return stub_launch(); }
hipError_t launch_head_proj(const HeadProjArgs&, hipStream_t) { return stub_launch(); }
hipError_t launch_attention(const AttnArgs&, hipStream_t) { return stub_launch(); }
}  // namespace avdit

// ------------------------------------------------------------------ helpers ---------------
static int g_checks = 0, g_failures = 0;

static void expect(bool ok, const char* what, int line) {
  ++g_checks;
  if (!ok) {
    ++g_failures;
    std::printf("FAIL line %d: %s (last error: %s)\n", line, what, dit_last_error());
  }
}
#define EXPECT(c) expect((c), #c, __LINE__)

// A call that must be rejected during validation: the status and no launch.
#define REJECT(call, code)                 \
  do {                                     \
    g_launches = 0;                        \
    const int st_ = (call);                \
    EXPECT(st_ == (code));                 \
    EXPECT(g_launches == 0);               \
    EXPECT(std::strlen(dit_last_error()) > 0); \
  } while (0)

static void* fake(uint64_t a) { return reinterpret_cast<void*>(a); }
template <class T>
static T* fp(uint64_t a) { return reinterpret_cast<T*>(a); }

static dit_dims dims(int D, int H, int Dh, int F) {
  dit_dims d{};
  d.hidden = D; d.heads = H; d.head_dim = Dh; d.ffn = F; d.n_mod = 2;
  d.norm_eps = 1e-6f; d.qk_eps = 1e-6f; d.rope_base = 10000.0f;
  return d;
}

static dit_block_weights weights(uint64_t base = 1 << 16) {
  dit_block_weights w{};
  w.w_qkv = fp<const uint16_t>(base);
  w.w_o = fp<const uint16_t>(base + 0x1000);
  w.w_gate_up = fp<const uint16_t>(base + 0x2000);
  w.w_down = fp<const uint16_t>(base + 0x3000);
  w.norm1_g = fp<const float>(base + 0x4000);
  w.norm2_g = fp<const float>(base + 0x5000);
  w.q_g = fp<const float>(base + 0x6000);
  w.k_g = fp<const float>(base + 0x7000);
  w.ada = fp<const float>(base + 0x8000);
  return w;
}

static dit_cache_policy policy(int mode, double s = 0.2, double e = 0.8, int r = 2, int c = 1) {
  dit_cache_policy p{};
  p.mode = mode; p.start_ratio = s; p.end_ratio = e; p.refresh_interval = r;
  p.max_consecutive_reuse = c; p.threshold = NAN;
  return p;
}

// ------------------------------------------------------------------ checks ----------------
static void schedules() {
  const double ratios[][2] = {{0.2, 0.8}, {0.0, 1.0}, {0.0, 0.0}, {0.5, 0.5}, {0.1, 0.9},
                              {0.25, 0.75}, {0.3, 0.31}, {1.0, 1.0}};
  const int rc[][2] = {{2, 1}, {1, 1}, {3, 2}, {4, 9}, {2, 0}};
  std::vector<uint8_t> hit(200);
  for (int mode : {DIT_CACHE_OFF, DIT_CACHE_VELOCITY, DIT_CACHE_EXTRAPOLATE})
    for (auto& r : ratios)
      for (auto& q : rc)
        for (int n = 0; n <= 120; n += (n < 60 ? 1 : 7)) {
          dit_cache_policy p = policy(mode, r[0], r[1], q[0], q[1]);
          EXPECT(dit_cache_schedule(&p, n, hit.data()) == DIT_OK);
          std::printf("S %d %.2f %.2f %d %d %d ", mode, r[0], r[1], q[0], q[1], n);
          for (int i = 0; i < n; ++i) std::putchar(hit[i] ? '1' : '0');
          std::putchar('\n');
        }
  dit_cache_policy bad = policy(DIT_CACHE_VELOCITY);
  bad.threshold = 0.1;
  REJECT(dit_cache_schedule(&bad, 49, hit.data()), DIT_ERR_UNSUPPORTED);
  bad = policy(DIT_CACHE_VELOCITY, 0.9, 0.1);
  REJECT(dit_cache_schedule(&bad, 49, hit.data()), DIT_ERR_INVALID);
  bad = policy(DIT_CACHE_VELOCITY);
  REJECT(dit_cache_schedule(&bad, 49, nullptr), DIT_ERR_INVALID);
}

static void block_validation() {
  dit_dims d = dims(256, 4, 64, 683);
  dit_layout lay{512, 96, 640, nullptr};
  dit_workspace_map m{};
  const size_t need = dit_workspace_size(&d, &lay, 0, &m);
  EXPECT(need > 0 && m.total == need);
  EXPECT(m.qkv >= m.h + 640 * 256 * 2 && m.act > m.h2 && m.ffn_ld == 688);
  dit_block_weights w = weights();
  void* ws = fake(1ull << 40);
  float* temb = fp<float>(1 << 12);
  uint16_t* x = fp<uint16_t>(1 << 20);
  uint16_t* y = fp<uint16_t>(1 << 22);

  g_launches = 0;
  EXPECT(dit_block_forward(&d, &lay, &w, temb, x, y, 0, ws, need, nullptr) == DIT_OK);
  EXPECT(g_launches == 8);   // norm1, qkv, q/k norm + rope, attention, out, norm2, gate/up, down
  EXPECT(std::strlen(dit_last_error()) == 0);

  REJECT(dit_block_forward(nullptr, &lay, &w, temb, x, y, 0, ws, need, nullptr), DIT_ERR_INVALID);
  dit_dims bad = dims(256, 4, 96, 683);
  REJECT(dit_block_forward(&bad, &lay, &w, temb, x, y, 0, ws, need, nullptr), DIT_ERR_UNSUPPORTED);
  bad = dims(250, 4, 64, 683);
  REJECT(dit_block_forward(&bad, &lay, &w, temb, x, y, 0, ws, need, nullptr), DIT_ERR_INVALID);
  bad = dims(256, 4, 64, 683);
  bad.n_mod = 3;
  REJECT(dit_block_forward(&bad, &lay, &w, temb, x, y, 0, ws, need, nullptr), DIT_ERR_UNSUPPORTED);
  dit_layout short_lay{600, 96, 640, nullptr};
  REJECT(dit_block_forward(&d, &short_lay, &w, temb, x, y, 0, ws, need, nullptr), DIT_ERR_INVALID);
  REJECT(dit_block_forward(&d, &lay, &w, temb, x, y, 7, ws, need, nullptr), DIT_ERR_INVALID);
  REJECT(dit_block_forward(&d, &lay, &w, temb, x, y, 0, ws, need - 1, nullptr), DIT_ERR_WORKSPACE);
  REJECT(dit_block_forward(&d, &lay, &w, temb, x, y, 0, fake((1ull << 40) + 64), need, nullptr),
         DIT_ERR_INVALID);
  REJECT(dit_block_forward(&d, &lay, &w, temb, x, x + 64, 0, ws, need, nullptr), DIT_ERR_INVALID);
  REJECT(dit_block_forward(&d, &lay, &w, temb, x + 4, y, 0, ws, need, nullptr), DIT_ERR_INVALID);
  REJECT(dit_block_forward(&d, &lay, &w, temb + 1, x, y, 0, ws, need, nullptr), DIT_ERR_INVALID);
  dit_block_weights wb = w;
  wb.k_g = fp<const float>(0x6004);
  REJECT(dit_block_forward(&d, &lay, &wb, temb, x, y, 0, ws, need, nullptr), DIT_ERR_INVALID);
  wb = w;
  wb.w_down = nullptr;
  REJECT(dit_block_forward(&d, &lay, &wb, temb, x, y, 0, ws, need, nullptr), DIT_ERR_INVALID);

  // operand spans of 2 GiB or more
  dit_dims h3 = dims(3072, 24, 128, 8192);
  dit_layout huge{120000, 11072, 131072, nullptr};
  EXPECT(dit_workspace_size(&h3, &huge, 0, nullptr) == 0);
  REJECT(dit_block_forward(&h3, &huge, &w, temb, x, y, 0, ws, (size_t)1 << 40, nullptr),
         DIT_ERR_UNSUPPORTED);
  dit_layout qkv_limit{116509, 0, 116509, nullptr};
  REJECT(dit_block_forward(&h3, &qkv_limit, &w, temb, x, y, 0, ws, (size_t)1 << 40, nullptr),
         DIT_ERR_UNSUPPORTED);
  dit_layout ok_limit{116508, 0, 116508, nullptr};
  EXPECT(dit_workspace_size(&h3, &ok_limit, 0, nullptr) > 0);

  // an empty sequence validates and launches nothing
  dit_layout empty{0, 0, 0, nullptr};
  const size_t need0 = dit_workspace_size(&d, &empty, 0, nullptr);
  g_launches = 0;
  EXPECT(dit_block_forward(&d, &empty, &w, temb, x, y, 0, ws, need0, nullptr) == DIT_OK);
  EXPECT(g_launches == 0);

  // a launch the runtime rejects: DIT_ERR_DEVICE and nothing launched after it
  for (int k = 0; k < 8; ++k) {
    g_launches = 0;
    g_fail_at = k;
    EXPECT(dit_block_forward(&d, &lay, &w, temb, x, y, 0, ws, need, nullptr) == DIT_ERR_DEVICE);
    EXPECT(g_launches == k + 1);
    EXPECT(std::strstr(dit_last_error(), "launch failed") != nullptr);
  }
  g_fail_at = -1;
}

static void batched_validation() {
  dit_dims d = dims(3072, 24, 128, 8192);
  dit_block_weights w = weights();
  std::vector<dit_layout> four(4, dit_layout{30720, 2048, 32768, nullptr});
  EXPECT(dit_workspace_size_batched(&d, four.data(), 4, nullptr) == 0);   // SwiGLU rows: 2 GiB
  REJECT(dit_block_forward_batched(&d, four.data(), 4, &w, fp<float>(1 << 12), fp<uint16_t>(1 << 20),
                                   fp<uint16_t>(1ull << 36), 0, fake(1ull << 40), (size_t)1 << 40,
                                   nullptr),
         DIT_ERR_UNSUPPORTED);
  std::vector<dit_layout> many(65, dit_layout{10, 0, 256, nullptr});
  EXPECT(dit_workspace_size_batched(&d, many.data(), 65, nullptr) == 0);
  std::vector<dit_layout> mixed = {{100, 0, 256, nullptr}, {10, 0, 512, nullptr}};
  EXPECT(dit_workspace_size_batched(&d, mixed.data(), 2, nullptr) == 0);
  std::vector<dit_layout> two = {{1000, 24, 1024, nullptr}, {500, 12, 1024, nullptr}};
  const size_t need = dit_workspace_size_batched(&d, two.data(), 2, nullptr);
  EXPECT(need > 0);
  g_launches = 0;
  EXPECT(dit_block_forward_batched(&d, two.data(), 2, &w, fp<float>(1 << 12), fp<uint16_t>(1 << 20),
                                   fp<uint16_t>(1ull << 36), 0, fake(1ull << 40), need,
                                   nullptr) == DIT_OK);
  EXPECT(g_launches == 8);
}

static void loop_checks() {
  dit_dims d = dims(256, 4, 64, 683);
  dit_layout lay{512, 96, 640, nullptr};
  const int B = 2, N = 49;
  dit_block_weights w[B] = {weights(1 << 16), weights(1 << 17)};
  const size_t need = dit_workspace_size(&d, &lay, B, nullptr);
  std::vector<float> sig(N + 1);
  for (int k = 0; k <= N; ++k) sig[k] = (float)(1.0 - (double)k / N);
  float* temb = fp<float>(1 << 12);
  float* x = fp<float>(1 << 24);
  void* ws = fake(1ull << 40);
  std::vector<uint8_t> flags(N);

  for (int mode : {DIT_CACHE_OFF, DIT_CACHE_VELOCITY, DIT_CACHE_EXTRAPOLATE}) {
    dit_cache_policy p = policy(mode);
    dit_loop_stats st{};
    st.step_hit = flags.data();
    g_launches = 0;
    EXPECT(denoise_loop(&d, &lay, w, B, N, sig.data(), sig.data(), temb, &p, x, 0, &st, ws, need,
                        nullptr) == DIT_OK);
    const int calls = mode == DIT_CACHE_OFF ? 49 : 34;
    EXPECT(st.dit_calls == calls && st.cache_hits == N - calls);
    EXPECT(st.executed_blocks == (int64_t)calls * B && st.skipped_blocks == (int64_t)(N - calls) * B);
    const double V = 608, D = 256, F = 683;
    EXPECT(st.useful_flops == (double)calls * B * (8 * V * D * D + 6 * V * D * F + 4 * V * V * D));
    // one latent conversion, 8 launches per executed block, one Euler step per interval
    EXPECT(g_launches == 1 + calls * B * 8 + N);
    int hits = 0;
    for (uint8_t h : flags) hits += h;
    EXPECT(hits == N - calls);
    g_launches = 0;
    EXPECT(denoise_loop_f32(&d, &lay, w, B, N, sig.data(), sig.data(), temb, &p, x, 0, &st, ws,
                            need, nullptr) == DIT_OK);
    EXPECT(g_launches == 1 + calls * B * 8 + N);
  }
  dit_cache_policy p = policy(DIT_CACHE_VELOCITY);
  dit_loop_stats st{};
  REJECT(denoise_loop(&d, &lay, w, 0, N, sig.data(), sig.data(), temb, &p, x, 0, &st, ws, need,
                      nullptr), DIT_ERR_INVALID);
  REJECT(denoise_loop(&d, &lay, w, B, N, sig.data(), sig.data(), temb, &p, x, 0, &st, ws,
                      need - 256, nullptr), DIT_ERR_WORKSPACE);
  std::vector<float> nan_sig(sig);
  nan_sig[17] = NAN;
  REJECT(denoise_loop(&d, &lay, w, B, N, nan_sig.data(), sig.data(), temb, &p, x, 0, &st, ws, need,
                      nullptr), DIT_ERR_INVALID);
  dit_cache_policy thr = policy(DIT_CACHE_VELOCITY);
  thr.threshold = 0.05;
  REJECT(denoise_loop(&d, &lay, w, B, N, sig.data(), sig.data(), temb, &thr, x, 0, &st, ws, need,
                      nullptr), DIT_ERR_UNSUPPORTED);
  REJECT(denoise_loop(&d, &lay, w, B, N, sig.data(), sig.data(), temb + 2, &p, x, 0, &st, ws, need,
                      nullptr), DIT_ERR_INVALID);
  dit_block_weights wb[B] = {weights(1 << 16), weights(1 << 17)};
  wb[1].ada = fp<const float>((1 << 17) + 0x8008);
  REJECT(denoise_loop(&d, &lay, wb, B, N, sig.data(), sig.data(), temb, &p, x, 0, &st, ws, need,
                      nullptr), DIT_ERR_INVALID);
  // a failure in the middle of the loop stops it there
  g_launches = 0;
  g_fail_at = 100;
  EXPECT(denoise_loop(&d, &lay, w, B, N, sig.data(), sig.data(), temb, &p, x, 0, &st, ws, need,
                      nullptr) == DIT_ERR_DEVICE);
  EXPECT(g_launches == 101);
  g_fail_at = -1;
}

static void other_entry_points() {
  dit_layout lay{300, 77, 400, nullptr};
  REJECT(step_update(fp<float>(1 << 20), fp<uint16_t>(1 << 22), nullptr, &lay, 100, -0.1f, -0.1f,
                     nullptr), DIT_ERR_INVALID);
  REJECT(step_update(fp<float>(1 << 20), fp<uint16_t>(1 << 22), nullptr, &lay, 256, INFINITY,
                     -0.1f, nullptr), DIT_ERR_INVALID);
  REJECT(step_update(fp<float>((1 << 20) + 4), fp<uint16_t>(1 << 22), nullptr, &lay, 256, -0.1f,
                     -0.1f, nullptr), DIT_ERR_INVALID);
  g_launches = 0;
  EXPECT(step_update(fp<float>(1 << 20), fp<uint16_t>(1 << 22), nullptr, &lay, 256, -0.1f, -0.1f,
                     nullptr) == DIT_OK);
  EXPECT(g_launches == 1);

  const int32_t valid[2] = {10, 700};
  const uint16_t* q = fp<const uint16_t>(1 << 20);
  uint16_t* o = fp<uint16_t>(1 << 24);
  REJECT(dit_attention_forward(q, q, q, o, 2, 640, 4, 64, 640 * 256, 256, 640 * 256, 256, valid,
                               nullptr, nullptr, 0, nullptr), DIT_ERR_INVALID);
  REJECT(dit_attention_forward(q, q, q, o, 1, 640, 4, 96, 0, 384, 0, 384, valid, nullptr, nullptr,
                               0, nullptr), DIT_ERR_UNSUPPORTED);
  REJECT(dit_attention_forward(q, q, q, o, 1, 116509, 24, 128, 0, 9216, 0, 3072, valid, nullptr,
                               nullptr, 0, nullptr), DIT_ERR_UNSUPPORTED);
  REJECT(dit_attention_forward(q, q, q, o, 1, 640, 4, 64, 0, 256, 0, 256, valid,
                               fp<const float>(1 << 12), nullptr, 0, nullptr), DIT_ERR_INVALID);

  dit_dims d = dims(256, 4, 64, 683);
  dit_layout hl{512, 96, 640, nullptr};
  const size_t need = dit_head_workspace_size(&d, &hl, 64);
  EXPECT(need == (size_t)2 * 256 * 4 + (size_t)2 * 64 * 4);   // the folded table: mul, cst
  dit_head_weights hw{fp<const float>(1 << 12), fp<const float>(1 << 13),
                      fp<const uint16_t>(1 << 16), fp<const float>(1 << 14), 64};
  g_launches = 0;
  EXPECT(dit_velocity_head(&d, &hl, &hw, fp<float>(1 << 15), fp<uint16_t>(1 << 20),
                           fp<float>(1 << 24), fake(1ull << 40), need, nullptr) == DIT_OK);
  EXPECT(g_launches == 2);   // table fold, one projection over both modalities
  dit_head_weights bad = hw;
  bad.out_channels = 60;
  REJECT(dit_velocity_head(&d, &hl, &bad, fp<float>(1 << 15), fp<uint16_t>(1 << 20),
                           fp<float>(1 << 24), fake(1ull << 40), need, nullptr), DIT_ERR_INVALID);
  bad = hw;
  bad.norm_g = fp<const float>((1 << 12) + 4);
  REJECT(dit_velocity_head(&d, &hl, &bad, fp<float>(1 << 15), fp<uint16_t>(1 << 20),
                           fp<float>(1 << 24), fake(1ull << 40), need, nullptr), DIT_ERR_INVALID);
  // the head reads its input through 64-bit addresses: long sequences have no span limit
  dit_dims wide = dims(8192, 64, 128, 8192);
  dit_layout long_l{131072, 0, 131072, nullptr};
  EXPECT(dit_head_workspace_size(&wide, &long_l, 128) == (size_t)2 * 8192 * 4 + (size_t)2 * 128 * 4);
}

// dit_last_error is per thread: a failure on one thread is not seen, or cleared, by another.
static void error_state_is_thread_local() {
  dit_dims bad = dims(250, 4, 64, 683);
  dit_layout lay{10, 0, 16, nullptr};
  EXPECT(dit_workspace_size(&bad, &lay, 0, nullptr) == 0);
  const std::string mine = dit_last_error();
  EXPECT(!mine.empty());
  std::string other = "unset";
  std::thread t([&] {
    dit_dims d = dims(256, 4, 64, 683);
    (void)dit_workspace_size(&d, &lay, 0, nullptr);
    other = dit_last_error();
  });
  t.join();
  EXPECT(other.empty());
  EXPECT(mine == dit_last_error());
}

int main() {
  schedules();
  block_validation();
  batched_validation();
  loop_checks();
  other_entry_points();
  error_state_is_thread_local();
  std::printf("DONE %d %d\n", g_checks, g_failures);
  return g_failures == 0 ? 0 : 1;
}
