// Drives the C ABI's host code (built with the HIP stubs) and the fp64 oracle under
// AddressSanitizer and UndefinedBehaviorSanitizer.  Prints one line per failed expectation
// and exits non-zero if any failed; a sanitizer finding aborts the run by itself.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "../../include/softembed.h"

extern int g_launches;
extern int g_event_records;
extern int g_marked_launches;

extern "C" {
int oracle_row_stats(const float* logits, int64_t ld, int64_t n_rows, int64_t vocab,
                     double* row_max, int32_t* row_argmax, double* row_lse, double* row_entropy);
int oracle_soft_embed(const float* logits, int64_t ld, int64_t n_rows, int64_t vocab, int64_t s,
                      int64_t e, const float* w_f32, const uint16_t* w_bf16, int64_t ld_w,
                      int64_t d, double gamma, int round_p_bf16, double* out, int64_t ld_out);
int oracle_soft_embed_ranges(const float* logits, int64_t ld, int64_t n_rows, int64_t vocab,
                             int64_t s, int64_t e, const int64_t* bounds, int64_t n_ranges,
                             const float* w_f32, const uint16_t* w_bf16, int64_t ld_w,
                             int64_t d, double gamma, int round_q_bf16, double* out,
                             int64_t ld_out);
double oracle_round_bf16(double x);
}

static int failures = 0;
#define EXPECT(cond)                                                              \
  do {                                                                            \
    if (!(cond)) {                                                                \
      std::printf("FAILED %s:%d: %s\n", __FILE__, __LINE__, #cond);               \
      ++failures;                                                                 \
    }                                                                             \
  } while (0)

// placeholder device addresses: 256-byte aligned, never dereferenced by the host code
static void* P(uintptr_t k) { return reinterpret_cast<void*>((uintptr_t)0x100000 * k); }
static float* F(uintptr_t k) { return static_cast<float*>(P(k)); }
static uint16_t* H(uintptr_t k) { return static_cast<uint16_t*>(P(k)); }
static int32_t* I(uintptr_t k) { return static_cast<int32_t*>(P(k)); }

static void abi() {
  const int64_t L = 256, V = 262144, s = 65536, e = 131072, d = 2816;
  const size_t big = (size_t)1 << 40;
  // statistics
  EXPECT(se_row_stats(F(1), V, L, V, F(2), F(3), F(4), I(5), nullptr) == SE_OK);
  EXPECT(se_row_stats(F(1), V - 4, L, V, F(2), F(3), F(4), I(5), nullptr) == SE_ERR_SHAPE);
  EXPECT(se_row_stats(nullptr, V, L, V, F(2), F(3), F(4), I(5), nullptr) == SE_ERR_NULL);
  EXPECT(se_row_stats(F(1), V, 0, V, nullptr, nullptr, nullptr, nullptr, nullptr) == SE_OK);
  // probabilities
  EXPECT(se_probs_bf16(F(1), V, F(2), L, V, s, e, H(3), V, nullptr) == SE_OK);
  EXPECT(se_probs_bf16(F(1), V, F(2), L, V, s + 4, e, H(3), V, nullptr) == SE_ERR_ALIGN);
  EXPECT(se_probs_bf16(F(1), V, F(2), 70000, V, s, e, H(3), V, nullptr) == SE_OK);
  // workspace sizes and the contraction
  const size_t ws = se_soft_embed_workspace_bytes(L, s, e, d);
  EXPECT(ws == (size_t)23 * 11 * 256 * 256 * 4);
  EXPECT(se_soft_embed_splits(L, s, e, d) == 23);
  EXPECT(se_soft_embed_splits(0, s, e, d) == 0);
  EXPECT(se_soft_embed(H(1), V, L, V, s, e, H(2), e - s, d, d, 53.f, F(3), d, P(4), ws,
                       nullptr) == SE_OK);
  EXPECT(se_soft_embed(H(1), V, L, V, s, e, H(2), e - s, d, d, 53.f, F(3), d, P(4), ws - 1,
                       nullptr) == SE_ERR_WORKSPACE);
  EXPECT(se_soft_embed(H(1), V, L, V, 0, V, H(2), e - s, d, d, 53.f, F(3), d, P(4), big,
                       nullptr) == SE_ERR_SLICE);
  EXPECT(se_soft_embed_fused(F(1), V, F(2), L, V, s, e, H(3), e - s, d, d, 53.f, F(4), d, P(5),
                             big, nullptr) == SE_OK);
  EXPECT(se_soft_embed_fused(F(1), V, F(2), L, V, s, s, H(3), e - s, d, d, 53.f, F(4), d,
                             nullptr, 0, nullptr) == SE_OK);          // empty slice: zeros
  EXPECT(se_soft_embed_fused(F(1), 4210496, F(2), L, V, s, e, H(3), e - s, d, d, 53.f, F(4), d,
                             P(5), big, nullptr) == SE_ERR_SHAPE);    // 32-bit offsets
  // staged, step, one-read step, one-pass, e4m3
  const size_t wss = se_soft_embed_staged_workspace_bytes(L, s, e, d);
  EXPECT(se_soft_embed_staged(F(1), V, F(2), L, V, s, e, H(3), e - s, d, d, 53.f, F(4), d, P(5),
                              wss, nullptr) == SE_OK);
  EXPECT(se_soft_embed_step(F(1), V, L, V, s, e, H(3), e - s, d, d, 53.f, F(4), d, F(6), F(7),
                            F(8), I(9), P(5), wss, nullptr) == SE_OK);
  EXPECT(se_soft_embed_step(F(1), V, 8192, V, 0, V, H(3), V, d, d, 53.f, F(4), d, F(6), F(7),
                            F(8), I(9), P(5), big, nullptr) == SE_ERR_SHAPE);
  EXPECT(se_soft_embed_step(F(1), V, L, V, s, s, H(3), 0, d, d, 53.f, F(4), d, F(6), F(7), F(8),
                            I(9), nullptr, 0, nullptr) == SE_OK);
  const size_t ws1 = se_soft_embed_step_onepass_workspace_bytes(L, V, s, e, d);
  EXPECT(ws1 > wss);
  EXPECT(se_soft_embed_step_onepass(F(1), V, L, V, s, e, H(3), e - s, d, d, 53.f, F(4), d, F(6),
                                    F(7), F(8), I(9), P(5), ws1, nullptr) == SE_OK);
  EXPECT(se_soft_embed_step_onepass(F(1), V, 2048, V, 0, V, H(3), V, d, d, 53.f, F(4), d, F(6),
                                    F(7), F(8), I(9), P(5), big, nullptr) == SE_OK);
  const size_t wso = se_soft_embed_onepass_workspace_bytes(L, 0, V, d);
  EXPECT(se_soft_embed_onepass(F(1), V, L, V, 0, V, H(3), V, d, d, 53.f, F(4), d, F(6), F(7),
                               F(8), I(9), P(5), wso, nullptr) == SE_OK);
  EXPECT(se_soft_embed_onepass(F(1), V, L, V, 8, 8, H(3), V, d, d, 53.f, F(4), d, F(6), F(7),
                               F(8), I(9), P(5), wso, nullptr) == SE_ERR_SLICE);
  EXPECT(se_quantize_table_fp8(H(1), d, e - s, d, static_cast<uint8_t*>(P(2)), d, F(3),
                               nullptr) == SE_OK);
  EXPECT(se_soft_embed_step_fp8(F(1), V, L, V, s, e, static_cast<uint8_t*>(P(3)), F(10), e - s,
                                d, d, 53.f, F(4), d, F(6), F(7), F(8), I(9), P(5), wss,
                                nullptr) == SE_OK);
  EXPECT(se_soft_embed_fp8(H(1), V, L, V, s, e, static_cast<uint8_t*>(P(3)), nullptr, e - s, d,
                           d, 53.f, F(4), d, P(5), big, nullptr) == SE_ERR_NULL);
  // the one-read e4m3 step: 16-byte aligned scales, its workspace; a 4-byte offset is refused
  EXPECT(se_soft_embed_step_onepass_fp8(F(1), V, L, V, s, e, static_cast<uint8_t*>(P(3)), F(10),
                                        e - s, d, d, 53.f, F(4), d, F(6), F(7), F(8), I(9), P(5),
                                        ws1, nullptr) == SE_OK);
  EXPECT(se_soft_embed_step_onepass_fp8(F(1), V, L, V, s, e, static_cast<uint8_t*>(P(3)),
                                        F(10) + 1, e - s, d, d, 53.f, F(4), d, F(6), F(7), F(8),
                                        I(9), P(5), ws1, nullptr) == SE_ERR_ALIGN);
  // slices, sampler, partial sums
  EXPECT(se_merge_slices(F(1), 4, L * d, L, d, d, F(2), F(3), F(4), I(5), F(6), d, F(7), F(8),
                         F(9), I(10), nullptr) == SE_OK);
  EXPECT(se_accept_converge(F(1), I(2), 1, 256, 8.0, 3, 0.05, 64, static_cast<uint8_t*>(P(3)),
                            I(4), I(5), I(6), static_cast<uint8_t*>(P(7)),
                            static_cast<uint8_t*>(P(8)), nullptr) == SE_OK);
  EXPECT(se_accept_converge(F(1), I(2), 1, 2048, 8.0, 3, 0.05, 64, static_cast<uint8_t*>(P(3)),
                            I(4), I(5), I(6), static_cast<uint8_t*>(P(7)),
                            static_cast<uint8_t*>(P(8)), nullptr) == SE_ERR_SHAPE);
  EXPECT(se_reduce_partials(F(1), 4, L * d, L, d, d, F(2), d, H(3), d, nullptr) == SE_OK);
  // launch markers: two events (start, end) per launch, in order, until fewer than two
  // remain; the dispatch stamps them, so nothing is recorded on the stream
  std::vector<void*> ev(5, P(20));
  EXPECT(se_set_launch_events(ev.data(), 5) == SE_OK);
  const int rec0 = g_event_records, marked0 = g_marked_launches;
  EXPECT(se_soft_embed_step_onepass(F(1), V, L, V, s, e, H(3), e - s, d, d, 53.f, F(4), d, F(6),
                                    F(7), F(8), I(9), P(5), ws1, nullptr) == SE_OK);
  EXPECT(se_launch_events_used() == 4);
  EXPECT(g_marked_launches - marked0 == 2);
  EXPECT(g_event_records - rec0 == 0);
  EXPECT(se_set_launch_events(nullptr, 0) == SE_OK && se_launch_events_used() == 0);
  EXPECT(se_set_launch_events(nullptr, -1) == SE_ERR_SHAPE);
  EXPECT(g_launches > 30);
}

static void oracle() {
  // small seeded rows, including V = 1, an empty slice and ranges
  const int64_t L = 3, V = 37, d = 5;
  std::vector<float> x(L * V), w(V * d);
  uint32_t r = 12345u;
  auto rnd = [&r]() {
    r = r * 1664525u + 1013904223u;
    return (float)((r >> 8) & 0xFFFF) / 65536.f - 0.5f;
  };
  for (auto& v : x) v = 6.f * rnd();
  for (auto& v : w) v = rnd();
  std::vector<double> mx(L), lse(L), h(L), out(L * d), out2(L * d);
  std::vector<int32_t> am(L);
  EXPECT(oracle_row_stats(x.data(), V, L, V, mx.data(), am.data(), lse.data(), h.data()) == 0);
  EXPECT(oracle_soft_embed(x.data(), V, L, V, 3, 30, w.data(), nullptr, d, d, 2.0, 0,
                           out.data(), d) == 0);
  const int64_t b[4] = {3, 10, 11, 30};
  EXPECT(oracle_soft_embed_ranges(x.data(), V, L, V, 3, 30, b, 3, w.data(), nullptr, d, d, 2.0,
                                  0, out2.data(), d) == 0);
  for (int64_t i = 0; i < L * d; ++i) EXPECT(std::fabs(out[i] - out2[i]) < 1e-12);
  EXPECT(oracle_soft_embed(x.data(), V, L, V, 7, 7, w.data(), nullptr, d, d, 2.0, 1,
                           out.data(), d) == 0);
  for (int64_t i = 0; i < L * d; ++i) EXPECT(out[i] == 0.0);
  EXPECT(oracle_row_stats(x.data(), V, L, 1, mx.data(), am.data(), lse.data(), h.data()) == 0);
  EXPECT(h[0] == 0.0 && am[0] == 0);
  const int64_t bad[3] = {3, 3, 30};
  EXPECT(oracle_soft_embed_ranges(x.data(), V, L, V, 3, 30, bad, 2, w.data(), nullptr, d, d, 1.0,
                                  0, out.data(), d) == 4);
  x[5] = INFINITY;
  EXPECT(oracle_row_stats(x.data(), V, L, V, mx.data(), am.data(), lse.data(), h.data()) == 1);
  EXPECT(oracle_round_bf16(1.0 + 1.0 / 512) == 1.0);
  EXPECT(oracle_round_bf16(1.0 + 3.0 / 512) == 1.0 + 4.0 / 512);
}

int main() {
  abi();
  oracle();
  std::printf("%s: %d failed expectations\n", failures ? "FAIL" : "OK", failures);
  return failures ? 1 : 0;
}
