// Host-side checks of libdiffattn's argument validation, built with AddressSanitizer and
// UndefinedBehaviorSanitizer (host code only; g++ compiles api.cpp for this driver).
// Every call here is rejected, or is an empty problem, before any HIP call, so no GPU is
// needed. Tensor pointers are fake addresses that the library must never dereference.
// Exit status 0 when every expected status comes back; a sanitizer report aborts.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <limits>

#include "diffattn.h"

static int g_fail = 0;
#define EXPECT(expr, want)                                                              \
  do {                                                                                  \
    const int got_ = static_cast<int>(expr);                                            \
    if (got_ != static_cast<int>(want)) {                                               \
      std::fprintf(stderr, "%s:%d: %s = %d, expected %d\n", __FILE__, __LINE__, #expr,  \
                   got_, static_cast<int>(want));                                       \
      ++g_fail;                                                                         \
    }                                                                                   \
  } while (0)

static const uintptr_t A = uintptr_t(1) << 32;
static void* addr(int i) { return reinterpret_cast<void*>(A * (i + 1)); }
static void* at(uintptr_t x) { return reinterpret_cast<void*>(x); }

static diffattn_problem prob(int64_t b, int64_t h, int64_t n, int32_t d, int32_t t) {
  diffattn_problem p;
  std::memset(&p, 0, sizeof(p));
  p.batch = b; p.heads = h; p.seqlen = n; p.head_dim = d; p.causal = 1;
  p.rms_eps = 1e-5f; p.dtype = t; p.out_layout = DIFFATTN_LAYOUT_BHN; p.kv_heads = 0;
  return p;
}

static diffattn_status fwd(const diffattn_problem* p, void** x, const diffattn_saved* sv,
                           void* ws, size_t wsb) {
  return diffattn_fwd(p, x[0], x[1], x[2], x[3], x[4],
                      static_cast<const diffattn_lambda_state*>(x[5]),
                      static_cast<const float*>(x[6]), x[7], sv, ws, wsb, nullptr);
}

int main() {
  // status strings, including an unknown code
  for (int s = 0; s <= 5; ++s)
    if (std::strncmp(diffattn_status_string(static_cast<diffattn_status>(s)), "DIFFATTN_", 9))
      ++g_fail;
  EXPECT(diffattn_last_hip_error(), 0);

  // problem descriptor checks through the forward
  void* x[8];
  for (int i = 0; i < 8; ++i) x[i] = addr(i);
  diffattn_problem p = prob(1, 2, 64, 64, DIFFATTN_BF16);
  EXPECT(fwd(nullptr, x, nullptr, addr(40), 1 << 20), DIFFATTN_E_ARG);
  { diffattn_problem q = p; q.batch = -1; EXPECT(fwd(&q, x, nullptr, addr(40), 1 << 20), DIFFATTN_E_ARG); }
  { diffattn_problem q = p; q.head_dim = 0; EXPECT(fwd(&q, x, nullptr, addr(40), 1 << 20), DIFFATTN_E_ARG); }
  { diffattn_problem q = p; q.head_dim = 128; EXPECT(fwd(&q, x, nullptr, addr(40), 1 << 20), DIFFATTN_E_UNSUPPORTED); }
  { diffattn_problem q = p; q.causal = 0; EXPECT(fwd(&q, x, nullptr, addr(40), 1 << 20), DIFFATTN_E_UNSUPPORTED); }
  { diffattn_problem q = p; q.rms_eps = std::nanf(""); EXPECT(fwd(&q, x, nullptr, addr(40), 1 << 20), DIFFATTN_E_ARG); }
  { diffattn_problem q = p; q.rms_eps = INFINITY; EXPECT(fwd(&q, x, nullptr, addr(40), 1 << 20), DIFFATTN_E_ARG); }
  { diffattn_problem q = p; q.dtype = 7; EXPECT(fwd(&q, x, nullptr, addr(40), 1 << 20), DIFFATTN_E_ARG); }
  { diffattn_problem q = p; q.out_layout = 5; EXPECT(fwd(&q, x, nullptr, addr(40), 1 << 20), DIFFATTN_E_ARG); }
  { diffattn_problem q = p; q.kv_heads = 3; EXPECT(fwd(&q, x, nullptr, addr(40), 1 << 20), DIFFATTN_E_ARG); }
  // sizes whose products overflow int64 (must be rejected without overflowing)
  { diffattn_problem q = prob(int64_t(1) << 40, int64_t(1) << 20, 64, 64, DIFFATTN_BF16);
    EXPECT(fwd(&q, x, nullptr, addr(40), 1 << 20), DIFFATTN_E_ARG);
    EXPECT(diffattn_workspace_bytes(DIFFATTN_OP_BWD, &q), 0);
    EXPECT(diffattn_workspace_bytes(DIFFATTN_OP_DECODE, &q), 0); }
  { diffattn_problem q = prob(std::numeric_limits<int64_t>::max(), 2, 2, 64, DIFFATTN_BF16);
    EXPECT(fwd(&q, x, nullptr, addr(40), 1 << 20), DIFFATTN_E_ARG); }
  { diffattn_problem q = prob(1, 1, (int64_t(1) << 22) + 1, 64, DIFFATTN_BF16);
    EXPECT(fwd(&q, x, nullptr, addr(40), 1 << 20), DIFFATTN_E_UNSUPPORTED); }
  // null, misaligned and overlapping pointers; workspace missing or too small
  { void* y[8]; std::memcpy(y, x, sizeof(y)); y[3] = nullptr; EXPECT(fwd(&p, y, nullptr, addr(40), 1 << 20), DIFFATTN_E_ARG); }
  { void* y[8]; std::memcpy(y, x, sizeof(y)); y[2] = at(A * 3 + 2); EXPECT(fwd(&p, y, nullptr, addr(40), 1 << 20), DIFFATTN_E_ARG); }
  { void* y[8]; std::memcpy(y, x, sizeof(y)); y[7] = at(A + 64); EXPECT(fwd(&p, y, nullptr, addr(40), 1 << 20), DIFFATTN_E_ARG); }
  const size_t need = diffattn_workspace_bytes(DIFFATTN_OP_FWD, &p);
  EXPECT(need, 64);
  EXPECT(fwd(&p, x, nullptr, nullptr, 0), DIFFATTN_E_WORKSPACE);
  EXPECT(fwd(&p, x, nullptr, addr(40), need - 1), DIFFATTN_E_WORKSPACE);
  EXPECT(fwd(&p, x, nullptr, addr(7), need), DIFFATTN_E_ARG);
  { diffattn_saved sv = {static_cast<float*>(addr(20)), static_cast<float*>(addr(21)),
                         static_cast<float*>(addr(22)), nullptr, static_cast<float*>(addr(24))};
    EXPECT(fwd(&p, x, &sv, addr(40), 1 << 20), DIFFATTN_E_ARG); }
  // empty problems: valid, no pointer needed
  { void* nul[8] = {}; diffattn_problem q = prob(0, 2, 16, 64, DIFFATTN_BF16);
    EXPECT(fwd(&q, nul, nullptr, nullptr, 0), DIFFATTN_OK);
    EXPECT(diffattn_decode(&q, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                           nullptr, nullptr, nullptr, 0, nullptr), DIFFATTN_OK);
    EXPECT(diffattn_decode_noalloc(&q, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                                   nullptr, nullptr, nullptr, nullptr), DIFFATTN_OK); }

  // lambda and lambda for many layers
  float* f[5];
  for (int i = 0; i < 5; ++i) f[i] = static_cast<float*>(addr(64 * i));
  auto* stp = reinterpret_cast<diffattn_lambda_state*>(f[4]);
  EXPECT(diffattn_lambda(0, 1, f[0], f[1], f[2], f[3], stp, nullptr), DIFFATTN_E_ARG);
  EXPECT(diffattn_lambda(2000, 1, f[0], f[1], f[2], f[3], stp, nullptr), DIFFATTN_E_ARG);
  EXPECT(diffattn_lambda(64, 0, f[0], f[1], f[2], f[3], stp, nullptr), DIFFATTN_E_ARG);
  EXPECT(diffattn_lambda(64, 1, nullptr, f[1], f[2], f[3], stp, nullptr), DIFFATTN_E_ARG);
  EXPECT(diffattn_lambda(64, 1, f[0], f[1], f[2], f[3],
                         reinterpret_cast<diffattn_lambda_state*>(at(A + 8)), nullptr),
         DIFFATTN_E_ARG);
  EXPECT(diffattn_lambda_layers(64, -1, 1, 0, 0.f, f[0], f[1], f[2], f[3], stp, nullptr), DIFFATTN_E_ARG);
  EXPECT(diffattn_lambda_layers(64, 4, 2147483646, 0, 0.f, f[0], f[1], f[2], f[3], stp, nullptr), DIFFATTN_E_ARG);
  EXPECT(diffattn_lambda_layers(64, 4, 1, 1, std::nanf(""), f[0], f[1], f[2], f[3], stp, nullptr), DIFFATTN_E_ARG);
  EXPECT(diffattn_lambda_layers(64, 0, 1, 0, 0.f, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr), DIFFATTN_OK);

  // decode and the allocation-free decode
  void* dq[9];
  for (int i = 0; i < 9; ++i) dq[i] = addr(64 * i);
  diffattn_problem pd = prob(64, 16, 8192, 64, DIFFATTN_BF16);
  const size_t dneed = diffattn_workspace_bytes(DIFFATTN_OP_DECODE, &pd);
  auto dec = [&](const diffattn_problem* q, void** y, void* ws, size_t n) {
    return diffattn_decode(q, y[0], y[1], y[2], y[3], y[4], static_cast<const int32_t*>(y[5]),
                           static_cast<const diffattn_lambda_state*>(y[6]),
                           static_cast<const float*>(y[7]), y[8], ws, n, nullptr);
  };
  auto dna = [&](const diffattn_problem* q, void** y) {
    return diffattn_decode_noalloc(q, y[0], y[1], y[2], y[3], y[4],
                                   static_cast<const int32_t*>(y[5]),
                                   static_cast<const diffattn_lambda_state*>(y[6]),
                                   static_cast<const float*>(y[7]), y[8], nullptr);
  };
  EXPECT(dec(&pd, dq, nullptr, dneed), DIFFATTN_E_WORKSPACE);
  EXPECT(dec(&pd, dq, addr(64 * 40), dneed - 4), DIFFATTN_E_WORKSPACE);
  { void* y[9]; std::memcpy(y, dq, sizeof(y)); y[8] = dq[2]; EXPECT(dec(&pd, y, addr(64 * 40), dneed), DIFFATTN_E_ARG); }
  { diffattn_problem big = prob(64, 16, int64_t(1) << 20, 64, DIFFATTN_BF16);
    EXPECT(dna(&big, dq), DIFFATTN_E_SCRATCH); }
  { void* y[9]; std::memcpy(y, dq, sizeof(y)); y[0] = nullptr; EXPECT(dna(&pd, y), DIFFATTN_E_ARG); }

  // cache append
  diffattn_problem pa = prob(4, 2, 128, 64, DIFFATTN_BF16);
  EXPECT(diffattn_cache_append(&pa, addr(0), addr(64), addr(128), addr(192), addr(256), addr(320),
                               nullptr, nullptr), DIFFATTN_E_ARG);
  EXPECT(diffattn_cache_append(&pa, addr(0), addr(64), addr(320), addr(192), addr(256), addr(320),
                               static_cast<int32_t*>(addr(384)), nullptr), DIFFATTN_E_ARG);

  // backward
  {
    diffattn_problem pb = prob(2, 2, 128, 64, DIFFATTN_BF16);
    const size_t bneed = diffattn_workspace_bytes(DIFFATTN_OP_BWD, &pb);
    void* b[27];
    for (int i = 0; i < 27; ++i) b[i] = addr(64 * i);
    diffattn_saved sv = {static_cast<float*>(addr(64 * 40)), static_cast<float*>(addr(64 * 41)),
                         static_cast<float*>(addr(64 * 42)), static_cast<float*>(addr(64 * 43)),
                         static_cast<float*>(addr(64 * 44))};
    auto bwd = [&](const diffattn_problem* q, void** y, const diffattn_saved* s, void* ws, size_t n) {
      return diffattn_bwd(q, y[0], y[1], y[2], y[3], y[4], static_cast<const float*>(y[5]),
                          static_cast<const float*>(y[6]), static_cast<const float*>(y[7]),
                          static_cast<const float*>(y[8]),
                          static_cast<const diffattn_lambda_state*>(y[9]),
                          static_cast<const float*>(y[10]), s, y[11], y[12], y[13], y[14], y[15],
                          y[16], static_cast<float*>(y[17]), static_cast<float*>(y[18]),
                          static_cast<float*>(y[19]), static_cast<float*>(y[20]),
                          static_cast<float*>(y[21]), static_cast<float*>(y[22]), ws, n, nullptr);
    };
    EXPECT(bwd(&pb, b, &sv, nullptr, bneed), DIFFATTN_E_WORKSPACE);
    EXPECT(bwd(&pb, b, nullptr, addr(64 * 60), bneed), DIFFATTN_E_ARG);
    { void* y[27]; std::memcpy(y, b, sizeof(y)); y[12] = b[0]; EXPECT(bwd(&pb, y, &sv, addr(64 * 60), bneed), DIFFATTN_E_ARG); }
    { diffattn_problem q = pb; q.head_dim = 16; EXPECT(bwd(&q, b, &sv, addr(64 * 60), bneed), DIFFATTN_E_UNSUPPORTED); }
  }

  // projections
  {
    diffattn_problem pp = prob(1, 16, 1024, 64, DIFFATTN_BF16);
    EXPECT(diffattn_qkv_proj(&pp, 100, addr(0), addr(64), addr(128), addr(192), addr(256),
                             addr(320), addr(384), nullptr), DIFFATTN_E_UNSUPPORTED);
    EXPECT(diffattn_qkv_proj(&pp, int64_t(1) << 17, addr(0), addr(64), addr(128), addr(192),
                             addr(256), addr(320), addr(384), nullptr), DIFFATTN_E_ARG);
    EXPECT(diffattn_out_proj(&pp, 2048, addr(0), addr(64), addr(0), nullptr), DIFFATTN_E_ARG);
  }

  if (g_fail) {
    std::fprintf(stderr, "%d check(s) failed\n", g_fail);
    return 1;
  }
  std::printf("abi checks passed\n");
  return 0;
}
