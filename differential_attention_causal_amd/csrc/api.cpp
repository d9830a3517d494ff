// libdiffattn C-ABI: argument validation, workspace sizing and kernel launches.
//
// Every entry point validates its arguments on the host before any HIP call, so the
// checks also run on a machine without a GPU. Launch failures are reported as
// DIFFATTN_E_HIP with the hipError_t kept per thread.
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <cmath>

#include <hip/hip_runtime.h>
#include <rocprofiler-sdk-roctx/roctx.h>

#include "diffattn.h"
#include "launch.h"

namespace {

thread_local int g_last_hip = 0;

bool env_log() {
  // Read once; the initialisation of a local static is thread-safe.
  static const bool on = [] {
    const char* e = getenv("DIFFATTN_LOG");
    return e != nullptr && e[0] == '1';
  }();
  return on;
}

// One marker range per entry-point call, named after the entry point (shown by
// rocprofv3 --marker-trace; a no-op when no tool is attached). With DIFFATTN_LOG=1 the
// call and its problem shape are also written to stderr.
struct CallRange {
  CallRange(const char* name, const diffattn_problem* p) {
    roctxRangePushA(name);
    if (!env_log()) return;
    if (p) {
      fprintf(stderr, "[diffattn] %s B=%lld H=%lld N=%lld d=%d kv_heads=%lld dtype=%d\n", name,
              static_cast<long long>(p->batch), static_cast<long long>(p->heads),
              static_cast<long long>(p->seqlen), p->head_dim,
              static_cast<long long>(p->kv_heads), static_cast<int>(p->dtype));
    } else {
      fprintf(stderr, "[diffattn] %s\n", name);
    }
  }
  ~CallRange() { roctxRangePop(); }
  CallRange(const CallRange&) = delete;
  CallRange& operator=(const CallRange&) = delete;
};

diffattn_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return DIFFATTN_OK;
  g_last_hip = static_cast<int>(e);
  if (env_log()) fprintf(stderr, "[diffattn] %s: hip error %d\n", what, static_cast<int>(e));
  return DIFFATTN_E_HIP;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

struct Span {
  const void* p;
  size_t n;
};

bool overlap(Span a, Span b) {
  if (!a.p || !b.p || a.n == 0 || b.n == 0) return false;
  const uintptr_t x = reinterpret_cast<uintptr_t>(a.p), y = reinterpret_cast<uintptr_t>(b.p);
  return x < y + b.n && y < x + a.n;
}

// Any output span overlapping any input span, or two outputs overlapping each other.
bool any_overlap(const Span* outs, int no, const Span* ins, int ni) {
  for (int i = 0; i < no; ++i) {
    for (int j = 0; j < ni; ++j)
      if (overlap(outs[i], ins[j])) return true;
    for (int j = i + 1; j < no; ++j)
      if (overlap(outs[i], outs[j])) return true;
  }
  return false;
}

// Longest bf16 sequence (forward, backward) or cache (decode): the kernels address one
// head's K and V rows through 32-bit buffer offsets (N * 256 bytes for V).
constexpr int64_t kMaxSeqBf16 = int64_t(1) << 22;

size_t elem_bytes(int32_t t) { return t == DIFFATTN_FP32 ? 4 : 2; }

// Validates the problem descriptor. Sets *empty when there is nothing to compute.
diffattn_status check_problem(const diffattn_problem* p, bool* empty) {
  if (!p) return DIFFATTN_E_ARG;
  if (p->batch < 0 || p->heads < 0 || p->seqlen < 0) return DIFFATTN_E_ARG;
  if (p->head_dim <= 0) return DIFFATTN_E_ARG;
  if (p->dtype != DIFFATTN_FP32 && p->dtype != DIFFATTN_BF16) return DIFFATTN_E_ARG;
  if (!(p->rms_eps >= 0.0f) || !isfinite(p->rms_eps)) return DIFFATTN_E_ARG;
  if (p->out_layout != DIFFATTN_LAYOUT_BHN && p->out_layout != DIFFATTN_LAYOUT_BNH)
    return DIFFATTN_E_ARG;
  if (p->kv_heads < 0 || p->kv_heads > p->heads) return DIFFATTN_E_ARG;
  if (p->kv_heads > 0 && p->heads % p->kv_heads != 0) return DIFFATTN_E_ARG;
  if (p->causal != 1) return DIFFATTN_E_UNSUPPORTED;
  // Largest tensor: [B, H, N, 2d] float32 must stay far from int64 overflow.
  int64_t t = 0;
  if (__builtin_mul_overflow(p->batch, p->heads, &t) ||
      __builtin_mul_overflow(t, p->seqlen, &t) ||
      __builtin_mul_overflow(t, static_cast<int64_t>(2 * p->head_dim) * 4, &t) ||
      t > (static_cast<int64_t>(1) << 46))
    return DIFFATTN_E_ARG;
  *empty = p->batch == 0 || p->heads == 0 || p->seqlen == 0;
  return DIFFATTN_OK;
}

// Heads of K1, K2 and V: p->kv_heads, or heads when it is 0.
int64_t kv_heads_of(const diffattn_problem* p) { return p->kv_heads > 0 ? p->kv_heads : p->heads; }

size_t decode_ws_bytes(const diffattn_problem* p) {
  int gq = 0, ns = 0, sl = 0;
  diffattn::decode_geometry(p->batch, p->heads, p->heads / kv_heads_of(p), p->seqlen, &gq, &ns,
                            &sl);
  // per (b, h, split): two maps x (m, l, 2d accumulators)
  return static_cast<size_t>(p->batch) * p->heads * ns * 2 * (2 + 2 * p->head_dim) *
         sizeof(float);
}

}  // namespace

extern "C" {

const char* diffattn_status_string(diffattn_status s) {
  switch (s) {
    case DIFFATTN_OK: return "DIFFATTN_OK";
    case DIFFATTN_E_ARG: return "DIFFATTN_E_ARG: invalid argument";
    case DIFFATTN_E_UNSUPPORTED: return "DIFFATTN_E_UNSUPPORTED: unsupported configuration";
    case DIFFATTN_E_WORKSPACE: return "DIFFATTN_E_WORKSPACE: workspace missing or too small";
    case DIFFATTN_E_HIP: return "DIFFATTN_E_HIP: HIP runtime error";
    case DIFFATTN_E_SCRATCH:
      return "DIFFATTN_E_SCRATCH: problem needs more than the static decode scratch";
  }
  return "DIFFATTN_E_?: unknown status";
}

int diffattn_last_hip_error(void) { return g_last_hip; }

size_t diffattn_workspace_bytes(diffattn_op op, const diffattn_problem* p) {
  bool empty = false;
  if (check_problem(p, &empty) != DIFFATTN_OK || empty) return 0;
  switch (op) {
    case DIFFATTN_OP_FWD:
      return p->dtype == DIFFATTN_BF16
                 ? diffattn::fwd_bf16_workspace_bytes(p->batch, p->heads, p->seqlen)
                 : 0;
    case DIFFATTN_OP_DECODE: return decode_ws_bytes(p);
    case DIFFATTN_OP_BWD:
      return diffattn::bwd_workspace_floats(p->batch, p->heads, p->seqlen, p->head_dim) *
             sizeof(float);
  }
  return 0;
}

diffattn_status diffattn_lambda(int32_t dim, int32_t layer_idx, const float* lq1,
                                const float* lk1, const float* lq2, const float* lk2,
                                diffattn_lambda_state* state_out, void* stream) {
  const CallRange range("diffattn_lambda", nullptr);
  if (dim < 1 || dim > 1024 || layer_idx < 1) return DIFFATTN_E_ARG;
  if (!lq1 || !lk1 || !lq2 || !lk2 || !state_out) return DIFFATTN_E_ARG;
  if (!aligned(lq1, 4) || !aligned(lk1, 4) || !aligned(lq2, 4) || !aligned(lk2, 4) ||
      !aligned(state_out, 8))
    return DIFFATTN_E_ARG;
  const size_t vb = static_cast<size_t>(dim) * sizeof(float);
  const Span out[1] = {{state_out, sizeof(diffattn_lambda_state)}};
  const Span in[4] = {{lq1, vb}, {lk1, vb}, {lq2, vb}, {lk2, vb}};
  if (any_overlap(out, 1, in, 4)) return DIFFATTN_E_ARG;
  return hip_status(diffattn::launch_lambda(dim, layer_idx, lq1, lk1, lq2, lk2, state_out,
                                            static_cast<hipStream_t>(stream)),
                    "lambda");
}

diffattn_status diffattn_lambda_layers(int32_t dim, int32_t n_layers, int32_t first_layer,
                                       int32_t fixed_init, float lambda_init,
                                       const float* lq1, const float* lk1, const float* lq2,
                                       const float* lk2, diffattn_lambda_state* states_out,
                                       void* stream) {
  const CallRange range("diffattn_lambda_layers", nullptr);
  if (dim < 1 || dim > 1024 || n_layers < 0 || n_layers > 65535 || first_layer < 1)
    return DIFFATTN_E_ARG;
  if (first_layer > INT32_MAX - n_layers) return DIFFATTN_E_ARG;
  if (fixed_init != 0 && fixed_init != 1) return DIFFATTN_E_ARG;
  if (fixed_init && !std::isfinite(lambda_init)) return DIFFATTN_E_ARG;
  if (n_layers == 0) return DIFFATTN_OK;
  if (!lq1 || !lk1 || !lq2 || !lk2 || !states_out) return DIFFATTN_E_ARG;
  if (!aligned(lq1, 4) || !aligned(lk1, 4) || !aligned(lq2, 4) || !aligned(lk2, 4) ||
      !aligned(states_out, 8))
    return DIFFATTN_E_ARG;
  const size_t vb = static_cast<size_t>(dim) * n_layers * sizeof(float);
  const Span out[1] = {{states_out, sizeof(diffattn_lambda_state) * n_layers}};
  const Span in[4] = {{lq1, vb}, {lk1, vb}, {lq2, vb}, {lk2, vb}};
  if (any_overlap(out, 1, in, 4)) return DIFFATTN_E_ARG;
  const double init = fixed_init ? static_cast<double>(lambda_init) : 0.0;
  return hip_status(diffattn::launch_lambda_layers(dim, n_layers, first_layer, fixed_init != 0,
                                                   init, lq1, lk1, lq2, lk2, states_out,
                                                   static_cast<hipStream_t>(stream)),
                    "lambda_layers");
}

diffattn_status diffattn_fwd(const diffattn_problem* p, const void* q1, const void* q2,
                             const void* k1, const void* k2, const void* v,
                             const diffattn_lambda_state* lam, const float* rms_weight,
                             void* out, const diffattn_saved* saved, void* workspace,
                             size_t workspace_bytes, void* stream) {
  const CallRange range("diffattn_fwd", p);
  bool empty = false;
  diffattn_status st = check_problem(p, &empty);
  if (st != DIFFATTN_OK) return st;
  const int d = p->head_dim;
  if (p->dtype == DIFFATTN_FP32) {
    if (d != 16 && d != 32 && d != 64) return DIFFATTN_E_UNSUPPORTED;
    if (saved) return DIFFATTN_E_UNSUPPORTED;
    if (p->batch * p->heads > 65535) return DIFFATTN_E_UNSUPPORTED;
  } else {
    if (d != 64) return DIFFATTN_E_UNSUPPORTED;
    if (p->seqlen > kMaxSeqBf16) return DIFFATTN_E_UNSUPPORTED;
  }
  if (empty) return DIFFATTN_OK;
  if (!q1 || !q2 || !k1 || !k2 || !v || !lam || !out) return DIFFATTN_E_ARG;
  const size_t need = diffattn_workspace_bytes(DIFFATTN_OP_FWD, p);
  if (need > 0 && (!workspace || workspace_bytes < need)) return DIFFATTN_E_WORKSPACE;
  if (need > 0 && !aligned(workspace, 16)) return DIFFATTN_E_ARG;
  const void* ptrs[6] = {q1, q2, k1, k2, v, out};
  for (const void* x : ptrs)
    if (!aligned(x, 16)) return DIFFATTN_E_ARG;
  if (!aligned(lam, 8) || (rms_weight && !aligned(rms_weight, 16))) return DIFFATTN_E_ARG;
  const size_t rows = static_cast<size_t>(p->batch) * p->heads * p->seqlen;
  const size_t eb = elem_bytes(p->dtype);
  const size_t qk = rows * d * eb, vb = rows * 2 * d * eb;
  const size_t kv_rows = static_cast<size_t>(p->batch) * kv_heads_of(p) * p->seqlen;
  const size_t kk = kv_rows * d * eb, kvb = kv_rows * 2 * d * eb;
  const Span in[7] = {{q1, qk}, {q2, qk}, {k1, kk}, {k2, kk}, {v, kvb},
                      {lam, sizeof(diffattn_lambda_state)},
                      {rms_weight, static_cast<size_t>(p->heads) * 2 * d * sizeof(float)}};
  diffattn::FwdArgs a;
  memset(&a, 0, sizeof(a));
  if (saved) {
    const diffattn_saved& s = *saved;
    if (!s.lse1 || !s.lse2 || !s.o1 || !s.o2 || !s.rstd) return DIFFATTN_E_ARG;
    if (!aligned(s.lse1, 4) || !aligned(s.lse2, 4) || !aligned(s.rstd, 4) ||
        !aligned(s.o1, 16) || !aligned(s.o2, 16))
      return DIFFATTN_E_ARG;
    const size_t rb = rows * sizeof(float), ob = rows * 2 * d * sizeof(float);
    const Span outs[7] = {{out, vb}, {s.lse1, rb}, {s.lse2, rb}, {s.o1, ob}, {s.o2, ob},
                          {s.rstd, rb}, {workspace, need}};
    if (any_overlap(outs, 7, in, 7)) return DIFFATTN_E_ARG;
    a.saved = s;
    a.training = true;
  } else {
    const Span outs[2] = {{out, vb}, {workspace, need}};
    if (any_overlap(outs, 2, in, 7)) return DIFFATTN_E_ARG;
  }
  a.workspace = need > 0 ? workspace : nullptr;
  a.q1 = q1; a.q2 = q2; a.k1 = k1; a.k2 = k2; a.v = v;
  a.lam = lam;
  a.rms_weight = rms_weight;
  a.out = out;
  a.B = p->batch; a.H = p->heads; a.N = p->seqlen;
  a.G = static_cast<int>(p->heads / kv_heads_of(p));
  a.d = d;
  a.eps = p->rms_eps;
  a.out_bnh = p->out_layout == DIFFATTN_LAYOUT_BNH;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (p->dtype == DIFFATTN_FP32) return hip_status(diffattn::launch_fwd_fp32(a, s), "fwd_fp32");
  return hip_status(diffattn::launch_fwd_bf16(a, s), "fwd_bf16");
}

}  // extern "C"

namespace {

// The decode inputs' byte spans (for the overlap checks); returns the output's bytes.
size_t decode_spans(const diffattn_problem* p, const void* q1, const void* q2, const void* k1c,
                    const void* k2c, const void* vc, const int32_t* cache_len,
                    const diffattn_lambda_state* lam, const float* rms_weight, Span* in) {
  const int d = p->head_dim;
  const size_t bh = static_cast<size_t>(p->batch) * p->heads;
  const size_t bhk = static_cast<size_t>(p->batch) * kv_heads_of(p);
  const size_t qb = bh * d * 2, kb = bhk * p->seqlen * d * 2, vb = bhk * p->seqlen * 2 * d * 2;
  in[0] = {q1, qb}; in[1] = {q2, qb}; in[2] = {k1c, kb}; in[3] = {k2c, kb}; in[4] = {vc, vb};
  in[5] = {cache_len, static_cast<size_t>(p->batch) * 4};
  in[6] = {lam, sizeof(diffattn_lambda_state)};
  in[7] = {rms_weight, static_cast<size_t>(p->heads) * 2 * d * sizeof(float)};
  return bh * 2 * d * 2;
}

// Validation shared by the two decode entry points (all but the overlap checks, which
// follow each one's scratch check); fills *a (except a->partial) and *need (the
// partials' bytes). *empty: nothing to compute.
diffattn_status decode_prepare(const diffattn_problem* p, const void* q1, const void* q2,
                               const void* k1c, const void* k2c, const void* vc,
                               const int32_t* cache_len, const diffattn_lambda_state* lam,
                               const float* rms_weight, void* out, diffattn::DecodeArgs* a,
                               size_t* need, bool* empty) {
  diffattn_status st = check_problem(p, empty);
  if (st != DIFFATTN_OK) return st;
  if (p->dtype != DIFFATTN_BF16 || p->head_dim != 64) return DIFFATTN_E_UNSUPPORTED;
  if (p->batch * p->heads > 65535 || p->seqlen > kMaxSeqBf16) return DIFFATTN_E_UNSUPPORTED;
  if (*empty) return DIFFATTN_OK;
  if (!q1 || !q2 || !k1c || !k2c || !vc || !lam || !out) return DIFFATTN_E_ARG;
  const void* ptrs[6] = {q1, q2, k1c, k2c, vc, out};
  for (const void* x : ptrs)
    if (!aligned(x, 16)) return DIFFATTN_E_ARG;
  if (!aligned(lam, 8) || (rms_weight && !aligned(rms_weight, 16)) ||
      (cache_len && !aligned(cache_len, 4)))
    return DIFFATTN_E_ARG;
  *need = decode_ws_bytes(p);
  memset(a, 0, sizeof(*a));
  a->q1 = q1; a->q2 = q2; a->k1 = k1c; a->k2 = k2c; a->v = vc;
  a->cache_len = cache_len;
  a->lam = lam;
  a->rms_weight = rms_weight;
  a->out = out;
  a->B = p->batch; a->H = p->heads; a->L = p->seqlen;
  a->G = static_cast<int>(p->heads / kv_heads_of(p));
  diffattn::decode_geometry(a->B, a->H, a->G, a->L, &a->gq, &a->n_split, &a->split_len);
  a->d = p->head_dim;
  a->eps = p->rms_eps;
  return DIFFATTN_OK;
}

}  // namespace

extern "C" {

diffattn_status diffattn_decode(const diffattn_problem* p, const void* q1, const void* q2,
                                const void* k1c, const void* k2c, const void* vc,
                                const int32_t* cache_len, const diffattn_lambda_state* lam,
                                const float* rms_weight, void* out, void* workspace,
                                size_t workspace_bytes, void* stream) {
  const CallRange range("diffattn_decode", p);
  diffattn::DecodeArgs a;
  size_t need = 0;
  bool empty = false;
  diffattn_status st = decode_prepare(p, q1, q2, k1c, k2c, vc, cache_len, lam, rms_weight, out,
                                      &a, &need, &empty);
  if (st != DIFFATTN_OK || empty) return st;
  if (!workspace || workspace_bytes < need) return DIFFATTN_E_WORKSPACE;
  if (!aligned(workspace, 16)) return DIFFATTN_E_ARG;
  Span in[8];
  const size_t out_bytes = decode_spans(p, q1, q2, k1c, k2c, vc, cache_len, lam, rms_weight, in);
  const Span outs[2] = {{out, out_bytes}, {workspace, need}};
  if (any_overlap(outs, 2, in, 8)) return DIFFATTN_E_ARG;
  a.partial = static_cast<float*>(workspace);
  return hip_status(diffattn::launch_decode_bf16(a, static_cast<hipStream_t>(stream)), "decode");
}

diffattn_status diffattn_decode_noalloc(const diffattn_problem* p, const void* q1,
                                        const void* q2, const void* k1c, const void* k2c,
                                        const void* vc, const int32_t* cache_len,
                                        const diffattn_lambda_state* lam,
                                        const float* rms_weight, void* out, void* stream) {
  const CallRange range("diffattn_decode_noalloc", p);
  diffattn::DecodeArgs a;
  size_t need = 0;
  bool empty = false;
  diffattn_status st = decode_prepare(p, q1, q2, k1c, k2c, vc, cache_len, lam, rms_weight, out,
                                      &a, &need, &empty);
  if (st != DIFFATTN_OK || empty) return st;
  if (need > DIFFATTN_DECODE_SCRATCH_BYTES) return DIFFATTN_E_SCRATCH;
  Span in[8];
  const size_t out_bytes = decode_spans(p, q1, q2, k1c, k2c, vc, cache_len, lam, rms_weight, in);
  const Span outs[1] = {{out, out_bytes}};
  if (any_overlap(outs, 1, in, 8)) return DIFFATTN_E_ARG;
  float* ptr = nullptr;   // device address of the static scratch on the current device
  st = hip_status(diffattn::decode_scratch(&ptr), "decode scratch lookup");
  if (st != DIFFATTN_OK) return st;
  a.partial = ptr;
  return hip_status(diffattn::launch_decode_bf16(a, static_cast<hipStream_t>(stream)),
                    "decode_noalloc");
}

diffattn_status diffattn_cache_append(const diffattn_problem* p, const void* k1_new,
                                      const void* k2_new, const void* v_new, void* k1c,
                                      void* k2c, void* vc, int32_t* cache_len, void* stream) {
  const CallRange range("diffattn_cache_append", p);
  bool empty = false;
  diffattn_status st = check_problem(p, &empty);
  if (st != DIFFATTN_OK) return st;
  if (p->dtype != DIFFATTN_BF16 || p->head_dim != 64) return DIFFATTN_E_UNSUPPORTED;
  if (p->seqlen > kMaxSeqBf16) return DIFFATTN_E_UNSUPPORTED;
  if (empty) return DIFFATTN_OK;
  if (!k1_new || !k2_new || !v_new || !k1c || !k2c || !vc || !cache_len) return DIFFATTN_E_ARG;
  const void* ptrs[6] = {k1_new, k2_new, v_new, k1c, k2c, vc};
  for (const void* x : ptrs)
    if (!aligned(x, 16)) return DIFFATTN_E_ARG;
  if (!aligned(cache_len, 4)) return DIFFATTN_E_ARG;
  const int d = p->head_dim;
  const size_t bh = static_cast<size_t>(p->batch) * kv_heads_of(p);   // cache heads
  const size_t kr = bh * d * 2, vr = bh * 2 * d * 2;
  const size_t kc = kr * p->seqlen, vcb = vr * p->seqlen;
  const Span in[3] = {{k1_new, kr}, {k2_new, kr}, {v_new, vr}};
  const Span outs[4] = {{k1c, kc}, {k2c, kc}, {vc, vcb},
                        {cache_len, static_cast<size_t>(p->batch) * 4}};
  if (any_overlap(outs, 4, in, 3)) return DIFFATTN_E_ARG;
  diffattn::AppendArgs a;
  a.k1n = k1_new; a.k2n = k2_new; a.vn = v_new;
  a.k1c = k1c; a.k2c = k2c; a.vc = vc;
  a.cache_len = cache_len;
  a.B = p->batch; a.H = kv_heads_of(p); a.L = p->seqlen;
  return hip_status(diffattn::launch_cache_append_bf16(a, static_cast<hipStream_t>(stream)),
                    "cache_append");
}

// Shapes the projection GEMMs take: K (d_model, or H 2d for W_O) a multiple of 64 up to
// 65536, M = B N rows below 2^31, d a multiple of 32 (so no 32-column block of the fused
// QKV output straddles two tensors).
diffattn_status check_proj(const diffattn_problem* p, int64_t d_model, bool* empty) {
  diffattn_status st = check_problem(p, empty);
  if (st != DIFFATTN_OK) return st;
  if (d_model < 64 || d_model > 65536) return DIFFATTN_E_ARG;
  if (p->dtype != DIFFATTN_BF16) return DIFFATTN_E_UNSUPPORTED;
  const int d = p->head_dim;
  if (d % 32 != 0 || d > 256 || d_model % 64 != 0) return DIFFATTN_E_UNSUPPORTED;
  if (p->heads * 2 * d > 65536) return DIFFATTN_E_UNSUPPORTED;
  if (p->batch * p->seqlen >= (int64_t(1) << 31)) return DIFFATTN_E_UNSUPPORTED;
  // The GEMM numbers its 256 x 256 output tiles with 32-bit integers.
  const int64_t m_tiles = (p->batch * p->seqlen + 255) / 256;
  const int64_t n_widest = std::max<int64_t>(d_model, 6 * p->heads * d);
  if (m_tiles * ((n_widest + 255) / 256) >= (int64_t(1) << 31)) return DIFFATTN_E_UNSUPPORTED;
  return DIFFATTN_OK;
}

diffattn_status diffattn_qkv_proj(const diffattn_problem* p, int64_t d_model, const void* x,
                                  const void* w_qkv, void* q1, void* q2, void* k1, void* k2,
                                  void* v, void* stream) {
  const CallRange range("diffattn_qkv_proj", p);
  bool empty = false;
  diffattn_status st = check_proj(p, d_model, &empty);
  if (st != DIFFATTN_OK) return st;
  if (empty) return DIFFATTN_OK;
  const void* ptrs[7] = {x, w_qkv, q1, q2, k1, k2, v};
  for (const void* ptr : ptrs)
    if (!ptr || !aligned(ptr, 16)) return DIFFATTN_E_ARG;
  const size_t m = static_cast<size_t>(p->batch) * p->seqlen;
  const size_t hd = static_cast<size_t>(p->heads) * p->head_dim;
  const size_t hkd = static_cast<size_t>(kv_heads_of(p)) * p->head_dim;
  const Span in[2] = {{x, m * d_model * 2}, {w_qkv, 2 * (hd + 2 * hkd) * d_model * 2}};
  const Span outs[5] = {{q1, m * hd * 2}, {q2, m * hd * 2}, {k1, m * hkd * 2},
                        {k2, m * hkd * 2}, {v, m * hkd * 4}};
  if (any_overlap(outs, 5, in, 2)) return DIFFATTN_E_ARG;
  diffattn::QkvProjArgs a;
  a.x = x; a.w = w_qkv;
  a.q1 = q1; a.q2 = q2; a.k1 = k1; a.k2 = k2; a.v = v;
  a.B = p->batch; a.H = p->heads; a.N = p->seqlen; a.d_model = d_model;
  a.Hkv = kv_heads_of(p);
  a.d = p->head_dim;
  return hip_status(diffattn::launch_qkv_proj_bf16(a, static_cast<hipStream_t>(stream)),
                    "qkv_proj");
}

diffattn_status diffattn_out_proj(const diffattn_problem* p, int64_t d_model, const void* attn,
                                  const void* w_o, void* y, void* stream) {
  const CallRange range("diffattn_out_proj", p);
  bool empty = false;
  diffattn_status st = check_proj(p, d_model, &empty);
  if (st != DIFFATTN_OK) return st;
  if (empty) return DIFFATTN_OK;
  const void* ptrs[3] = {attn, w_o, y};
  for (const void* ptr : ptrs)
    if (!ptr || !aligned(ptr, 16)) return DIFFATTN_E_ARG;
  const size_t m = static_cast<size_t>(p->batch) * p->seqlen;
  const size_t k = static_cast<size_t>(p->heads) * 2 * p->head_dim;
  const Span in[2] = {{attn, m * k * 2}, {w_o, static_cast<size_t>(d_model) * k * 2}};
  const Span outs[1] = {{y, m * d_model * 2}};
  if (any_overlap(outs, 1, in, 2)) return DIFFATTN_E_ARG;
  diffattn::OutProjArgs a;
  a.attn = attn; a.w = w_o; a.y = y;
  a.M = static_cast<int64_t>(m); a.d_model = d_model; a.k = static_cast<int64_t>(k);
  return hip_status(diffattn::launch_out_proj_bf16(a, static_cast<hipStream_t>(stream)),
                    "out_proj");
}

diffattn_status diffattn_bwd(const diffattn_problem* p, const void* q1, const void* q2,
                             const void* k1, const void* k2, const void* v, const float* lq1,
                             const float* lk1, const float* lq2, const float* lk2,
                             const diffattn_lambda_state* lam, const float* rms_weight,
                             const diffattn_saved* saved, const void* dout, void* dq1,
                             void* dq2, void* dk1, void* dk2, void* dv, float* d_attn,
                             float* dlq1, float* dlk1, float* dlq2, float* dlk2,
                             float* d_rms_weight, void* workspace, size_t workspace_bytes,
                             void* stream) {
  const CallRange range("diffattn_bwd", p);
  bool empty = false;
  diffattn_status st = check_problem(p, &empty);
  if (st != DIFFATTN_OK) return st;
  if (p->dtype != DIFFATTN_BF16 || p->head_dim != 64) return DIFFATTN_E_UNSUPPORTED;
  if (p->seqlen > kMaxSeqBf16) return DIFFATTN_E_UNSUPPORTED;
  const int d = p->head_dim;
  // The lambda-vector gradients exist even for an empty problem (they are then zero).
  if (!lq1 || !lk1 || !lq2 || !lk2 || !lam || !dlq1 || !dlk1 || !dlq2 || !dlk2)
    return DIFFATTN_E_ARG;
  if (!empty) {
    if (!q1 || !q2 || !k1 || !k2 || !v || !saved || !dout || !dq1 || !dq2 || !dk1 || !dk2 ||
        !dv || !d_attn)
      return DIFFATTN_E_ARG;
    const diffattn_saved& s = *saved;
    if (!s.lse1 || !s.lse2 || !s.o1 || !s.o2 || !s.rstd) return DIFFATTN_E_ARG;
    const void* p16[14] = {q1, q2, k1, k2, v, dout, dq1, dq2, dk1, dk2, dv, d_attn, s.o1, s.o2};
    for (const void* x : p16)
      if (!aligned(x, 16)) return DIFFATTN_E_ARG;
    if (!aligned(s.lse1, 4) || !aligned(s.lse2, 4) || !aligned(s.rstd, 4))
      return DIFFATTN_E_ARG;
  }
  const void* p4[4] = {lq1, lk1, lq2, lk2};
  for (const void* x : p4)
    if (!aligned(x, 4)) return DIFFATTN_E_ARG;
  if (!aligned(dlq1, 4) || !aligned(dlk1, 4) || !aligned(dlq2, 4) || !aligned(dlk2, 4) ||
      !aligned(lam, 8) || (rms_weight && !aligned(rms_weight, 16)) ||
      (d_rms_weight && !aligned(d_rms_weight, 4)))
    return DIFFATTN_E_ARG;
  const size_t need = diffattn_workspace_bytes(DIFFATTN_OP_BWD, p);
  if (need > 0 && (!workspace || workspace_bytes < need)) return DIFFATTN_E_WORKSPACE;
  if (workspace && !aligned(workspace, 16)) return DIFFATTN_E_ARG;
  const size_t rows = static_cast<size_t>(p->batch) * p->heads * p->seqlen;
  const size_t kv_rows = static_cast<size_t>(p->batch) * kv_heads_of(p) * p->seqlen;
  const size_t qk = rows * d * 2, vb = rows * 2 * d * 2, rb = rows * 4, ob = rows * 2 * d * 4;
  const size_t kk = kv_rows * d * 2, kvb = kv_rows * 2 * d * 2;
  const size_t lb = static_cast<size_t>(d) * 4;
  const diffattn_saved s = saved ? *saved : diffattn_saved{nullptr, nullptr, nullptr, nullptr, nullptr};
  const Span in[16] = {{q1, qk}, {q2, qk}, {k1, kk}, {k2, kk}, {v, kvb}, {dout, vb},
                       {lq1, lb}, {lk1, lb}, {lq2, lb}, {lk2, lb},
                       {lam, sizeof(diffattn_lambda_state)},
                       {rms_weight, static_cast<size_t>(p->heads) * 2 * d * sizeof(float)},
                       {s.lse1, rb}, {s.lse2, rb}, {s.o1, ob}, {s.o2, ob}};
  const size_t wb = static_cast<size_t>(p->heads) * 2 * d * sizeof(float);
  const Span outs[12] = {{dq1, qk}, {dq2, qk}, {dk1, kk}, {dk2, kk}, {dv, kvb}, {d_attn, ob},
                         {dlq1, lb}, {dlk1, lb}, {dlq2, lb}, {dlk2, lb}, {workspace, need},
                         {d_rms_weight, wb}};
  if (any_overlap(outs, 12, in, 16)) return DIFFATTN_E_ARG;
  for (int i = 0; i < 12; ++i)
    if (overlap(outs[i], {s.rstd, rb})) return DIFFATTN_E_ARG;
  diffattn::BwdArgs a;
  memset(&a, 0, sizeof(a));
  a.q1 = q1; a.q2 = q2; a.k1 = k1; a.k2 = k2; a.v = v; a.dout = dout;
  a.lq1 = lq1; a.lk1 = lk1; a.lq2 = lq2; a.lk2 = lk2;
  a.lam = lam;
  a.rms_weight = rms_weight;
  a.saved = s;
  a.dq1 = dq1; a.dq2 = dq2; a.dk1 = dk1; a.dk2 = dk2; a.dv = dv;
  a.d_attn = d_attn;
  a.dlq1 = dlq1; a.dlk1 = dlk1; a.dlq2 = dlq2; a.dlk2 = dlk2;
  a.d_rms_weight = d_rms_weight;
  a.dout_bnh = p->out_layout == DIFFATTN_LAYOUT_BNH;
  a.ws = static_cast<float*>(workspace);
  a.B = empty ? 0 : p->batch; a.H = p->heads; a.N = p->seqlen;
  a.G = p->heads > 0 ? static_cast<int>(p->heads / kv_heads_of(p)) : 1;
  a.d = d;
  return hip_status(diffattn::launch_bwd_bf16(a, static_cast<hipStream_t>(stream)), "bwd");
}

}  // extern "C"
