// Host-side launchers implemented in the .hip files; called only by api.cpp after the
// arguments have been validated. Each returns hipSuccess or the launch error.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "diffattn.h"

namespace diffattn {

// Runs `set` (which sets kernel attributes, such as the dynamic LDS size) once for each
// device the calling thread has current: the attributes belong to a device. The flag word
// is atomic, so first calls from several threads at once are safe (each may set the same
// attribute). Devices beyond the 64th are set on every call.
template <typename F>
inline hipError_t once_per_device(std::atomic<uint64_t>& done, F&& set) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = (dev >= 0 && dev < 64) ? (uint64_t{1} << dev) : 0;
  if (bit != 0 && (done.load(std::memory_order_acquire) & bit) != 0) return hipSuccess;
  e = set();
  if (e == hipSuccess && bit != 0) done.fetch_or(bit, std::memory_order_acq_rel);
  return e;
}

// All tensors contiguous [B, H, N, feature]; shapes already validated.
struct FwdArgs {
  const void *q1, *q2, *k1, *k2, *v;
  const diffattn_lambda_state* lam;
  const float* rms_weight;   // [H, 2d] or nullptr
  void* out;
  diffattn_saved saved;      // all-null fields = inference
  bool training;
  void* workspace;           // bf16: per row block, 8 words of row flags
  int64_t B, H, N;
  int G;                     // query heads per K/V head (K1, K2, V have H / G heads)
  int d;
  float eps;
  bool out_bnh;              // out is [B, N, H, 2d] instead of [B, H, N, 2d]
};

struct DecodeArgs {
  const void *q1, *q2, *k1, *k2, *v;
  const int32_t* cache_len;
  const diffattn_lambda_state* lam;
  const float* rms_weight;
  void* out;
  float* partial;            // workspace
  int64_t B, H, L;
  int G;                     // query heads per cache head (caches have H / G heads)
  int gq;                    // query heads per workgroup (divides G)
  int n_split, split_len;
  int d;
  float eps;
};

struct BwdArgs {
  const void *q1, *q2, *k1, *k2, *v, *dout;
  const float *lq1, *lk1, *lq2, *lk2;
  const diffattn_lambda_state* lam;
  const float* rms_weight;
  diffattn_saved saved;
  void *dq1, *dq2, *dk1, *dk2, *dv;
  float* d_attn;
  float *dlq1, *dlk1, *dlq2, *dlk2;
  float* d_rms_weight;       // [H, 2d] or nullptr
  bool dout_bnh;             // dout is [B, N, H, 2d] instead of [B, H, N, 2d]
  float* ws;                 // workspace (float32)
  int64_t B, H, N;
  int G;                     // query heads per K/V head (k1, k2, v, dk1, dk2, dv: H / G heads)
  int d;
};

struct AppendArgs {
  const void *k1n, *k2n, *vn;  // new rows [B, H, d] / [B, H, 2d]
  void *k1c, *k2c, *vc;        // caches [B, H, L, d] / [B, H, L, 2d]
  int32_t* cache_len;          // [B], updated in place
  int64_t B, H, L;
};

// x [B, N, d_model] times the fused weight w [(H + 2 Hkv) 2d, d_model] (rows: W_Q, W_K,
// W_V), scattered into q1, q2 [B, H, N, d], k1, k2 [B, Hkv, N, d] and v [B, Hkv, N, 2d].
struct QkvProjArgs {
  const void *x, *w;
  void *q1, *q2, *k1, *k2, *v;
  int64_t B, H, N, d_model;
  int64_t Hkv;               // heads of k1, k2, v
  int d;
};

// y [M, d_model] = attn [M, k] times w [d_model, k] transposed.
struct OutProjArgs {
  const void *attn, *w;
  void* y;
  int64_t M, d_model, k;
};

hipError_t launch_qkv_proj_bf16(const QkvProjArgs& a, hipStream_t s);
hipError_t launch_out_proj_bf16(const OutProjArgs& a, hipStream_t s);

hipError_t launch_lambda(int dim, int layer, const float* lq1, const float* lk1,
                         const float* lq2, const float* lk2, diffattn_lambda_state* out,
                         hipStream_t s);
hipError_t launch_lambda_layers(int dim, int n_layers, int first, bool fixed, double init_value,
                                const float* lq1, const float* lk1, const float* lq2,
                                const float* lk2, diffattn_lambda_state* out, hipStream_t s);
hipError_t launch_fwd_fp32(const FwdArgs& a, hipStream_t s);
hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t s);
size_t fwd_bf16_workspace_bytes(int64_t B, int64_t H, int64_t N);
hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t s);
hipError_t launch_bwd_bf16(const BwdArgs& a, hipStream_t s);
hipError_t launch_cache_append_bf16(const AppendArgs& a, hipStream_t s);

// Device address of the static decode scratch (DIFFATTN_DECODE_SCRATCH_BYTES) on the
// current device, looked up once per device.
hipError_t decode_scratch(float** out);
// Decode geometry shared by the workspace query and the launcher: query heads per
// workgroup, and the splits of the cache.
void decode_geometry(int64_t B, int64_t H, int64_t G, int64_t L, int* gq, int* n_split,
                     int* split_len);
// Backward workspace floats.
size_t bwd_workspace_floats(int64_t B, int64_t H, int64_t N, int d);

}  // namespace diffattn
