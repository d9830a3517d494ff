// lambda and lambda_init of one layer (or of several layers in one launch), in float64 on
// the device.
//
// lambda_init = 0.8 - 0.6 * exp(-0.3 * (l - 1)) and
// lambda = exp(lq1 . lk1) - exp(lq2 . lk2) + lambda_init
// ("Differential Transformer: Transformer que cancela ruido de atencao",
//  pt.news.hada.io, section "Como a atencao diferencial funciona").
// One scalar per layer, shared by every head (intoai.pub, "Differential Attention With
// Multiple Heads").
//
// Each step is one rounded float64 operation in the order written (contraction into
// fused multiply-adds is switched off), the dot products are summed in index order,
// and the float32 fields are the float64 results rounded once to nearest even.
#include "common.h"
#include "launch.h"

namespace diffattn {

#pragma clang fp contract(off)

// Lane j's 64-bit value, read by every lane (j is the same in every lane).
__device__ __forceinline__ double lane_value(double x, int j) {
  const uint64_t u = static_cast<uint64_t>(__double_as_longlong(x));
  const uint32_t lo = __builtin_amdgcn_readlane(static_cast<uint32_t>(u), j);
  const uint32_t hi = __builtin_amdgcn_readlane(static_cast<uint32_t>(u >> 32), j);
  return __longlong_as_double(static_cast<long long>((static_cast<uint64_t>(hi) << 32) | lo));
}

// sum_i x[i] y[i] in float64, summed in index order, in every lane of the wavefront. The
// lanes load and multiply 64 terms at once (a product of two float32 values is exact in
// float64); the running sum then takes the terms one by one in index order.
__device__ __forceinline__ double ordered_dot(int dim, const float* __restrict__ x,
                                              const float* __restrict__ y, int lane) {
  double s = 0.0;
  for (int c = 0; c < dim; c += 64) {
    const int i = c + lane;
    const double p = i < dim ? static_cast<double>(x[i]) * static_cast<double>(y[i]) : 0.0;
    const int n = dim - c < 64 ? dim - c : 64;
    for (int j = 0; j < n; ++j) s = s + lane_value(p, j);
  }
  return s;
}

// One layer's state, computed by a whole wavefront and written by lane 0; with `fixed`,
// lambda_init is init_value (the pages also try one lambda_init for every layer alike,
// for example 0.8; same section), else the schedule. (The library is built assuming no
// NaNs, so no NaN serves as a marker here.)
__device__ __forceinline__ void lambda_state(int dim, int layer, bool fixed, double init_value,
                                             const float* __restrict__ lq1,
                                             const float* __restrict__ lk1,
                                             const float* __restrict__ lq2,
                                             const float* __restrict__ lk2,
                                             diffattn_lambda_state* __restrict__ out, int lane) {
  const double a = ordered_dot(dim, lq1, lk1, lane);
  const double b = ordered_dot(dim, lq2, lk2, lane);
  double init;
  if (fixed) {
    init = init_value;
  } else {
    const double t = -0.3 * static_cast<double>(layer - 1);
    const double e = exp(t);
    init = 0.8 - 0.6 * e;
  }
  const double ea = exp(a);
  const double eb = exp(b);
  const double lam = (ea - eb) + init;
  if (lane != 0) return;
  diffattn_lambda_state s;
  s.lambda = lam;
  s.lambda_init = init;
  s.exp_a = ea;
  s.exp_b = eb;
  s.lambda_f = static_cast<float>(lam);
  s.lambda_init_f = static_cast<float>(init);
  s.one_minus_init_f = static_cast<float>(1.0 - init);
  s.pad = 0.0f;
  *out = s;
}

// Workgroup k (one wavefront): layer first + k, vectors at k dim, state k.
__global__ void __launch_bounds__(64) lambda_kernel(int dim, int first, int fixed,
                                                    double init_value,
                                                    const float* __restrict__ lq1,
                                                    const float* __restrict__ lk1,
                                                    const float* __restrict__ lq2,
                                                    const float* __restrict__ lk2,
                                                    diffattn_lambda_state* __restrict__ out) {
  const int64_t k = blockIdx.x;
  lambda_state(dim, first + static_cast<int>(k), fixed != 0, init_value, lq1 + k * dim,
               lk1 + k * dim, lq2 + k * dim, lk2 + k * dim, out + k,
               static_cast<int>(threadIdx.x));
}

hipError_t launch_lambda(int dim, int layer, const float* lq1, const float* lk1,
                         const float* lq2, const float* lk2, diffattn_lambda_state* out,
                         hipStream_t s) {
  return launch_lambda_layers(dim, 1, layer, false, 0.0, lq1, lk1, lq2, lk2, out, s);
}

hipError_t launch_lambda_layers(int dim, int n_layers, int first, bool fixed, double init_value,
                                const float* lq1, const float* lk1, const float* lq2,
                                const float* lk2, diffattn_lambda_state* out, hipStream_t s) {
  hipLaunchKernelGGL(lambda_kernel, dim3(static_cast<unsigned>(n_layers)), dim3(64), 0, s, dim,
                     first, fixed ? 1 : 0, init_value, lq1, lk1, lq2, lk2, out);
  return hipGetLastError();
}

}  // namespace diffattn
