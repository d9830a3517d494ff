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

// One layer's state; with `fixed`, lambda_init is init_value (the pages also try one
// lambda_init for every layer alike, for example 0.8; same section), else the schedule.
// (The library is built assuming no NaNs, so no NaN serves as a marker here.)
__device__ __noinline__ void lambda_state(int dim, int layer, bool fixed, double init_value,
                                          const float* __restrict__ lq1,
                                          const float* __restrict__ lk1,
                                          const float* __restrict__ lq2,
                                          const float* __restrict__ lk2,
                                          diffattn_lambda_state* __restrict__ out) {
  // Each product of two float32 values is exact in float64; the sums round once per term.
  double a = 0.0, b = 0.0;
  for (int i = 0; i < dim; ++i) a = a + static_cast<double>(lq1[i]) * static_cast<double>(lk1[i]);
  for (int i = 0; i < dim; ++i) b = b + static_cast<double>(lq2[i]) * static_cast<double>(lk2[i]);
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

// Workgroup k: layer first + k, vectors at k dim, state k.
__global__ void __launch_bounds__(64) lambda_kernel(int dim, int first, int fixed,
                                                    double init_value,
                                                    const float* __restrict__ lq1,
                                                    const float* __restrict__ lk1,
                                                    const float* __restrict__ lq2,
                                                    const float* __restrict__ lk2,
                                                    diffattn_lambda_state* __restrict__ out) {
  if (threadIdx.x != 0) return;
  const int64_t k = blockIdx.x;
  lambda_state(dim, first + static_cast<int>(k), fixed != 0, init_value, lq1 + k * dim,
               lk1 + k * dim, lq2 + k * dim, lk2 + k * dim, out + k);
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
