// lambda and lambda_init of one layer, in float64 on the device.
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

__global__ void __launch_bounds__(64) lambda_kernel(int dim, int layer, const float* __restrict__ lq1,
                                                    const float* __restrict__ lk1,
                                                    const float* __restrict__ lq2,
                                                    const float* __restrict__ lk2,
                                                    diffattn_lambda_state* __restrict__ out) {
  if (threadIdx.x != 0) return;
  // Each product of two float32 values is exact in float64; the sums round once per term.
  double a = 0.0, b = 0.0;
  for (int i = 0; i < dim; ++i) a = a + static_cast<double>(lq1[i]) * static_cast<double>(lk1[i]);
  for (int i = 0; i < dim; ++i) b = b + static_cast<double>(lq2[i]) * static_cast<double>(lk2[i]);
  const double t = -0.3 * static_cast<double>(layer - 1);
  const double e = exp(t);
  const double init = 0.8 - 0.6 * e;
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

hipError_t launch_lambda(int dim, int layer, const float* lq1, const float* lk1,
                         const float* lq2, const float* lk2, diffattn_lambda_state* out,
                         hipStream_t s) {
  hipLaunchKernelGGL(lambda_kernel, dim3(1), dim3(64), 0, s, dim, layer, lq1, lk1, lq2, lk2, out);
  return hipGetLastError();
}

}  // namespace diffattn
