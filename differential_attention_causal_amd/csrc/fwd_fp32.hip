// Causal DiffAttn forward in float32 on the vector ALUs: the parity path for float32
// tensors (small heads, d in {16, 32, 64}).
//
// One wavefront owns one query row i. Keys are visited in chunks of 64 (one per lane)
// with an online softmax per map: running maximum m and normaliser l, so that
// O = acc1 / l1 - lambda * acc2 / l2 equals (A1 - lambda A2) V exactly in real
// arithmetic ("Differential Transformer: Transformer que cancela ruido de atencao",
// pt.news.hada.io, "Como a atencao diferencial funciona", DiffAttn equation; causal mask
// from intoai.pub "A Deeper Dive Into Attention Calculations"). The row is then RMS-
// normalised over its 2d channels and scaled by (1 - lambda_init) (intoai.pub
// "Differential Attention With Multiple Heads").
#include "common.h"
#include "launch.h"

namespace diffattn {

template <int D>
__global__ void __launch_bounds__(256) fwd_fp32_kernel(
    const float* __restrict__ q1, const float* __restrict__ q2, const float* __restrict__ k1,
    const float* __restrict__ k2, const float* __restrict__ v,
    const diffattn_lambda_state* __restrict__ lamst, const float* __restrict__ rms_w,
    float* __restrict__ out, int64_t H, int64_t N, float eps, int out_bnh, int64_t G) {
  constexpr int DV = 2 * D;
  constexpr int CPL = (DV + 63) / 64;  // output columns per lane
  __shared__ float qs[4][2][D];
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int64_t bh = blockIdx.y;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 4 + wv;
  const bool row_ok = i < N;
  const int64_t ii = row_ok ? i : N - 1;
  const float* Q1 = q1 + (bh * N + ii) * D;
  const float* Q2 = q2 + (bh * N + ii) * D;
  const int64_t kvh = (bh / H) * (H / G) + (bh % H) / G;   // K/V head (G per group)
  const float* K1 = k1 + kvh * N * D;
  const float* K2 = k2 + kvh * N * D;
  const float* V = v + kvh * N * DV;
  if (lane < D) {
    qs[wv][0][lane] = Q1[lane];
    qs[wv][1][lane] = Q2[lane];
  }
  __syncthreads();
  const float lam = lamst->lambda_f;
  const float scale = 1.0f / sqrtf(static_cast<float>(D));
  float m1 = -INFINITY, m2 = -INFINITY, l1 = 0.f, l2 = 0.f;
  float acc1[CPL], acc2[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) acc1[c] = acc2[c] = 0.f;

  for (int64_t c0 = 0; c0 <= ii; c0 += 64) {
    const int64_t j = c0 + lane;
    float s1 = -INFINITY, s2 = -INFINITY;
    if (j <= ii) {
      float d1 = 0.f, d2 = 0.f;
      for (int t = 0; t < D; ++t) {
        d1 = fmaf(qs[wv][0][t], K1[j * D + t], d1);
        d2 = fmaf(qs[wv][1][t], K2[j * D + t], d2);
      }
      s1 = d1 * scale;
      s2 = d2 * scale;
    }
    const float mn1 = fmaxf(m1, wave_max(s1));
    const float mn2 = fmaxf(m2, wave_max(s2));
    const float a1 = expf(m1 - mn1), a2 = expf(m2 - mn2);  // m = -inf at start gives 0
    const float p1 = (j <= ii) ? expf(s1 - mn1) : 0.f;
    const float p2 = (j <= ii) ? expf(s2 - mn2) : 0.f;
    l1 = l1 * a1 + wave_sum(p1);
    l2 = l2 * a2 + wave_sum(p2);
    m1 = mn1;
    m2 = mn2;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      acc1[c] *= a1;
      acc2[c] *= a2;
    }
    const int64_t jn = (ii - c0 + 1) < 64 ? (ii - c0 + 1) : 64;
    for (int jj = 0; jj < jn; ++jj) {
      const float pj1 = __shfl(p1, jj);
      const float pj2 = __shfl(p2, jj);
      const float* vr = V + (c0 + jj) * DV;
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        const int col = lane + 64 * c;
        if (col < DV) {
          const float vv = vr[col];
          acc1[c] = fmaf(pj1, vv, acc1[c]);
          acc2[c] = fmaf(pj2, vv, acc2[c]);
        }
      }
    }
  }
  float o[CPL];
  float ss = 0.f;
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const int col = lane + 64 * c;
    o[c] = acc1[c] / l1 - lam * (acc2[c] / l2);
    if (col < DV) ss = fmaf(o[c], o[c], ss);
  }
  ss = wave_sum(ss);
  const float rstd = 1.0f / sqrtf(ss / static_cast<float>(DV) + eps);
  const float g = lamst->one_minus_init_f;
  const int64_t h = bh % H;
  if (row_ok) {
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const int col = lane + 64 * c;
      if (col < DV) {
        const float w = rms_w ? rms_w[h * DV + col] : 1.0f;
        const int64_t yrow = out_bnh ? ((bh / H) * N + i) * H + h : bh * N + i;
        out[yrow * DV + col] = g * (w * (o[c] * rstd));
      }
    }
  }
}

hipError_t launch_fwd_fp32(const FwdArgs& a, hipStream_t s) {
  dim3 grid(static_cast<unsigned>((a.N + 3) / 4), static_cast<unsigned>(a.B * a.H));
  dim3 block(256);
#define DA_LAUNCH(DD)                                                                       \
  hipLaunchKernelGGL(fwd_fp32_kernel<DD>, grid, block, 0, s,                               \
                     static_cast<const float*>(a.q1), static_cast<const float*>(a.q2),      \
                     static_cast<const float*>(a.k1), static_cast<const float*>(a.k2),      \
                     static_cast<const float*>(a.v), a.lam, a.rms_weight,                   \
                     static_cast<float*>(a.out), a.H, a.N, a.eps, a.out_bnh ? 1 : 0,   \
                     static_cast<int64_t>(a.G))
  switch (a.d) {
    case 16: DA_LAUNCH(16); break;
    case 32: DA_LAUNCH(32); break;
    case 64: DA_LAUNCH(64); break;
    default: return hipErrorInvalidValue;
  }
#undef DA_LAUNCH
  return hipGetLastError();
}

}  // namespace diffattn
