// Backward pass of causal DiffAttn (bf16, d = 64, V and output 128 wide).
//
// The pages print no gradient formulas; these follow from the forward definition by the
// chain rule (forward: DiffAttn equation of "Differential Transformer: Transformer que
// cancela ruido de atencao", pt.news.hada.io, "Como a atencao diferencial funciona";
// per-head RMSNorm and the (1 - lambda_init) factor, intoai.pub "Differential Attention
// With Multiple Heads"). With O = O1 - lambda O2, O_k = A_k V, r = rstd and
// g = (1 - lambda_init) w dY:
//   G   = dL/dO = r g - O r^3 rowsum(g O) / 2d           (bwd_pre_kernel)
//   D_k = rowsum(G O_k)
//   dV  = (A1 - lambda A2)^T G                            (bwd_dkdv_kernel)
//   dP  = G V^T
//   dS1 = A1 (dP - D1),  dS2 = -lambda A2 (dP - D2)
//   dK_k = s dS_k^T Q_k                                   (bwd_dkdv_kernel)
//   dQ_k = s dS_k K_k                                     (bwd_dq_kernel)
//   dlambda = -sum over rows of D2; lambda = exp(lq1.lk1) - exp(lq2.lk2) + lambda_init gives
//   dlq1 = dlambda e^a lk1, dlk1 = dlambda e^a lq1, dlq2 = -dlambda e^b lk2,
//   dlk2 = -dlambda e^b lq2                               (lambda_grad_kernel)
// A_k is recomputed from the log-sum-exps the forward saved: A_k = exp(S_k - lse_k).
//
// Two MFMA kernels, no atomics (deterministic):
//  * bwd_dkdv_kernel: a workgroup owns 128 keys (32 per wavefront) with dV^T, dK1^T, dK2^T
//    accumulating in registers, and streams the query tiles at or after its keys.
//  * bwd_dq_kernel: a workgroup owns 128 queries with dQ1^T, dQ2^T in registers and
//    streams the key tiles up to its diagonal.
// Score tiles are formed so that each lane's registers hold 8 consecutive contraction
// indices per k-step (rows of the A operand permuted, bits 2 and 3 swapped), which makes
// them directly the B operand of the following product; A operands that need the
// contraction index contiguous come from the transposing LDS read ds_read_b64_tr_b16.
#include "common.h"
#include "launch.h"

namespace diffattn {
namespace bwd {

#define LDS_AS __attribute__((address_space(3)))

constexpr int D = 64;
constexpr int DV = 128;
constexpr int NT = 256;   // 4 wavefronts
constexpr int BW = 128;   // rows (keys or queries) owned by a workgroup
constexpr int TB = 64;    // rows per streamed tile

// Row layout: rows of RB bytes; 16-byte unit u of row r stored at u ^ swizzle(r), so the
// 16 permuted operand rows a group of 16 lanes reads hit 16 different bank slots.
__device__ __forceinline__ int rsw8(int r) { return ((r ^ (r >> 2)) & 1) | (r & 2) | ((r >> 1) & 4); }
__device__ __forceinline__ int rsw16(int r) { return (r & 15) ^ (((r >> 3) & 1) << 2); }
// Transposed-read layout: 32-column regions of [TB rows][64 B]; 16-byte chunk c of row r
// stored at c ^ tsw(r).
__device__ __forceinline__ int tsw(int r) { return 2 * ((r >> 1) & 1); }
constexpr int TREG = TB * 64;   // bytes per 32-column region

__device__ __forceinline__ int perm_row(int m) {
  return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}
// Index (0..31 within a 32-row sub-tile) held in score register j by lane half h.
__device__ __forceinline__ int idx_of(int j, int h) { return 16 * (j >> 3) + 8 * h + (j & 7); }

__device__ __forceinline__ bf16x8 ld8(const char* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
// A operand from a transposed-read region: lane reads 8 consecutive rows of one column.
__device__ __forceinline__ bf16x8 ld_tr(const char* p) {
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)(p));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)(p + 4 * 64));
  const s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}

// Per-lane base of the transposed reads (row 0 of region 0).
__device__ __forceinline__ int tr_base(int lane) {
  const int G = lane >> 4, j = (lane >> 2) & 3, a = lane & 3;
  const int row = 8 * (G >> 1) + j;
  const int cp = 2 * (G & 1) + (a >> 1);
  return row * 64 + 16 * (cp ^ tsw(row)) + 8 * (a & 1);
}

// Copies rows [r0, r0 + TB) of a [N, W] bf16 tensor (rows >= N read as zero) into a row
// layout (rowbuf, may be null) and a transposed-read layout (trbuf, may be null).
template <int W>
__device__ __forceinline__ void stage_tile(const bf16_t* __restrict__ src, int r0, int N,
                                           char* rowbuf, char* trbuf, int tid) {
  constexpr int CPR = W / 8;            // 16-byte chunks per row
  constexpr int PER = TB * CPR / NT;    // chunks per thread
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int ch = tid + NT * i;
    const int row = ch / CPR, cc = ch % CPR;
    const int gr = r0 + row;
    u32x4 x = {0u, 0u, 0u, 0u};
    if (gr < N) x = *reinterpret_cast<const u32x4*>(src + static_cast<int64_t>(gr) * W + 8 * cc);
    if (rowbuf) {
      const int sw = (CPR == 8) ? rsw8(row) : rsw16(row);
      *reinterpret_cast<u32x4*>(rowbuf + row * (W * 2) + 16 * (cc ^ sw)) = x;
    }
    if (trbuf) {
      const int region = cc >> 2, c = cc & 3;
      *reinterpret_cast<u32x4*>(trbuf + region * TREG + row * 64 + 16 * (c ^ tsw(row))) = x;
    }
  }
}

// Row-layout A operand address for operand row m (permuted) of sub-tile sub, k-step kb.
template <int W>
__device__ __forceinline__ int row_addr(int m, int h, int sub, int kb) {
  const int row = 32 * sub + perm_row(m);
  const int sw = (W == 64) ? rsw8(row) : rsw16(row);
  return row * (W * 2) + 16 * ((2 * kb + h) ^ sw);
}

__device__ __forceinline__ bf16x8 to_bf16x8(const float* x) {
  f32x8 t;
#pragma unroll
  for (int e = 0; e < 8; ++e) t[e] = x[e];
  return __builtin_convertvector(t, bf16x8);
}

// ------------------------------------------------------------------------ bwd_pre
// 8 rows per workgroup, 32 threads per row, 4 channels per thread.
__global__ void __launch_bounds__(256) bwd_pre_kernel(
    const float* __restrict__ o1, const float* __restrict__ o2, const float* __restrict__ rstd,
    const bf16_t* __restrict__ dout, const diffattn_lambda_state* __restrict__ lamst,
    const float* __restrict__ rms_w, float* __restrict__ d_attn, bf16_t* __restrict__ gb,
    float* __restrict__ dd1, float* __restrict__ dd2, float* __restrict__ part, int64_t rows,
    int64_t N, int64_t H) {
  __shared__ float red[8];
  const int tid = threadIdx.x;
  const int t = tid & 31;
  const int64_t r = static_cast<int64_t>(blockIdx.x) * 8 + (tid >> 5);
  float d2 = 0.f;
  if (r < rows) {
    const int64_t hh = (r / N) % H;
    const float lam = lamst->lambda_f;
    const float gsc = lamst->one_minus_init_f;
    const f32x4 a = *reinterpret_cast<const f32x4*>(o1 + r * DV + 4 * t);
    const f32x4 b = *reinterpret_cast<const f32x4*>(o2 + r * DV + 4 * t);
    const u32x2 dy = *reinterpret_cast<const u32x2*>(dout + r * DV + 4 * t);
    f32x4 w = {1.f, 1.f, 1.f, 1.f};
    if (rms_w) w = *reinterpret_cast<const f32x4*>(rms_w + hh * DV + 4 * t);
    const float dyv[4] = {__uint_as_float(dy[0] << 16), __uint_as_float(dy[0] & 0xffff0000u),
                          __uint_as_float(dy[1] << 16), __uint_as_float(dy[1] & 0xffff0000u)};
    const float rs = rstd[r];
    float o[4], g[4], go = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      o[e] = a[e] - lam * b[e];
      g[e] = gsc * w[e] * dyv[e];
      go = fmaf(g[e], o[e], go);
    }
#pragma unroll
    for (int off = 16; off > 0; off >>= 1) go += __shfl_xor(go, off);
    const float k3 = rs * rs * rs * go * (1.0f / DV);
    // The D_k used in dS pair with dP = G V^T, which the MFMAs form from the bf16-rounded
    // G, so they are formed from the same rounded values: for a row that sees one key
    // dP - D_k is then zero up to summation order, as it is exactly. dlambda = -sum D2 is
    // summed from the float32 G (d2), where that rounding would swamp rows whose D2 is a
    // near-cancellation.
    f32x4 G;
    float d1 = 0.f, d2b = 0.f;
    u32x2 gp;
#pragma unroll
    for (int e = 0; e < 4; ++e) G[e] = rs * g[e] - o[e] * k3;
    gp[0] = pack_bf16x2(G[0], G[1]);
    gp[1] = pack_bf16x2(G[2], G[3]);
    const float gr[4] = {__uint_as_float(gp[0] << 16), __uint_as_float(gp[0] & 0xffff0000u),
                         __uint_as_float(gp[1] << 16), __uint_as_float(gp[1] & 0xffff0000u)};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      d1 = fmaf(gr[e], a[e], d1);
      d2b = fmaf(gr[e], b[e], d2b);
      d2 = fmaf(G[e], b[e], d2);
    }
#pragma unroll
    for (int off = 16; off > 0; off >>= 1) {
      d1 += __shfl_xor(d1, off);
      d2b += __shfl_xor(d2b, off);
      d2 += __shfl_xor(d2, off);
    }
    *reinterpret_cast<f32x4*>(d_attn + r * DV + 4 * t) = G;
    *reinterpret_cast<u32x2*>(gb + r * DV + 4 * t) = gp;
    if (t == 0) {
      dd1[r] = d1;
      dd2[r] = d2b;
    }
  }
  if (t == 0) red[tid >> 5] = r < rows ? d2 : 0.f;
  __syncthreads();
  if (tid == 0) {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) s += red[i];
    part[blockIdx.x] = s;   // sum of D2 (float32 G) over this block's rows
  }
}

// ------------------------------------------------------------------------ lambda grads
__global__ void __launch_bounds__(256) lambda_grad_kernel(
    const float* __restrict__ part, int64_t nparts, const diffattn_lambda_state* __restrict__ lamst,
    const float* __restrict__ lq1, const float* __restrict__ lk1, const float* __restrict__ lq2,
    const float* __restrict__ lk2, float* __restrict__ dlq1, float* __restrict__ dlk1,
    float* __restrict__ dlq2, float* __restrict__ dlk2, int d) {
  __shared__ double red[256];
  const int tid = threadIdx.x;
  double s = 0.0;
  for (int64_t i = tid; i < nparts; i += 256) s += static_cast<double>(part[i]);
  red[tid] = s;
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if (tid < off) red[tid] += red[tid + off];
    __syncthreads();
  }
  const double dlam = -red[0];
  const double ea = lamst->exp_a, eb = lamst->exp_b;
  for (int i = tid; i < d; i += 256) {
    dlq1[i] = static_cast<float>(dlam * ea * static_cast<double>(lk1[i]));
    dlk1[i] = static_cast<float>(dlam * ea * static_cast<double>(lq1[i]));
    dlq2[i] = static_cast<float>(-dlam * eb * static_cast<double>(lk2[i]));
    dlk2[i] = static_cast<float>(-dlam * eb * static_cast<double>(lq2[i]));
  }
}

// ------------------------------------------------------------------------ dK, dV
// LDS: Q1, Q2 in row and transposed layouts, G in row and transposed layouts, and the
// tile's lse1, lse2 (log2 units), D1, D2.
constexpr int KV_Q1R = 0;
constexpr int KV_Q2R = KV_Q1R + TB * D * 2;
constexpr int KV_Q1T = KV_Q2R + TB * D * 2;
constexpr int KV_Q2T = KV_Q1T + 2 * TREG;
constexpr int KV_GR = KV_Q2T + 2 * TREG;
constexpr int KV_GT = KV_GR + TB * DV * 2;
constexpr int KV_VEC = KV_GT + 4 * TREG;
constexpr int KV_LDS = KV_VEC + 4 * TB * 4;

__global__ void __launch_bounds__(NT, 1) bwd_dkdv_kernel(
    const bf16_t* __restrict__ q1, const bf16_t* __restrict__ q2, const bf16_t* __restrict__ k1,
    const bf16_t* __restrict__ k2, const bf16_t* __restrict__ v, const bf16_t* __restrict__ gb,
    const float* __restrict__ lse1, const float* __restrict__ lse2, const float* __restrict__ dd1,
    const float* __restrict__ dd2, const diffattn_lambda_state* __restrict__ lamst,
    bf16_t* __restrict__ dk1, bf16_t* __restrict__ dk2, bf16_t* __restrict__ dv, int BH, int N,
    int nkb) {
  __shared__ __attribute__((aligned(16))) char lds[KV_LDS];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int m = lane & 31, h = lane >> 5;
  const int bid = blockIdx.x;
  const int bh = bid % BH;
  const int kb = bid / BH;             // early key blocks see the most queries: first
  const int k0 = kb * BW;
  const int k0w = k0 + 32 * wv;
  const int64_t ho = static_cast<int64_t>(bh) * N;
  const bf16_t* Q1 = q1 + ho * D;
  const bf16_t* Q2 = q2 + ho * D;
  const bf16_t* Gg = gb + ho * DV;

  // Resident B operands: K^T and V^T columns of this wave's 32 keys.
  bf16x8 kf1[4], kf2[4], vf[8];
  {
    const int key = k0w + m;
    const bool ok = key < N;
    const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const u32x4 a = ok ? *reinterpret_cast<const u32x4*>(k1 + (ho + key) * D + 16 * i + 8 * h) : z;
      const u32x4 b = ok ? *reinterpret_cast<const u32x4*>(k2 + (ho + key) * D + 16 * i + 8 * h) : z;
      kf1[i] = __builtin_bit_cast(bf16x8, a);
      kf2[i] = __builtin_bit_cast(bf16x8, b);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const u32x4 a = ok ? *reinterpret_cast<const u32x4*>(v + (ho + key) * DV + 16 * i + 8 * h) : z;
      vf[i] = __builtin_bit_cast(bf16x8, a);
    }
  }
  const float lam = lamst->lambda_f;
  const float c = kLog2e / 8.0f;
  f32x16 adv[4], adk1[2], adk2[2];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
#pragma unroll
    for (int b = 0; b < 4; ++b) adv[b][j] = 0.f;
#pragma unroll
    for (int b = 0; b < 2; ++b) adk1[b][j] = adk2[b][j] = 0.f;
  }
  const int trb = tr_base(lane);
  const float* vec = reinterpret_cast<const float*>(lds + KV_VEC);
  const int key = k0w + m;

  const int n_qt = (N + TB - 1) / TB;
  for (int qt = k0 / TB; qt < n_qt; ++qt) {
    const int qb = qt * TB;
    __syncthreads();
    stage_tile<D>(Q1, qb, N, lds + KV_Q1R, lds + KV_Q1T, tid);
    stage_tile<D>(Q2, qb, N, lds + KV_Q2R, lds + KV_Q2T, tid);
    stage_tile<DV>(Gg, qb, N, lds + KV_GR, lds + KV_GT, tid);
    if (tid < TB) {
      const int q = qb + tid;
      float* vw = reinterpret_cast<float*>(lds + KV_VEC);
      // rows beyond N: lse = +inf makes their weights exactly zero
      vw[tid] = q < N ? lse1[ho + q] * kLog2e : INFINITY;
      vw[TB + tid] = q < N ? lse2[ho + q] * kLog2e : INFINITY;
      vw[2 * TB + tid] = q < N ? dd1[ho + q] : 0.f;
      vw[3 * TB + tid] = q < N ? dd2[ho + q] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const int qs = qb + 32 * sub;
      if (qs + 31 < k0w) continue;  // every query of the sub-tile precedes every key
      f32x16 s1, s2, dp;
#pragma unroll
      for (int j = 0; j < 16; ++j) s1[j] = s2[j] = dp[j] = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int ra = row_addr<D>(m, h, sub, i);
        s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ld8(lds + KV_Q1R + ra), kf1[i], s1, 0, 0, 0);
        s2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ld8(lds + KV_Q2R + ra), kf2[i], s2, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int ra = row_addr<DV>(m, h, sub, i);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ld8(lds + KV_GR + ra), vf[i], dp, 0, 0, 0);
      }
      // Weights and score gradients; register j holds query qs + idx_of(j, h) for key.
      float pc[16], g1[16], g2[16];
      const bool need_mask = qs < k0w + 31;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int qi = 32 * sub + idx_of(j, h);
        float p1 = fast_exp2(fmaf(s1[j], c, -vec[qi]));
        float p2 = fast_exp2(fmaf(s2[j], c, -vec[TB + qi]));
        if (need_mask && key > qb + qi) {
          p1 = 0.f;
          p2 = 0.f;
        }
        pc[j] = p1 - lam * p2;
        g1[j] = p1 * (dp[j] - vec[2 * TB + qi]);
        g2[j] = -lam * p2 * (dp[j] - vec[3 * TB + qi]);
      }
      const bf16x8 pca = to_bf16x8(pc), pcb = to_bf16x8(pc + 8);
      const bf16x8 g1a = to_bf16x8(g1), g1b = to_bf16x8(g1 + 8);
      const bf16x8 g2a = to_bf16x8(g2), g2b = to_bf16x8(g2 + 8);
      // dV^T[dv][key] += G^T (P1 - lambda P2); dK_k^T[d][key] += Q_k^T dS_k
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const char* p = lds + KV_GT + b * TREG + trb + (32 * sub) * 64;
        adv[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ld_tr(p), pca, adv[b], 0, 0, 0);
        adv[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ld_tr(p + 16 * 64), pcb, adv[b], 0, 0, 0);
      }
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const char* p1 = lds + KV_Q1T + b * TREG + trb + (32 * sub) * 64;
        const char* p2 = lds + KV_Q2T + b * TREG + trb + (32 * sub) * 64;
        adk1[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ld_tr(p1), g1a, adk1[b], 0, 0, 0);
        adk1[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ld_tr(p1 + 16 * 64), g1b, adk1[b], 0, 0, 0);
        adk2[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ld_tr(p2), g2a, adk2[b], 0, 0, 0);
        adk2[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ld_tr(p2 + 16 * 64), g2b, adk2[b], 0, 0, 0);
      }
    }
  }
  // Stores: register j of block b holds channel 32 b + 8 (j / 4) + 4 h + j % 4 of key.
  if (key < N) {
    const float s = 0.125f;  // 1 / sqrt(64)
#pragma unroll
    for (int b = 0; b < 4; ++b) {
#pragma unroll
      for (int jg = 0; jg < 4; ++jg) {
        const int col = 32 * b + 8 * jg + 4 * h;
        u32x2 pk = {pack_bf16x2(adv[b][4 * jg], adv[b][4 * jg + 1]),
                    pack_bf16x2(adv[b][4 * jg + 2], adv[b][4 * jg + 3])};
        *reinterpret_cast<u32x2*>(dv + (ho + key) * DV + col) = pk;
      }
    }
#pragma unroll
    for (int b = 0; b < 2; ++b) {
#pragma unroll
      for (int jg = 0; jg < 4; ++jg) {
        const int col = 32 * b + 8 * jg + 4 * h;
        u32x2 p1 = {pack_bf16x2(s * adk1[b][4 * jg], s * adk1[b][4 * jg + 1]),
                    pack_bf16x2(s * adk1[b][4 * jg + 2], s * adk1[b][4 * jg + 3])};
        u32x2 p2 = {pack_bf16x2(s * adk2[b][4 * jg], s * adk2[b][4 * jg + 1]),
                    pack_bf16x2(s * adk2[b][4 * jg + 2], s * adk2[b][4 * jg + 3])};
        *reinterpret_cast<u32x2*>(dk1 + (ho + key) * D + col) = p1;
        *reinterpret_cast<u32x2*>(dk2 + (ho + key) * D + col) = p2;
      }
    }
  }
}

// ------------------------------------------------------------------------ dQ
// LDS: K1, K2 in row and transposed layouts, V in the row layout.
constexpr int Q_K1R = 0;
constexpr int Q_K2R = Q_K1R + TB * D * 2;
constexpr int Q_K1T = Q_K2R + TB * D * 2;
constexpr int Q_K2T = Q_K1T + 2 * TREG;
constexpr int Q_VR = Q_K2T + 2 * TREG;
constexpr int Q_LDS = Q_VR + TB * DV * 2;

__global__ void __launch_bounds__(NT, 1) bwd_dq_kernel(
    const bf16_t* __restrict__ q1, const bf16_t* __restrict__ q2, const bf16_t* __restrict__ k1,
    const bf16_t* __restrict__ k2, const bf16_t* __restrict__ v, const bf16_t* __restrict__ gb,
    const float* __restrict__ lse1, const float* __restrict__ lse2, const float* __restrict__ dd1,
    const float* __restrict__ dd2, const diffattn_lambda_state* __restrict__ lamst,
    bf16_t* __restrict__ dq1, bf16_t* __restrict__ dq2, int BH, int N, int nqb) {
  __shared__ __attribute__((aligned(16))) char lds[Q_LDS];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int m = lane & 31, h = lane >> 5;
  const int bid = blockIdx.x;
  const int bh = bid % BH;
  const int qb = nqb - 1 - bid / BH;   // late query blocks see the most keys: first
  const int q0 = qb * BW;
  const int q0w = q0 + 32 * wv;
  const int64_t ho = static_cast<int64_t>(bh) * N;
  const int q = q0w + m;
  const bool qok = q < N;

  // Resident B operands: Q^T and G^T columns of this wave's 32 queries.
  bf16x8 qf1[4], qf2[4], gf[8];
  {
    const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const u32x4 a = qok ? *reinterpret_cast<const u32x4*>(q1 + (ho + q) * D + 16 * i + 8 * h) : z;
      const u32x4 b = qok ? *reinterpret_cast<const u32x4*>(q2 + (ho + q) * D + 16 * i + 8 * h) : z;
      qf1[i] = __builtin_bit_cast(bf16x8, a);
      qf2[i] = __builtin_bit_cast(bf16x8, b);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const u32x4 a = qok ? *reinterpret_cast<const u32x4*>(gb + (ho + q) * DV + 16 * i + 8 * h) : z;
      gf[i] = __builtin_bit_cast(bf16x8, a);
    }
  }
  const float l1 = qok ? lse1[ho + q] * kLog2e : INFINITY;
  const float l2 = qok ? lse2[ho + q] * kLog2e : INFINITY;
  const float D1 = qok ? dd1[ho + q] : 0.f;
  const float D2 = qok ? dd2[ho + q] : 0.f;
  const float lam = lamst->lambda_f;
  const float c = kLog2e / 8.0f;
  f32x16 aq1[2], aq2[2];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
#pragma unroll
    for (int b = 0; b < 2; ++b) aq1[b][j] = aq2[b][j] = 0.f;
  }
  const int trb = tr_base(lane);

  const int kend = min(N, q0 + BW);
  const int n_kt = (kend + TB - 1) / TB;
  for (int kt = 0; kt < n_kt; ++kt) {
    const int kb0 = kt * TB;
    __syncthreads();
    stage_tile<D>(k1 + ho * D, kb0, N, lds + Q_K1R, lds + Q_K1T, tid);
    stage_tile<D>(k2 + ho * D, kb0, N, lds + Q_K2R, lds + Q_K2T, tid);
    stage_tile<DV>(v + ho * DV, kb0, N, lds + Q_VR, nullptr, tid);
    __syncthreads();
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const int ks = kb0 + 32 * sub;
      if (ks > q0w + 31) continue;  // every key of the sub-tile follows every query
      f32x16 s1, s2, dp;
#pragma unroll
      for (int j = 0; j < 16; ++j) s1[j] = s2[j] = dp[j] = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int ra = row_addr<D>(m, h, sub, i);
        s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ld8(lds + Q_K1R + ra), qf1[i], s1, 0, 0, 0);
        s2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ld8(lds + Q_K2R + ra), qf2[i], s2, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int ra = row_addr<DV>(m, h, sub, i);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ld8(lds + Q_VR + ra), gf[i], dp, 0, 0, 0);
      }
      float g1[16], g2[16];
      const bool need_mask = ks + 31 > q0w;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        float p1 = fast_exp2(fmaf(s1[j], c, -l1));
        float p2 = fast_exp2(fmaf(s2[j], c, -l2));
        if (need_mask && ks + idx_of(j, h) > q) {
          p1 = 0.f;
          p2 = 0.f;
        }
        g1[j] = p1 * (dp[j] - D1);
        g2[j] = -lam * p2 * (dp[j] - D2);
      }
      const bf16x8 g1a = to_bf16x8(g1), g1b = to_bf16x8(g1 + 8);
      const bf16x8 g2a = to_bf16x8(g2), g2b = to_bf16x8(g2 + 8);
      // dQ_k^T[d][q] += K_k^T dS_k^T
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const char* p1 = lds + Q_K1T + b * TREG + trb + (32 * sub) * 64;
        const char* p2 = lds + Q_K2T + b * TREG + trb + (32 * sub) * 64;
        aq1[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ld_tr(p1), g1a, aq1[b], 0, 0, 0);
        aq1[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ld_tr(p1 + 16 * 64), g1b, aq1[b], 0, 0, 0);
        aq2[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ld_tr(p2), g2a, aq2[b], 0, 0, 0);
        aq2[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ld_tr(p2 + 16 * 64), g2b, aq2[b], 0, 0, 0);
      }
    }
  }
  if (qok) {
    const float s = 0.125f;  // 1 / sqrt(64)
#pragma unroll
    for (int b = 0; b < 2; ++b) {
#pragma unroll
      for (int jg = 0; jg < 4; ++jg) {
        const int col = 32 * b + 8 * jg + 4 * h;
        u32x2 p1 = {pack_bf16x2(s * aq1[b][4 * jg], s * aq1[b][4 * jg + 1]),
                    pack_bf16x2(s * aq1[b][4 * jg + 2], s * aq1[b][4 * jg + 3])};
        u32x2 p2 = {pack_bf16x2(s * aq2[b][4 * jg], s * aq2[b][4 * jg + 1]),
                    pack_bf16x2(s * aq2[b][4 * jg + 2], s * aq2[b][4 * jg + 3])};
        *reinterpret_cast<u32x2*>(dq1 + (ho + q) * D + col) = p1;
        *reinterpret_cast<u32x2*>(dq2 + (ho + q) * D + col) = p2;
      }
    }
  }
}

}  // namespace bwd

// Workspace (floats): bf16 G [rows, 128] (64 floats per row), D1 and D2 [rows], and one
// partial sum of D2 per 8 rows.
size_t bwd_workspace_floats(int64_t B, int64_t H, int64_t N, int d) {
  (void)d;
  const int64_t rows = B * H * N;
  return static_cast<size_t>(rows) * (bwd::DV / 2 + 2) + static_cast<size_t>((rows + 7) / 8) + 64;
}

hipError_t launch_bwd_bf16(const BwdArgs& a, hipStream_t s) {
  using namespace bwd;
  const int64_t rows = a.B * a.H * a.N;
  const int64_t nparts = (rows + 7) / 8;
  bf16_t* gbuf = reinterpret_cast<bf16_t*>(a.ws);
  float* dd1 = a.ws + rows * (DV / 2);
  float* dd2 = dd1 + rows;
  float* part = dd2 + rows;
  if (rows > 0) {
    hipLaunchKernelGGL(bwd_pre_kernel, dim3(static_cast<unsigned>(nparts)), dim3(256), 0, s,
                       a.saved.o1, a.saved.o2, a.saved.rstd, static_cast<const bf16_t*>(a.dout),
                       a.lam, a.rms_weight, a.d_attn, gbuf, dd1, dd2, part, rows, a.N, a.H);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int BH = static_cast<int>(a.B * a.H);
    const int N = static_cast<int>(a.N);
    const int nb = static_cast<int>((a.N + BW - 1) / BW);
    hipLaunchKernelGGL(bwd_dkdv_kernel, dim3(static_cast<unsigned>(BH * nb)), dim3(NT), 0, s,
                       static_cast<const bf16_t*>(a.q1), static_cast<const bf16_t*>(a.q2),
                       static_cast<const bf16_t*>(a.k1), static_cast<const bf16_t*>(a.k2),
                       static_cast<const bf16_t*>(a.v), gbuf, a.saved.lse1, a.saved.lse2, dd1,
                       dd2, a.lam, static_cast<bf16_t*>(a.dk1), static_cast<bf16_t*>(a.dk2),
                       static_cast<bf16_t*>(a.dv), BH, N, nb);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(bwd_dq_kernel, dim3(static_cast<unsigned>(BH * nb)), dim3(NT), 0, s,
                       static_cast<const bf16_t*>(a.q1), static_cast<const bf16_t*>(a.q2),
                       static_cast<const bf16_t*>(a.k1), static_cast<const bf16_t*>(a.k2),
                       static_cast<const bf16_t*>(a.v), gbuf, a.saved.lse1, a.saved.lse2, dd1,
                       dd2, a.lam, static_cast<bf16_t*>(a.dq1), static_cast<bf16_t*>(a.dq2), BH,
                       N, nb);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(lambda_grad_kernel, dim3(1), dim3(256), 0, s, part, rows > 0 ? nparts : 0,
                     a.lam, a.lq1, a.lk1, a.lq2, a.lk2, a.dlq1, a.dlk1, a.dlq2, a.dlk2, a.d);
  return hipGetLastError();
}

}  // namespace diffattn
