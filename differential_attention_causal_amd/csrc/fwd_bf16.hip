// Fused causal DiffAttn forward for bf16 tensors with d = 64 (V and output 128 wide), on
// the gfx950 matrix cores.
//
// What it computes, per head: O = (A1 - lambda A2) V with A_k the causal row softmax of
// Q_k K_k^T / sqrt(d) ("Differential Transformer: Transformer que cancela ruido de
// atencao", pt.news.hada.io, "Como a atencao diferencial funciona", DiffAttn equation;
// causal mask from intoai.pub "A Deeper Dive Into Attention Calculations"), then
// Y = (1 - lambda_init) * RMSNorm(O) per head (intoai.pub "Differential Attention With
// Multiple Heads").
//
// The pages note that the method can be run blockwise like ordinary attention with an
// extra pair of maps. Here that means: both maps are evaluated over key tiles with their
// own online-softmax state (running max m_k and normaliser l_k per query row), the two
// accumulators acc_k = sum_j exp(S_k - m_k) V_j share each V tile, and only at the end is
// O = acc1 / l1 - lambda acc2 / l2 formed, normalised and scaled. That is exact in real
// arithmetic; nothing is approximated.
//
// Work decomposition (one workgroup = 4 wavefronts = 128 query rows of one (b, h)):
//  * each wavefront owns 32 query rows and computes the transposed score tile
//    S^T = K Q^T (32 keys x 32 queries) with v_mfma_f32_32x32x16_bf16, so each lane
//    holds 16 scores of ONE query; the row max needs one exchange with lane ^ 32;
//  * the key rows fed to the MFMA are permuted (bits 2 and 3 of the row swapped) so
//    that the score registers are directly the B operand of O^T += V^T P^T, with each
//    lane's 8 keys contiguous in the transposed V tile;
//  * K1, K2 (64 keys x 64) and V^T (128 x 64 keys) tiles are staged through LDS, double
//    buffered, with XOR swizzles that keep the 16-byte reads conflict-free; V is
//    transposed in registers on its way to LDS;
//  * the diagonal tile applies the causal predicate key <= query as an integer compare;
//    tiles above the diagonal are skipped, rows beyond N and keys beyond N are zero
//    filled and masked by the same predicate;
//  * workgroups run longest-first (the last query tiles have the most keys), and
//    consecutive workgroup ids take different heads so that the tiles of one head land
//    on the same XCD (ids are dealt to the 8 XCDs round-robin) and share its L2.
#include "common.h"
#include "launch.h"

namespace diffattn {
namespace fwdbf16 {

constexpr int D = 64;
constexpr int DV = 128;
constexpr int BR = 128;       // query rows per workgroup
constexpr int BC = 64;        // keys per LDS stage
constexpr int NT = 256;       // threads per workgroup
constexpr int K_TILE = BC * D;      // bf16 elements, rows of 128 B
constexpr int V_TILE = DV * BC;     // bf16 elements, V^T rows of 128 B
constexpr int STAGE = 2 * K_TILE + V_TILE;

// 16-byte unit swizzle of a K row (key index within the stage). Lanes 0..7 of an MFMA
// operand read rows {0,1,2,3,8,9,10,11} (+16, +4 ...) which this maps to distinct units.
__device__ __forceinline__ int k_swz(int row) { return (row & 3) | ((row >> 1) & 4); }
// 16-byte unit swizzle of a V^T row (output channel). Distinct for 8 consecutive rows
// (operand reads) and for rows 8 apart (the transposing writes).
__device__ __forceinline__ int v_swz(int row) { return (row & 7) ^ ((row >> 3) & 7); }

// Physical key (0..31 within a 32-key sub-tile) held in score register j by lane half h.
__device__ __forceinline__ int key_of(int j, int h) { return 16 * (j >> 3) + 8 * h + (j & 7); }
// K row loaded into MFMA operand row m: swaps bits 2 and 3.
__device__ __forceinline__ int perm_row(int m) {
  return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}

struct StageRegs {
  u32x4 k1[2], k2[2], v[4];
};

__device__ __forceinline__ void load_stage(StageRegs& r, const bf16_t* __restrict__ K1,
                                           const bf16_t* __restrict__ K2,
                                           const bf16_t* __restrict__ V, int64_t k0,
                                           int64_t N, int tid) {
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int c = tid + NT * t;
    const int row = c >> 3, u = c & 7;
    const int64_t key = k0 + row;
    const u32x4 z = {0u, 0u, 0u, 0u};
    r.k1[t] = key < N ? *reinterpret_cast<const u32x4*>(K1 + key * D + u * 8) : z;
    r.k2[t] = key < N ? *reinterpret_cast<const u32x4*>(K2 + key * D + u * 8) : z;
  }
  const int kg = tid >> 4, dg = tid & 15;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int64_t key = k0 + 4 * kg + t;
    const u32x4 z = {0u, 0u, 0u, 0u};
    r.v[t] = key < N ? *reinterpret_cast<const u32x4*>(V + key * DV + dg * 8) : z;
  }
}

__device__ __forceinline__ void store_stage(const StageRegs& r, bf16_t* __restrict__ st,
                                            int tid) {
  bf16_t* K1s = st;
  bf16_t* K2s = st + K_TILE;
  bf16_t* Vt = st + 2 * K_TILE;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int c = tid + NT * t;
    const int row = c >> 3, u = c & 7;
    const int off = row * D + 8 * (u ^ k_swz(row));
    *reinterpret_cast<u32x4*>(K1s + off) = r.k1[t];
    *reinterpret_cast<u32x4*>(K2s + off) = r.k2[t];
  }
  // 4 keys x 8 channels per thread -> 8 channel rows of 4 keys each.
  const int kg = tid >> 4, dg = tid & 15;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    // channel c of keys (4kg, 4kg+1) and (4kg+2, 4kg+3), low half = earlier key
    const uint32_t x0 = r.v[0][c >> 1], x1 = r.v[1][c >> 1];
    const uint32_t x2 = r.v[2][c >> 1], x3 = r.v[3][c >> 1];
    const uint32_t lo = (c & 1) ? ((x0 >> 16) | (x1 & 0xffff0000u)) : ((x0 & 0xffffu) | (x1 << 16));
    const uint32_t hi = (c & 1) ? ((x2 >> 16) | (x3 & 0xffff0000u)) : ((x2 & 0xffffu) | (x3 << 16));
    const int row = 8 * dg + c;
    const int off = row * BC + 8 * ((kg >> 1) ^ v_swz(row)) + 4 * (kg & 1);
    u32x2 w = {lo, hi};
    *reinterpret_cast<u32x2*>(Vt + off) = w;
  }
}

__device__ __forceinline__ bf16x8 lds_read8(const bf16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ bf16x8 to_bf16x8(const f32x16& s, int base) {
  f32x8 t;
#pragma unroll
  for (int e = 0; e < 8; ++e) t[e] = s[base + e];
  return __builtin_convertvector(t, bf16x8);
}

// Online-softmax update of one map for one 32-key sub-tile. s holds raw dot products;
// c = log2(e) / sqrt(d). Returns exp2 weights in s; updates m (log2 domain, scaled), l
// (this lane's partial normaliser) and alpha (rescale factor for acc).
__device__ __forceinline__ float softmax_step(f32x16& s, float& m, float& l, float c) {
  float mx = s[0];
#pragma unroll
  for (int j = 1; j < 16; ++j) mx = fmaxf(mx, s[j]);
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  const float mn = fmaxf(m, mx * c);
  const float alpha = fast_exp2(m - mn);
  float sum = 0.f;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    s[j] = fast_exp2(fmaf(s[j], c, -mn));
    sum += s[j];
  }
  l = fmaf(l, alpha, sum);
  m = mn;
  return alpha;
}

__global__ void __launch_bounds__(NT) fwd_bf16_kernel(
    const bf16_t* __restrict__ q1, const bf16_t* __restrict__ q2,
    const bf16_t* __restrict__ k1, const bf16_t* __restrict__ k2,
    const bf16_t* __restrict__ v, const diffattn_lambda_state* __restrict__ lamst,
    const float* __restrict__ rms_w, bf16_t* __restrict__ out, float* __restrict__ sv_lse1,
    float* __restrict__ sv_lse2, float* __restrict__ sv_o1, float* __restrict__ sv_o2,
    float* __restrict__ sv_rstd, int64_t BH, int64_t H, int64_t N, int nqb, float eps) {
  __shared__ __attribute__((aligned(16))) bf16_t smem[2 * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int m = lane & 31;
  const int h = lane >> 5;

  // Longest-first over query tiles; consecutive ids walk the heads.
  const int64_t bid = blockIdx.x;
  const int64_t bh = bid % BH;
  const int qb = nqb - 1 - static_cast<int>(bid / BH);
  const int64_t q0 = static_cast<int64_t>(qb) * BR;
  const int64_t q0w = q0 + 32 * wv;

  const bf16_t* Q1 = q1 + bh * N * D;
  const bf16_t* Q2 = q2 + bh * N * D;
  const bf16_t* K1 = k1 + bh * N * D;
  const bf16_t* K2 = k2 + bh * N * D;
  const bf16_t* V = v + bh * N * DV;

  // Q^T operand: lane holds query q0w + m, channels 16 kb + 8 h .. + 7.
  bf16x8 qf1[4], qf2[4];
  {
    const int64_t q = q0w + m;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const u32x4 z = {0u, 0u, 0u, 0u};
      u32x4 a = q < N ? *reinterpret_cast<const u32x4*>(Q1 + q * D + 16 * kb + 8 * h) : z;
      u32x4 b = q < N ? *reinterpret_cast<const u32x4*>(Q2 + q * D + 16 * kb + 8 * h) : z;
      qf1[kb] = __builtin_bit_cast(bf16x8, a);
      qf2[kb] = __builtin_bit_cast(bf16x8, b);
    }
  }

  const float c = kLog2e / 8.0f;  // log2(e) / sqrt(64)
  float m1 = -INFINITY, m2 = -INFINITY, l1 = 0.f, l2 = 0.f;
  f32x16 acc1[4], acc2[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) {
#pragma unroll
    for (int j = 0; j < 16; ++j) acc1[b][j] = acc2[b][j] = 0.f;
  }

  const int64_t kend = (q0 + BR < N) ? q0 + BR : N;
  const int n_stages = static_cast<int>((kend + BC - 1) / BC);

  StageRegs regs;
  load_stage(regs, K1, K2, V, 0, N, tid);
  store_stage(regs, smem, tid);

  for (int st = 0; st < n_stages; ++st) {
    __syncthreads();
    const bool more = st + 1 < n_stages;
    if (more) load_stage(regs, K1, K2, V, static_cast<int64_t>(st + 1) * BC, N, tid);
    const bf16_t* buf = smem + (st & 1) * STAGE;
    const bf16_t* K1s = buf;
    const bf16_t* K2s = buf + K_TILE;
    const bf16_t* Vt = buf + 2 * K_TILE;
    const int64_t k0 = static_cast<int64_t>(st) * BC;

#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      const int64_t ks = k0 + 32 * sb;
      if (ks > q0w + 31) continue;  // whole sub-tile above this wave's diagonal
      f32x16 s1, s2;
#pragma unroll
      for (int j = 0; j < 16; ++j) s1[j] = s2[j] = 0.f;
      const int krow = 32 * sb + perm_row(m);
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const int off = krow * D + 8 * ((2 * kb + h) ^ k_swz(krow));
        s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_read8(K1s + off), qf1[kb], s1, 0, 0, 0);
        s2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_read8(K2s + off), qf2[kb], s2, 0, 0, 0);
      }
      if (ks + 31 > q0w) {  // diagonal sub-tile: key <= query
        const int64_t q = q0w + m;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int64_t key = ks + key_of(j, h);
          if (key > q) {
            s1[j] = -INFINITY;
            s2[j] = -INFINITY;
          }
        }
      }
      const float a1 = softmax_step(s1, m1, l1, c);
      const float a2 = softmax_step(s2, m2, l2, c);
      if (__any((a1 != 1.0f) || (a2 != 1.0f))) {
#pragma unroll
        for (int b = 0; b < 4; ++b) {
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            acc1[b][j] *= a1;
            acc2[b][j] *= a2;
          }
        }
      }
      const bf16x8 p1a = to_bf16x8(s1, 0), p1b = to_bf16x8(s1, 8);
      const bf16x8 p2a = to_bf16x8(s2, 0), p2b = to_bf16x8(s2, 8);
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int row = 32 * b + m;
        const int base = row * BC;
        const int sw = v_swz(row);
        const bf16x8 va = lds_read8(Vt + base + 8 * ((4 * sb + 0 + h) ^ sw));
        const bf16x8 vb = lds_read8(Vt + base + 8 * ((4 * sb + 2 + h) ^ sw));
        acc1[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, p1a, acc1[b], 0, 0, 0);
        acc2[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, p2a, acc2[b], 0, 0, 0);
        acc1[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vb, p1b, acc1[b], 0, 0, 0);
        acc2[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vb, p2b, acc2[b], 0, 0, 0);
      }
    }
    if (more) store_stage(regs, smem + ((st + 1) & 1) * STAGE, tid);
  }

  // Epilogue: combine the two lane halves' normalisers, form O, RMSNorm, scale, store.
  l1 += __shfl_xor(l1, 32);
  l2 += __shfl_xor(l2, 32);
  const float lam = lamst->lambda_f;
  const float g = lamst->one_minus_init_f;
  const float il1 = 1.0f / l1, il2 = 1.0f / l2;
  float ss = 0.f;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const float o1 = acc1[b][j] * il1;
      const float o2 = acc2[b][j] * il2;
      acc1[b][j] = o1;
      acc2[b][j] = o2;
      const float o = o1 - lam * o2;
      ss = fmaf(o, o, ss);
    }
  }
  ss += __shfl_xor(ss, 32);
  const float rstd = 1.0f / sqrtf(ss * (1.0f / DV) + eps);
  const int64_t q = q0w + m;
  if (q < N) {
    const int64_t hh = bh % H;
    bf16_t* Y = out + (bh * N + q) * DV;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
#pragma unroll
      for (int jg = 0; jg < 4; ++jg) {
        const int col = 32 * b + 8 * jg + 4 * h;
        float y[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float o = acc1[b][4 * jg + e] - lam * acc2[b][4 * jg + e];
          const float w = rms_w ? rms_w[hh * DV + col + e] : 1.0f;
          y[e] = g * (w * (o * rstd));
        }
        u32x2 pk = {pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
        *reinterpret_cast<u32x2*>(Y + col) = pk;
        if (sv_o1) {
          f32x4 a = {acc1[b][4 * jg], acc1[b][4 * jg + 1], acc1[b][4 * jg + 2], acc1[b][4 * jg + 3]};
          f32x4 bb = {acc2[b][4 * jg], acc2[b][4 * jg + 1], acc2[b][4 * jg + 2], acc2[b][4 * jg + 3]};
          *reinterpret_cast<f32x4*>(sv_o1 + (bh * N + q) * DV + col) = a;
          *reinterpret_cast<f32x4*>(sv_o2 + (bh * N + q) * DV + col) = bb;
        }
      }
    }
    if (sv_lse1 && h == 0) {
      // lse_k = ln(sum_j exp(S_kj)) = (m_k + log2 l_k) * ln 2, m_k in the scaled log2 domain.
      sv_lse1[bh * N + q] = (m1 + __log2f(l1)) * kLn2;
      sv_lse2[bh * N + q] = (m2 + __log2f(l2)) * kLn2;
      sv_rstd[bh * N + q] = rstd;
    }
  }
}

}  // namespace fwdbf16

hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t s) {
  using namespace fwdbf16;
  const int64_t BH = a.B * a.H;
  const int nqb = static_cast<int>((a.N + BR - 1) / BR);
  const int64_t nblk = BH * nqb;
  const diffattn_saved& sv = a.saved;
  hipLaunchKernelGGL(fwd_bf16_kernel, dim3(static_cast<unsigned>(nblk)), dim3(NT), 0, s,
                     static_cast<const bf16_t*>(a.q1), static_cast<const bf16_t*>(a.q2),
                     static_cast<const bf16_t*>(a.k1), static_cast<const bf16_t*>(a.k2),
                     static_cast<const bf16_t*>(a.v), a.lam, a.rms_weight,
                     static_cast<bf16_t*>(a.out), a.training ? sv.lse1 : nullptr,
                     a.training ? sv.lse2 : nullptr, a.training ? sv.o1 : nullptr,
                     a.training ? sv.o2 : nullptr, a.training ? sv.rstd : nullptr, BH, a.H,
                     a.N, nqb, a.eps);
  return hipGetLastError();
}

}  // namespace diffattn
