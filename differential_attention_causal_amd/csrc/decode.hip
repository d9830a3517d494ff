// Split-KV decode step for causal DiffAttn, bf16 cache, d = 64 (V and output 128 wide).
//
// One new query per (b, h) attends to every cached key 0 .. len-1 (it is the last row of
// the causal mask; intoai.pub "A Deeper Dive Into Attention Calculations"), through both
// maps of the DiffAttn equation (pt.news.hada.io "Como a atencao diferencial funciona").
// Generating a token re-reads the whole K1/K2/V cache from HBM (priorstack.com, "The
// Memory Wall: Why the KV Cache Constrains LLM Serving"), so the kernel is a streaming
// read: every cache byte is loaded exactly once, with 16-byte buffer loads marked
// non-temporal (policy bit nt: the data is not kept in the caches, which no later load
// would hit), and no LDS staging.
//
// Pass 1 (decode_split_kernel), grid = splits x (B*H): a workgroup of 4 wavefronts takes
// one split of the cache; each wavefront walks 64-key rounds of its share:
//   * scores: 8 lanes per key, each lane a 16-byte slice of the K1 and K2 rows, so one
//     wave instruction reads 8 whole rows (1 KiB contiguous); each lane's slice is dotted
//     with the query by v_dot2_f32_bf16 and the 8 partial sums are added across lanes;
//   * per map: running max m, normaliser l, and p_j = exp2(s_j log2(e)/sqrt(d) - m);
//   * values: 16 lanes per V row (16 bytes each), 4 rows per instruction; each lane keeps
//     8 output channels of both accumulators.
// The four wavefront states are merged in LDS and written as one partial
// (m, l, acc[128]) per map and split.
// Pass 2 (decode_combine_kernel), grid = B*H: exact log-sum-exp merge of the splits,
// O = acc1/l1 - lambda acc2/l2, RMSNorm over the 128 channels, x (1 - lambda_init).
#include "common.h"
#include "launch.h"

namespace diffattn {
namespace dec {

constexpr int D = 64;
constexpr int DV = 128;
constexpr int NT = 256;
constexpr int KEYS_PER_ROUND = 64;          // per wavefront
constexpr int SG = KEYS_PER_ROUND / 8;      // score groups of 8 keys (8 lanes per key)
constexpr int VI = KEYS_PER_ROUND / 4;      // value loads (16 lanes per row, 4 rows each)
constexpr int PART = 2 + DV;                // m, l, acc[DV]

__global__ void __launch_bounds__(NT, 2) decode_split_kernel(
    const bf16_t* __restrict__ q1, const bf16_t* __restrict__ q2,
    const bf16_t* __restrict__ k1, const bf16_t* __restrict__ k2,
    const bf16_t* __restrict__ v, const int32_t* __restrict__ cache_len,
    float* __restrict__ partial, int64_t H, int64_t L, int n_split, int rounds, int G) {
  __shared__ float red[4][2][PART];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int split = blockIdx.x;
  const int64_t bh = blockIdx.y;
  const int64_t b = bh / H;
  int64_t len = cache_len ? static_cast<int64_t>(cache_len[b]) : L;
  len = len < 1 ? 1 : (len > L ? L : len);
  const int64_t split_len = static_cast<int64_t>(KEYS_PER_ROUND) * 4 * rounds;
  const int64_t s0 = static_cast<int64_t>(split) * split_len;
  if (s0 >= len) return;  // the combine pass reads only splits that start below len

  // Cache rows through buffer resources bounded at len rows: keys at or beyond len read
  // as zero, and each load needs only a 32-bit lane offset plus the round's scalar offset.
  constexpr int kBufFlags = 0x00020000;  // raw 32-bit buffer, no swizzle
  // Cache head of this query head (grouped-query attention: G query heads per cache head).
  const int64_t kvh = b * (H / G) + (bh - b * H) / G;
  const __amdgpu_buffer_rsrc_t rk1 = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(k1 + kvh * L * D), 0, static_cast<int>(len * D * 2), kBufFlags);
  const __amdgpu_buffer_rsrc_t rk2 = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(k2 + kvh * L * D), 0, static_cast<int>(len * D * 2), kBufFlags);
  const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(v + kvh * L * DV), 0, static_cast<int>(len * DV * 2), kBufFlags);

  // Score lanes: key r = lane / 8 of each group of 8, channel slice c = lane % 8.
  const int r = lane >> 3, c = lane & 7;
  // This lane's 8 query channels of each map, as bf16 pairs for v_dot2 (each product of
  // two bf16 values is exact in float32; the sums are float32).
  // (Pairs are built element by element from bf16x8 vectors: bit-casting 32-bit lanes of
  // a u32x4 to bf16x2 here was compiled to feed the same pair to every dot product.)
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x8 qa = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(q1 + bh * D + 8 * c));
  const bf16x8 qb = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(q2 + bh * D + 8 * c));
  // Value lanes: channel slice e = lane % 16 (channels 8e..8e+7), key phase f = lane / 16.
  const int e = lane & 15, f = lane >> 4;
  const int ko = r * D * 2 + 16 * c;    // byte offset of this lane's K slice in a round
  const int vo = f * DV * 2 + 16 * e;   // byte offset of this lane's V slice in a round

  const float cs = kLog2e / 8.0f;  // log2(e) / sqrt(64)
  float m1 = -INFINITY, m2 = -INFINITY, l1 = 0.f, l2 = 0.f;
  float acc1[8], acc2[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) acc1[t] = acc2[t] = 0.f;

#pragma clang loop unroll(disable)
  for (int rd = 0; rd < rounds; ++rd) {
    const int64_t kb = s0 + (static_cast<int64_t>(wv) * rounds + rd) * KEYS_PER_ROUND;
    if (kb >= len) break;
    const int kbs = __builtin_amdgcn_readfirstlane(static_cast<int>(kb));
    // ---- scores of the keys kb + 8 g + r
    u32x4 kx[SG], ky[SG];
#pragma unroll
    for (int g = 0; g < SG; ++g) {
      kx[g] = __builtin_amdgcn_raw_buffer_load_b128(rk1, ko + g * 8 * D * 2, kbs * D * 2, 2);
      ky[g] = __builtin_amdgcn_raw_buffer_load_b128(rk2, ko + g * 8 * D * 2, kbs * D * 2, 2);
    }
    u32x4 vv[VI];
#pragma unroll
    for (int i = 0; i < VI; ++i)
      vv[i] = __builtin_amdgcn_raw_buffer_load_b128(rv, vo + i * 4 * DV * 2, kbs * DV * 2, 2);
    float s1[SG], s2[SG];
#pragma unroll
    for (int g = 0; g < SG; ++g) {
      float d1 = 0.f, d2 = 0.f;
      const bf16x8 ka = __builtin_bit_cast(bf16x8, kx[g]), kc = __builtin_bit_cast(bf16x8, ky[g]);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const bf16x2 q1p = {qa[2 * t], qa[2 * t + 1]}, k1p = {ka[2 * t], ka[2 * t + 1]};
        const bf16x2 q2p = {qb[2 * t], qb[2 * t + 1]}, k2p = {kc[2 * t], kc[2 * t + 1]};
        d1 = __builtin_amdgcn_fdot2_f32_bf16(q1p, k1p, d1, false);
        d2 = __builtin_amdgcn_fdot2_f32_bf16(q2p, k2p, d2, false);
      }
#pragma unroll
      for (int o = 1; o < 8; o <<= 1) {
        d1 += __shfl_xor(d1, o);
        d2 += __shfl_xor(d2, o);
      }
      const bool ok = kb + 8 * g + r < len;
      s1[g] = ok ? d1 * cs : -INFINITY;
      s2[g] = ok ? d2 * cs : -INFINITY;
    }
    float mx1 = s1[0], mx2 = s2[0];
#pragma unroll
    for (int g = 1; g < SG; ++g) {
      mx1 = fmaxf(mx1, s1[g]);
      mx2 = fmaxf(mx2, s2[g]);
    }
#pragma unroll
    for (int o = 8; o < 64; o <<= 1) {
      mx1 = fmaxf(mx1, __shfl_xor(mx1, o));
      mx2 = fmaxf(mx2, __shfl_xor(mx2, o));
    }
    const float mn1 = fmaxf(m1, mx1), mn2 = fmaxf(m2, mx2);
    const float al1 = fast_exp2(m1 - mn1), al2 = fast_exp2(m2 - mn2);
    float p1[SG], p2[SG], sum1 = 0.f, sum2 = 0.f;
#pragma unroll
    for (int g = 0; g < SG; ++g) {
      p1[g] = fast_exp2(s1[g] - mn1);
      p2[g] = fast_exp2(s2[g] - mn2);
      sum1 += p1[g];
      sum2 += p2[g];
    }
#pragma unroll
    for (int o = 8; o < 64; o <<= 1) {
      sum1 += __shfl_xor(sum1, o);
      sum2 += __shfl_xor(sum2, o);
    }
    l1 = fmaf(l1, al1, sum1);
    l2 = fmaf(l2, al2, sum2);
    m1 = mn1;
    m2 = mn2;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      acc1[t] *= al1;
      acc2[t] *= al2;
    }
    // ---- values: key 4 i + f, whose weight sits in register i/2 of lanes 8 * (key % 8)
#pragma unroll
    for (int i = 0; i < VI; ++i) {
      const int src = 32 * (i & 1) + 8 * f;
      const float w1 = __shfl(p1[i >> 1], src);
      const float w2 = __shfl(p2[i >> 1], src);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const float lo = __uint_as_float(vv[i][t] << 16);
        const float hi = __uint_as_float(vv[i][t] & 0xffff0000u);
        acc1[2 * t] = fmaf(w1, lo, acc1[2 * t]);
        acc1[2 * t + 1] = fmaf(w1, hi, acc1[2 * t + 1]);
        acc2[2 * t] = fmaf(w2, lo, acc2[2 * t]);
        acc2[2 * t + 1] = fmaf(w2, hi, acc2[2 * t + 1]);
      }
    }
  }
  // Sum the four key phases (lanes e, e+16, e+32, e+48 hold the same channels).
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    acc1[t] += __shfl_xor(acc1[t], 16);
    acc1[t] += __shfl_xor(acc1[t], 32);
    acc2[t] += __shfl_xor(acc2[t], 16);
    acc2[t] += __shfl_xor(acc2[t], 32);
  }
  if (lane == 0) {
    red[wv][0][0] = m1;
    red[wv][0][1] = l1;
    red[wv][1][0] = m2;
    red[wv][1][1] = l2;
  }
  if (f == 0) {
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      red[wv][0][2 + 8 * e + t] = acc1[t];
      red[wv][1][2 + 8 * e + t] = acc2[t];
    }
  }
  __syncthreads();
  // Merge the 4 wavefront states: thread = (map, channel). Waves with no valid key have
  // m = -inf and weight 0; wave 0 always has a valid key.
  float* out = partial + (bh * n_split + split) * 2 * PART;
  if (tid < 2 * DV) {
    const int mp = tid / DV, ch = tid % DV;
    float M = red[0][mp][0];
#pragma unroll
    for (int w = 1; w < 4; ++w) M = fmaxf(M, red[w][mp][0]);
    float A = 0.f, S = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float sc = fast_exp2(red[w][mp][0] - M);
      A = fmaf(red[w][mp][2 + ch], sc, A);
      S = fmaf(red[w][mp][1], sc, S);
    }
    out[mp * PART + 2 + ch] = A;
    if (ch == 0) {
      out[mp * PART + 0] = M;
      out[mp * PART + 1] = S;
    }
  }
}

// Grouped-query decode: GW query heads that share one cache head (GW divides the group
// size G) are served by one workgroup, so each cache byte is read once for all of them
// instead of once per query head. Same structure as decode_split_kernel, with every
// per-head quantity (queries, scores, weights, m, l, accumulators) held GW times over
// and 32-key rounds (to keep those in registers). Writes the same per-(b, h, split)
// partials, so decode_combine_kernel finishes both.
// Cross-lane reductions without the LDS crossbar. Score lanes come in groups of 8 (lanes
// 8 r .. 8 r + 7, one key per group). sum8 adds over a group (DPP: quad swaps 1 and 2,
// then the mirror inside 8 lanes); the *_groups forms combine the 8 groups of a
// wavefront, whose values are uniform within each group (the mirror inside 16 lanes
// pairs groups 2k and 2k + 1, then rows are exchanged by the permlane swaps).
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float sum8(float x) {
  x += dpp<0xB1>(x);    // quad_perm [1, 0, 3, 2]
  x += dpp<0x4E>(x);    // quad_perm [2, 3, 0, 1]
  x += dpp<0x141>(x);   // row_half_mirror
  return x;
}
template <bool MAX>
__device__ __forceinline__ float combine(float a, float b) { return MAX ? fmaxf(a, b) : a + b; }
// The swaps exchange rows between two registers that both start as x: afterwards each
// lane holds its own row's value in one and the partner row's in the other (rows of 16
// lanes paired 0-1, 2-3 by the 16-lane swap; halves of the wavefront by the 32-lane
// swap). Issued as assembly: the compiler's model of the swap builtins folded the two
// results into one. The s_nop wait states cover the vector-ALU write before the swap and
// the reads after it.
template <bool MAX>
__device__ __forceinline__ float across_groups(float x) {
  x = combine<MAX>(x, dpp<0x140>(x));   // row_mirror
  uint32_t a = __builtin_bit_cast(uint32_t, x), b = a;
  asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
  x = combine<MAX>(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b));
  a = __builtin_bit_cast(uint32_t, x);
  b = a;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
  return combine<MAX>(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b));
}

template <int GW>
__global__ void __launch_bounds__(NT, 2) decode_group_kernel(
    const bf16_t* __restrict__ q1, const bf16_t* __restrict__ q2,
    const bf16_t* __restrict__ k1, const bf16_t* __restrict__ k2,
    const bf16_t* __restrict__ v, const int32_t* __restrict__ cache_len,
    float* __restrict__ partial, int64_t H, int64_t L, int n_split, int rounds, int G) {
  constexpr int KPR = 32;                 // keys per wavefront round
  constexpr int SGG = KPR / 8;            // score groups of 8 keys
  constexpr int VIG = KPR / 4;            // value loads of 4 rows
  __shared__ float red[4][2 * GW][PART];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int split = blockIdx.x;
  const int64_t h0 = static_cast<int64_t>(blockIdx.y) * GW;   // first query head (b H + h)
  const int64_t b = h0 / H;
  int64_t len = cache_len ? static_cast<int64_t>(cache_len[b]) : L;
  len = len < 1 ? 1 : (len > L ? L : len);
  const int64_t split_len = static_cast<int64_t>(KPR) * 4 * rounds;
  const int64_t s0 = static_cast<int64_t>(split) * split_len;
  if (s0 >= len) return;

  const int64_t kvh = b * (H / G) + (h0 - b * H) / G;   // the shared cache head
  constexpr int kBufFlags = 0x00020000;
  const __amdgpu_buffer_rsrc_t rk1 = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(k1 + kvh * L * D), 0, static_cast<int>(len * D * 2), kBufFlags);
  const __amdgpu_buffer_rsrc_t rk2 = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(k2 + kvh * L * D), 0, static_cast<int>(len * D * 2), kBufFlags);
  const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(v + kvh * L * DV), 0, static_cast<int>(len * DV * 2), kBufFlags);

  const int r = lane >> 3, c = lane & 7;
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x8 qa[GW], qb[GW];
#pragma unroll
  for (int g = 0; g < GW; ++g) {
    qa[g] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(q1 + (h0 + g) * D + 8 * c));
    qb[g] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(q2 + (h0 + g) * D + 8 * c));
  }
  const int e = lane & 15, f = lane >> 4;
  const int ko = r * D * 2 + 16 * c;
  const int vo = f * DV * 2 + 16 * e;

  const float cs = kLog2e / 8.0f;
  float m1[GW], m2[GW], l1[GW], l2[GW], acc1[GW][8], acc2[GW][8];
#pragma unroll
  for (int g = 0; g < GW; ++g) {
    m1[g] = m2[g] = -INFINITY;
    l1[g] = l2[g] = 0.f;
#pragma unroll
    for (int t = 0; t < 8; ++t) acc1[g][t] = acc2[g][t] = 0.f;
  }

#pragma clang loop unroll(disable)
  for (int rd = 0; rd < rounds; ++rd) {
    const int64_t kb = s0 + (static_cast<int64_t>(wv) * rounds + rd) * KPR;
    if (kb >= len) break;
    const int kbs = __builtin_amdgcn_readfirstlane(static_cast<int>(kb));
    u32x4 kx[SGG], ky[SGG], vv[VIG];
#pragma unroll
    for (int sg = 0; sg < SGG; ++sg) {
      kx[sg] = __builtin_amdgcn_raw_buffer_load_b128(rk1, ko + sg * 8 * D * 2, kbs * D * 2, 2);
      ky[sg] = __builtin_amdgcn_raw_buffer_load_b128(rk2, ko + sg * 8 * D * 2, kbs * D * 2, 2);
    }
#pragma unroll
    for (int i = 0; i < VIG; ++i)
      vv[i] = __builtin_amdgcn_raw_buffer_load_b128(rv, vo + i * 4 * DV * 2, kbs * DV * 2, 2);
#pragma unroll
    for (int g = 0; g < GW; ++g) {
      float s1[SGG], s2[SGG];
#pragma unroll
      for (int sg = 0; sg < SGG; ++sg) {
        float d1 = 0.f, d2 = 0.f;
        const bf16x8 ka = __builtin_bit_cast(bf16x8, kx[sg]), kc = __builtin_bit_cast(bf16x8, ky[sg]);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const bf16x2 q1p = {qa[g][2 * t], qa[g][2 * t + 1]}, k1p = {ka[2 * t], ka[2 * t + 1]};
          const bf16x2 q2p = {qb[g][2 * t], qb[g][2 * t + 1]}, k2p = {kc[2 * t], kc[2 * t + 1]};
          d1 = __builtin_amdgcn_fdot2_f32_bf16(q1p, k1p, d1, false);
          d2 = __builtin_amdgcn_fdot2_f32_bf16(q2p, k2p, d2, false);
        }
        d1 = sum8(d1);
        d2 = sum8(d2);
        const bool ok = kb + 8 * sg + r < len;
        s1[sg] = ok ? d1 * cs : -INFINITY;
        s2[sg] = ok ? d2 * cs : -INFINITY;
      }
      float mx1 = s1[0], mx2 = s2[0];
#pragma unroll
      for (int sg = 1; sg < SGG; ++sg) {
        mx1 = fmaxf(mx1, s1[sg]);
        mx2 = fmaxf(mx2, s2[sg]);
      }
      mx1 = across_groups<true>(mx1);
      mx2 = across_groups<true>(mx2);
      const float mn1 = fmaxf(m1[g], mx1), mn2 = fmaxf(m2[g], mx2);
      const float al1 = fast_exp2(m1[g] - mn1), al2 = fast_exp2(m2[g] - mn2);
      float sum1 = 0.f, sum2 = 0.f;
#pragma unroll
      for (int sg = 0; sg < SGG; ++sg) {
        s1[sg] = fast_exp2(s1[sg] - mn1);   // now the weights p
        s2[sg] = fast_exp2(s2[sg] - mn2);
        sum1 += s1[sg];
        sum2 += s2[sg];
      }
      sum1 = across_groups<false>(sum1);
      sum2 = across_groups<false>(sum2);
      l1[g] = fmaf(l1[g], al1, sum1);
      l2[g] = fmaf(l2[g], al2, sum2);
      m1[g] = mn1;
      m2[g] = mn2;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        acc1[g][t] *= al1;
        acc2[g][t] *= al2;
      }
      // values: key 4 i + f, whose weight sits in register i / 2 of lanes 8 (key % 8)
#pragma unroll
      for (int i = 0; i < VIG; ++i) {
        const int src = 32 * (i & 1) + 8 * f;
        const float w1 = __shfl(s1[i >> 1], src);
        const float w2 = __shfl(s2[i >> 1], src);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const float lo = __uint_as_float(vv[i][t] << 16);
          const float hi = __uint_as_float(vv[i][t] & 0xffff0000u);
          acc1[g][2 * t] = fmaf(w1, lo, acc1[g][2 * t]);
          acc1[g][2 * t + 1] = fmaf(w1, hi, acc1[g][2 * t + 1]);
          acc2[g][2 * t] = fmaf(w2, lo, acc2[g][2 * t]);
          acc2[g][2 * t + 1] = fmaf(w2, hi, acc2[g][2 * t + 1]);
        }
      }
    }
  }
#pragma unroll
  for (int g = 0; g < GW; ++g) {
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      acc1[g][t] += __shfl_xor(acc1[g][t], 16);
      acc1[g][t] += __shfl_xor(acc1[g][t], 32);
      acc2[g][t] += __shfl_xor(acc2[g][t], 16);
      acc2[g][t] += __shfl_xor(acc2[g][t], 32);
    }
    if (lane == 0) {
      red[wv][2 * g][0] = m1[g];
      red[wv][2 * g][1] = l1[g];
      red[wv][2 * g + 1][0] = m2[g];
      red[wv][2 * g + 1][1] = l2[g];
    }
    if (f == 0) {
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        red[wv][2 * g][2 + 8 * e + t] = acc1[g][t];
        red[wv][2 * g + 1][2 + 8 * e + t] = acc2[g][t];
      }
    }
  }
  __syncthreads();
  // Merge the 4 wavefront states per head: thread = (map, channel), looping over heads.
  if (tid < 2 * DV) {
    const int mp = tid / DV, ch = tid % DV;
#pragma unroll
    for (int g = 0; g < GW; ++g) {
      float* out = partial + ((h0 + g) * n_split + split) * 2 * PART;
      const int row = 2 * g + mp;
      float M = red[0][row][0];
#pragma unroll
      for (int w = 1; w < 4; ++w) M = fmaxf(M, red[w][row][0]);
      float A = 0.f, S = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float sc = fast_exp2(red[w][row][0] - M);
        A = fmaf(red[w][row][2 + ch], sc, A);
        S = fmaf(red[w][row][1], sc, S);
      }
      out[mp * PART + 2 + ch] = A;
      if (ch == 0) {
        out[mp * PART + 0] = M;
        out[mp * PART + 1] = S;
      }
    }
  }
}

// One thread per map and channel (map k = threadIdx.x / 128). The partials of the
// splits are read in batches of CB independent loads, so the merge waits for memory once
// when there are at most CB splits and a few times per map otherwise; the order of the
// arithmetic (maximum over all splits first, then the rescaled sums in split order) does
// not depend on the batching.
constexpr int CB = 16;
__global__ void __launch_bounds__(2 * DV) decode_combine_kernel(
    const float* __restrict__ partial, const int32_t* __restrict__ cache_len,
    const diffattn_lambda_state* __restrict__ lamst, const float* __restrict__ rms_w,
    bf16_t* __restrict__ out, int64_t H, int64_t L, int n_split, int64_t split_len,
    float eps) {
  __shared__ float o2[DV];
  __shared__ float wsum[2];
  const int mp = threadIdx.x >> 7;
  const int ch = threadIdx.x & (DV - 1);
  const int64_t bh = blockIdx.x;
  const int64_t b = bh / H;
  int64_t len = cache_len ? static_cast<int64_t>(cache_len[b]) : L;
  len = len < 1 ? 1 : (len > L ? L : len);
  const int nv = static_cast<int>((len + split_len - 1) / split_len);
  const float* P = partial + bh * n_split * 2 * PART + mp * PART;
  float M = -INFINITY, A = 0.f, S = 0.f;
  if (nv <= CB) {
    float m[CB], l[CB], a[CB];
#pragma unroll
    for (int i = 0; i < CB; ++i) {
      const float* ps = P + (i < nv ? i : 0) * 2 * PART;
      m[i] = ps[0];
      l[i] = ps[1];
      a[i] = ps[2 + ch];
    }
#pragma unroll
    for (int i = 0; i < CB; ++i) M = fmaxf(M, m[i]);
#pragma unroll
    for (int i = 0; i < CB; ++i) {
      if (i < nv) {
        const float sc = fast_exp2(m[i] - M);
        S = fmaf(l[i], sc, S);
        A = fmaf(a[i], sc, A);
      }
    }
  } else {
    for (int s0 = 0; s0 < nv; s0 += CB) {
      float m[CB];
#pragma unroll
      for (int i = 0; i < CB; ++i) m[i] = P[(s0 + i < nv ? s0 + i : s0) * 2 * PART];
#pragma unroll
      for (int i = 0; i < CB; ++i) M = fmaxf(M, m[i]);
    }
    for (int s0 = 0; s0 < nv; s0 += CB) {
      float m[CB], l[CB], a[CB];
#pragma unroll
      for (int i = 0; i < CB; ++i) {
        const float* ps = P + (s0 + i < nv ? s0 + i : s0) * 2 * PART;
        m[i] = ps[0];
        l[i] = ps[1];
        a[i] = ps[2 + ch];
      }
#pragma unroll
      for (int i = 0; i < CB; ++i) {
        if (s0 + i < nv) {
          const float sc = fast_exp2(m[i] - M);
          S = fmaf(l[i], sc, S);
          A = fmaf(a[i], sc, A);
        }
      }
    }
  }
  const float o = A / S;
  if (mp == 1) o2[ch] = o;
  __syncthreads();
  // Map 1's wavefronts stay to the last barrier but do no more work.
  const float lam = lamst->lambda_f;
  const float y = o - lam * o2[ch];
  float ss = wave_sum(y * y);
  if (mp == 0 && (ch & 63) == 0) wsum[ch >> 6] = ss;
  __syncthreads();
  if (mp == 1) return;
  ss = wsum[0] + wsum[1];
  const float rstd = 1.0f / sqrtf(ss * (1.0f / DV) + eps);
  const float w = rms_w ? rms_w[(bh % H) * DV + ch] : 1.0f;
  out[bh * DV + ch] = f32_to_bf16(lamst->one_minus_init_f * (w * (y * rstd)));
}

}  // namespace dec

void decode_split_geometry(int64_t B, int64_t H, int64_t L, int* n_split, int* split_len) {
  // Rounds of 64 keys per wavefront, at most 2 per wavefront: many small workgroups, so
  // that the last partial wave of workgroups leaves little of the chip idle.
  const int64_t BH = B * H;
  int rounds = 2;
  while (rounds > 1) {
    const int64_t sl = static_cast<int64_t>(dec::KEYS_PER_ROUND) * 4 * rounds;
    if (BH * ((L + sl - 1) / sl) >= 4096) break;
    rounds >>= 1;
  }
  const int64_t sl = static_cast<int64_t>(dec::KEYS_PER_ROUND) * 4 * rounds;
  *split_len = static_cast<int>(sl);
  *n_split = static_cast<int>((L + sl - 1) / sl);
}

hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t s) {
  using namespace dec;
  const int rounds = a.split_len / (KEYS_PER_ROUND * 4);
  const int64_t BH = a.B * a.H;
  // Query heads served per workgroup: the largest of 4, 3, 2 dividing the group size.
  const int gw = a.G % 4 == 0 ? 4 : (a.G % 3 == 0 ? 3 : (a.G % 2 == 0 ? 2 : 1));
  auto group = [&](auto kern, int heads_per_wg) {
    // 32-key rounds: twice as many per split as the 64-key rounds of the single-head kernel.
    hipLaunchKernelGGL(kern, dim3(a.n_split, static_cast<unsigned>(BH / heads_per_wg)),
                       dim3(NT), 0, s, static_cast<const bf16_t*>(a.q1),
                       static_cast<const bf16_t*>(a.q2), static_cast<const bf16_t*>(a.k1),
                       static_cast<const bf16_t*>(a.k2), static_cast<const bf16_t*>(a.v),
                       a.cache_len, a.partial, a.H, a.L, a.n_split, 2 * rounds, a.G);
  };
  if (gw == 4) {
    group(decode_group_kernel<4>, 4);
  } else if (gw == 3) {
    group(decode_group_kernel<3>, 3);
  } else if (gw == 2) {
    group(decode_group_kernel<2>, 2);
  } else {
    hipLaunchKernelGGL(decode_split_kernel, dim3(a.n_split, static_cast<unsigned>(BH)),
                       dim3(NT), 0, s, static_cast<const bf16_t*>(a.q1),
                       static_cast<const bf16_t*>(a.q2), static_cast<const bf16_t*>(a.k1),
                       static_cast<const bf16_t*>(a.k2), static_cast<const bf16_t*>(a.v),
                       a.cache_len, a.partial, a.H, a.L, a.n_split, rounds, a.G);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_combine_kernel, dim3(static_cast<unsigned>(BH)), dim3(2 * DV), 0, s,
                     a.partial, a.cache_len, a.lam, a.rms_weight, static_cast<bf16_t*>(a.out),
                     a.H, a.L, a.n_split, static_cast<int64_t>(a.split_len), a.eps);
  return hipGetLastError();
}

}  // namespace diffattn
