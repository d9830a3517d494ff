// Split-KV decode step for causal DiffAttn, bf16 cache, d = 64 (V and output 128 wide).
//
// One new query per (b, h) attends to every cached key 0 .. len-1 (it is the last row of
// the causal mask; intoai.pub "A Deeper Dive Into Attention Calculations"), through both
// maps of the DiffAttn equation (pt.news.hada.io "Como a atencao diferencial funciona").
// Generating a token re-reads the whole K1/K2/V cache from HBM (priorstack.com, "The
// Memory Wall: Why the KV Cache Constrains LLM Serving"), so the kernel is a streaming
// read: every cache byte is loaded once per step, for all the query heads that share it,
// with loads marked non-temporal (policy bit nt: no later load would hit the caches).
//
// Pass 1 (decode_mfma_kernel), grid = splits x (query-head groups): a workgroup of 4
// wavefronts takes one split of one cache head for up to 32 of the query heads that
// share it (one, without grouped-query attention), on the matrix cores; it writes one
// partial (m, l, acc[128]) per query head, map and split.
// Pass 2 (decode_combine_kernel), grid = B*H: exact log-sum-exp merge of the splits,
// O = acc1/l1 - lambda acc2/l2, RMSNorm over the 128 channels, x (1 - lambda_init).
#include "common.h"
#include "launch.h"

namespace diffattn {
namespace dec {

constexpr int D = 64;
constexpr int DV = 128;
constexpr int NT = 256;
constexpr int PART = 2 + DV;                // m, l, acc[DV]

// Decode on the matrix cores. The gq query heads that share one cache head (gq = 1
// without grouped-query attention) are the columns of the B operand of v_mfma_f32_32x32x16_bf16 (32 columns, the
// first gq real, the rest zero), so one pass over a 32-key round of the cache serves all
// of them:
//   * S^T = K Q^T per map: 32 keys x 32 query columns. Operand row m holds key
//     perm_row(m) (bits 2 and 3 of the key swapped), so the 16 scores a lane holds for its
//     column, packed to bf16, are directly the B operand of the value product: register j
//     holds key key_of(j, h).
//   * weights p = exp2(s log2(e) / 8 - m) per map, with a per-column reference m: the
//     exact maximum of the wavefront's first round, moved (rescaling that column's
//     accumulator and normaliser) only when a later round's maximum passes it by 2^20,
//     so weights stay below 2^20.
//   * O^T += V^T P^T per map (4 regions of 32 channels, 2 steps of 16 keys), V^T read with
//     ds_read_b64_tr_b16.
// The cache streams from HBM into LDS through buffer loads with LDS as the destination:
// each wavefront has two 16 KiB buffers (a round's K1, K2 and V rows) and keeps two
// rounds in flight while it computes a third from registers (a round's operands move to
// registers first, which frees its buffer for the round after next). The loads are
// assembly and their waits explicit, so the compiler neither orders LDS reads behind
// them nor waits for later rounds. No barrier: each wavefront reads only its own
// buffers. The four wavefronts' states are merged in LDS and written as per-(b, h, split)
// partials for decode_combine_kernel.
namespace gq {
constexpr int KPR = 32;                 // keys per wavefront round
constexpr int KT = KPR * 128;           // a round's K1 (or K2) rows: [32][128 B]
constexpr int VREG = KPR * 64;          // a round's V rows, one 32-channel region: [32][64 B]
constexpr int BUF = 2 * KT + 4 * VREG;  // K1 | K2 | V, 16 KiB
constexpr int WAVE_LDS = 2 * BUF;       // two buffers per wavefront
constexpr int DMA_PER_ROUND = 16;       // 1 KiB loads: 4 K1, 4 K2, 8 V
static_assert(DMA_PER_ROUND == 16, "the loop's vmcnt waits count 16 loads per round");
constexpr float kMove = 20.0f;          // a column's reference moves past 2^20 growth
// K rows: 16-byte unit u of row r stored at u ^ k_swz(r), so the 32 operand rows read by
// one ds_read_b128 spread over the banks; V rows: chunk c of row r at c ^ v_swz(r).
__device__ __forceinline__ int k_swz(int row) {
  return ((row ^ (row >> 2)) & 1) | (row & 2) | ((row >> 1) & 4);
}
__device__ __forceinline__ int v_swz(int row) { return 2 * ((row >> 1) & 1); }
__device__ __forceinline__ int perm_row(int m) { return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1); }
__device__ __forceinline__ int key_of(int j, int h) { return 16 * (j >> 3) + 8 * h + (j & 7); }
__device__ __forceinline__ int chan_of(int j, int h) { return (j & 3) + 4 * h + 8 * (j >> 2); }
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef char __attribute__((address_space(3))) lds_char;
__device__ __forceinline__ u32x2 ds_read_tr16(const lds_char* p) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)p);
  return __builtin_bit_cast(u32x2, v);
}
__device__ __forceinline__ u32x4 ds_read_b128(const lds_char* p) {
  return *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(p);
}
// 16 bytes per lane from the buffer (offset voff) into LDS at m0 + 16 lane.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rs, uint32_t m0, int voff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen nt lds"
               :
               : "s"(m0), "v"(voff), "s"(rs));
}
__device__ __forceinline__ float max_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
// An accumulation register scaled in place through one vector register (the rare
// reference move), so the accumulators never leave the accumulation registers.
__device__ __forceinline__ float scale_acc(float x, float a) {
  float t;
  asm volatile("v_accvgpr_read_b32 %1, %0\n\tv_mul_f32 %1, %1, %2\n\tv_accvgpr_write_b32 %0, %1"
               : "+a"(x), "=&v"(t)
               : "v"(a));
  return x;
}
__device__ __forceinline__ void acc_pin(f32x16 (&a)[4]) {
  asm volatile("" : "+a"(a[0]), "+a"(a[1]), "+a"(a[2]), "+a"(a[3]));
}
}  // namespace gq

__global__ void __launch_bounds__(NT, 1) decode_mfma_kernel(
    const bf16_t* __restrict__ q1, const bf16_t* __restrict__ q2,
    const bf16_t* __restrict__ k1, const bf16_t* __restrict__ k2,
    const bf16_t* __restrict__ v, const int32_t* __restrict__ cache_len,
    float* __restrict__ partial, int64_t H, int64_t L, int n_split, int rounds, int G, int gq) {
  using namespace gq;
  extern __shared__ __attribute__((aligned(16))) char lds_raw[];
  lds_char* lds = (lds_char*)lds_raw;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31, h = lane >> 5;
  const int split = blockIdx.x;
  const int64_t h0 = static_cast<int64_t>(blockIdx.y) * gq;   // first query head (b H + h)
  const int64_t b = h0 / H;
  int64_t len = cache_len ? static_cast<int64_t>(cache_len[b]) : L;
  len = len < 1 ? 1 : (len > L ? L : len);
  const int64_t split_len = static_cast<int64_t>(KPR) * 4 * rounds;
  const int64_t s0 = static_cast<int64_t>(split) * split_len;
  if (s0 >= len) return;

  // Cache rows through buffer resources bounded at len rows: keys at or beyond len read
  // as zero (and are masked).
  const int64_t kvh = b * (H / G) + (h0 - b * H) / G;   // the shared cache head
  constexpr int kBufFlags = 0x00020000;
  const __amdgpu_buffer_rsrc_t rk1 = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(k1 + kvh * L * D), 0, static_cast<int>(len * D * 2), kBufFlags);
  const __amdgpu_buffer_rsrc_t rk2 = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(k2 + kvh * L * D), 0, static_cast<int>(len * D * 2), kBufFlags);
  const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(v + kvh * L * DV), 0, static_cast<int>(len * DV * 2), kBufFlags);

  // Query columns: lane (n, h) holds channels 16 kb + 8 h .. + 7 of query head h0 + n.
  bf16x8 qa[4], qb[4];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    u32x4 x = {0u, 0u, 0u, 0u}, y = {0u, 0u, 0u, 0u};
    if (n < gq) {
      x = *reinterpret_cast<const u32x4*>(q1 + (h0 + n) * D + 16 * kb + 8 * h);
      y = *reinterpret_cast<const u32x4*>(q2 + (h0 + n) * D + 16 * kb + 8 * h);
    }
    qa[kb] = __builtin_bit_cast(bf16x8, x);
    qb[kb] = __builtin_bit_cast(bf16x8, y);
  }
  // The query loads complete here, so the compiler's own waits for them stay out of the
  // loop, where a vmcnt wait would also stall on the cache loads in flight.
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) asm volatile("" : "+v"(qa[kb]), "+v"(qb[kb]));
  // DMA source offsets within a round (key rows from its first key): K block i holds rows
  // 8 i .. 8 i + 7 (lane: row 8 i + lane / 8, unit lane % 8), V block (region rg, half i)
  // rows 16 i .. 16 i + 15 of region rg (lane: row 16 i + lane / 4, chunk lane % 4).
  int kso[4], vso[2];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 8 * i + (lane >> 3), pu = lane & 7;
    kso[i] = row * (D * 2) + 16 * (pu ^ k_swz(row));
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int row = 16 * i + (lane >> 2), pc = lane & 3;
    vso[i] = row * (DV * 2) + 16 * (pc ^ v_swz(row));
  }
  // Operand reads: K row perm_row(n), unit (2 kb + h) ^ k_swz; V^T transposing reads.
  int kra;
  {
    const int kr = perm_row(n);
    kra = kr * 128;
  }
  const int ks = k_swz(perm_row(n));
  int vta;
  {
    const int g16 = lane >> 4, jj = (lane >> 2) & 3, a = lane & 3;
    const int row = 8 * (g16 >> 1) + jj;
    const int cp = 2 * (g16 & 1) + (a >> 1);
    vta = row * 64 + 16 * (cp ^ v_swz(row)) + 8 * (a & 1);
  }
  const uint32_t wbase = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds)) + wv * WAVE_LDS;
  lds_char* wbuf = lds + wv * WAVE_LDS;

  // The 16 loads of the round that starts at key kb into buffer c.
  auto issue = [&](int64_t kb, int c) __attribute__((always_inline)) {
    const int kbi = static_cast<int>(kb);
    const uint32_t dst = wbase + c * BUF;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      dma16(rk1, dst + 1024 * i, kbi * (D * 2) + kso[i]);
      dma16(rk2, dst + KT + 1024 * i, kbi * (D * 2) + kso[i]);
    }
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
        dma16(rv, dst + 2 * KT + VREG * rg + 1024 * i, kbi * (DV * 2) + vso[i] + 64 * rg);
    }
  };

  const float cs = kLog2e / 8.0f;
  f32x16 acc1[4], acc2[4];
#pragma unroll
  for (int rg = 0; rg < 4; ++rg) {
#pragma unroll
    for (int j = 0; j < 16; ++j) acc1[rg][j] = acc2[rg][j] = 0.f;
  }
  float m1 = -INFINITY, m2 = -INFINITY, l1 = 0.f, l2 = 0.f;

  const int64_t kfirst = s0 + static_cast<int64_t>(wv) * rounds * KPR;
  int nr = 0;   // rounds of this wavefront that start below len
  for (int rd = 0; rd < rounds; ++rd)
    if (kfirst + static_cast<int64_t>(rd) * KPR < len) nr = rd + 1;
  if (nr > 0) issue(kfirst, 0);
  if (nr > 1) issue(kfirst + KPR, 1);

  // One round of map k: scores, weights (with the rare move of a column's reference) and
  // the packed B operands of the value product.
  auto softmax = [&](f32x16 S, int64_t kb, bool first, float& m, float& l, f32x16 (&acc)[4],
                     bf16x8& pa, bf16x8& pb) __attribute__((always_inline)) {
    if (kb + KPR > len) {
      const int kl = static_cast<int>(len - kb);   // keys of this round below len
#pragma unroll
      for (int j = 0; j < 16; ++j)
        if (key_of(j, h) >= kl) S[j] = -INFINITY;
    }
    float mx = S[0];
#pragma unroll
    for (int j = 1; j < 16; ++j) mx = fmaxf(mx, S[j]);
    mx = max_halves(mx) * cs;
    if (first) {
      m = mx;
    } else {
      const bool mv = mx > m + kMove;
      if (__builtin_expect(__any(mv), 0)) {
        const float mn = mv ? mx : m;
        const float al = fast_exp2(m - mn);
        m = mn;
        l *= al;
#pragma unroll
        for (int rg = 0; rg < 4; ++rg)
#pragma unroll
          for (int j = 0; j < 16; ++j) acc[rg][j] = scale_acc(acc[rg][j], al);
      }
    }
    f32x8 x, y;
    float sum = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      x[e] = fast_exp2(fmaf(S[e], cs, -m));
      y[e] = fast_exp2(fmaf(S[8 + e], cs, -m));
      sum += x[e] + y[e];
    }
    l += sum;
    pa = __builtin_convertvector(x, bf16x8);
    pb = __builtin_convertvector(y, bf16x8);
  };

  acc_pin(acc1);
  acc_pin(acc2);
  for (int rd = 0; rd < nr; ++rd) {
    const int c = rd & 1;
    const int64_t kb = kfirst + static_cast<int64_t>(rd) * KPR;
    acc_pin(acc1);
    acc_pin(acc2);
    // This round's 16 loads are done; the next round's may still be in flight.
    if (rd + 1 < nr) {
      asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
    } else {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    const lds_char* bk = wbuf + c * BUF;
    u32x4 kx[4], ky[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int off = kra + 16 * ((2 * kk + h) ^ ks);
      kx[kk] = ds_read_b128(bk + off);
      ky[kk] = ds_read_b128(bk + KT + off);
    }
    u32x4 vt[2][4];
    const lds_char* vb = bk + 2 * KT + vta;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const u32x2 lo = ds_read_tr16(vb + VREG * rg + 1024 * t);
        const u32x2 hi = ds_read_tr16(vb + VREG * rg + 1024 * t + 4 * 64);
        vt[t][rg] = u32x4{lo[0], lo[1], hi[0], hi[1]};
      }
    }
    // Every read of buffer c is done before the round after next is loaded into it.
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if (rd + 2 < nr) issue(kb + 2 * KPR, c);
    f32x16 S1 = {}, S2 = {};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      S1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kx[kk]), qa[kk], S1, 0, 0, 0);
      S2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, ky[kk]), qb[kk], S2, 0, 0, 0);
    }
    bf16x8 p1a, p1b, p2a, p2b;
    softmax(S1, kb, rd == 0, m1, l1, acc1, p1a, p1b);
    softmax(S2, kb, rd == 0, m2, l2, acc2, p2a, p2b);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const bf16x8 va = __builtin_bit_cast(bf16x8, vt[t][rg]);
        acc1[rg] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, t ? p1b : p1a, acc1[rg], 0, 0, 0);
        acc2[rg] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, t ? p2b : p2a, acc2[rg], 0, 0, 0);
      }
    }
  }
  l1 += __shfl_xor(l1, 32);
  l2 += __shfl_xor(l2, 32);

  // Merge the four wavefronts per query head: red[w][q][map] = (m, l, acc[128]).
  __syncthreads();   // every wavefront is done with its buffers
  float* red = reinterpret_cast<float*>(lds_raw);
  auto slot = [&](int w, int q, int mp) { return red + ((w * gq + q) * 2 + mp) * PART; };
  if (n < gq) {
    float* r1 = slot(wv, n, 0);
    float* r2 = slot(wv, n, 1);
    if (h == 0) {
      r1[0] = m1; r1[1] = l1;
      r2[0] = m2; r2[1] = l2;
    }
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        r1[2 + 32 * rg + chan_of(j, h)] = acc1[rg][j];
        r2[2 + 32 * rg + chan_of(j, h)] = acc2[rg][j];
      }
    }
  }
  __syncthreads();
  for (int it = tid; it < gq * 2 * DV; it += NT) {
    const int q = it / (2 * DV), mp = (it / DV) & 1, ch = it % DV;
    float M = slot(0, q, mp)[0];
#pragma unroll
    for (int w = 1; w < 4; ++w) M = fmaxf(M, slot(w, q, mp)[0]);
    float A = 0.f, Ssum = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float* r = slot(w, q, mp);
      const float sc = fast_exp2(r[0] - M);   // 0 for a wavefront without keys (m = -inf)
      A = fmaf(r[2 + ch], sc, A);
      Ssum = fmaf(r[1], sc, Ssum);
    }
    float* out = partial + ((h0 + q) * n_split + split) * 2 * PART + mp * PART;
    out[2 + ch] = A;
    if (ch == 0) {
      out[0] = M;
      out[1] = Ssum;
    }
  }
}

// LDS bytes of decode_mfma_kernel for gq query heads per workgroup: the V buffers during
// the rounds, then the merge of the four wavefront states.
size_t decode_mfma_lds_bytes(int gq) {
  const size_t merge = static_cast<size_t>(4) * gq * 2 * PART * sizeof(float);
  const size_t bufs = static_cast<size_t>(4) * gq::WAVE_LDS;
  return merge > bufs ? merge : bufs;
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

void decode_geometry(int64_t B, int64_t H, int64_t G, int64_t L, int* gq, int* n_split,
                     int* split_len) {
  // The query heads of a group on the matrix cores, gq at a time: the largest divisor of
  // the group size up to 32 (the B operand's columns).
  int c = 1;
  for (int t = 1; t <= 32 && t <= G; ++t)
    if (G % t == 0) c = t;
  const int64_t groups = B * H / c;
  // 32-key rounds per wavefront, splits of 128 x rounds keys: as long as possible (up to
  // 8192 keys) while there is a workgroup for every compute unit, since a workgroup fills
  // its unit's LDS and each one that ends drains the unit's load pipeline; at least 512.
  int rounds = 64;
  while (rounds > 4 && groups * ((L + 128 * rounds - 1) / (128 * rounds)) < 256) rounds >>= 1;
  const int64_t sl = static_cast<int64_t>(dec::gq::KPR) * 4 * rounds;
  *gq = c;
  *split_len = static_cast<int>(sl);
  *n_split = static_cast<int>((L + sl - 1) / sl);
}

hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t s) {
  using namespace dec;
  const int64_t BH = a.B * a.H;
  const int gq = a.gq;
  const int rounds = a.split_len / (gq::KPR * 4);
  static std::atomic<uint64_t> attr_done{0};
  const hipError_t ea = once_per_device(attr_done, [] {
    return hipFuncSetAttribute(reinterpret_cast<const void*>(decode_mfma_kernel),
                               hipFuncAttributeMaxDynamicSharedMemorySize,
                               static_cast<int>(decode_mfma_lds_bytes(32)));
  });
  if (ea != hipSuccess) return ea;
  hipLaunchKernelGGL(decode_mfma_kernel, dim3(a.n_split, static_cast<unsigned>(BH / gq)),
                     dim3(NT), decode_mfma_lds_bytes(gq), s, static_cast<const bf16_t*>(a.q1),
                     static_cast<const bf16_t*>(a.q2), static_cast<const bf16_t*>(a.k1),
                     static_cast<const bf16_t*>(a.k2), static_cast<const bf16_t*>(a.v),
                     a.cache_len, a.partial, a.H, a.L, a.n_split, rounds, a.G, gq);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_combine_kernel, dim3(static_cast<unsigned>(BH)), dim3(2 * DV), 0, s,
                     a.partial, a.cache_len, a.lam, a.rms_weight, static_cast<bf16_t*>(a.out),
                     a.H, a.L, a.n_split, static_cast<int64_t>(a.split_len), a.eps);
  return hipGetLastError();
}

}  // namespace diffattn
