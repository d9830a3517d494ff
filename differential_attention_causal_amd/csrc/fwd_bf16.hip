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
//  * K1, K2 (64 keys x 64) and V^T tiles go through a ring of three LDS stages with one
//    barrier per 64 keys; V is transposed in registers on its way to LDS. Every LDS
//    operand read is a per-lane base register plus a compile-time offset (the stage loop
//    is unrolled over the ring), and the layouts keep those reads and the transposing
//    writes free of bank conflicts;
//  * software pipeline per 32-key sub-tile: the QK^T MFMAs of the next sub-tile are
//    issued with the exponentials of the current one, and its PV MFMAs with the next
//    sub-tile's row maxima;
//  * the running max moves lazily (see maybe_rescale), so the 256 accumulator registers
//    are rescaled only a handful of times per row;
//  * stages wholly below the query tile run without mask code; the last two stages apply
//    the causal predicate key <= query as an integer compare. Keys beyond N are clamped
//    loads that the same predicate masks; rows beyond N are not stored;
//  * workgroups run longest-first (the last query tiles have the most keys), and
//    consecutive workgroup ids take different heads so that the tiles of one head land
//    on the same XCD (ids are dealt to the 8 XCDs round-robin) and share its L2.
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace diffattn {
namespace fwdbf16 {

constexpr int D = 64;
constexpr int DV = 128;
constexpr int BR = 128;       // query rows per workgroup
constexpr int BC = 64;        // keys per LDS stage
constexpr int NT = 256;       // threads per workgroup
constexpr int NBUF = 3;       // LDS ring of stages

// LDS layout (bytes): [V^T stage 0..2][K1 stage 0..2][K2 stage 0..2].
// V^T stage: 4 blocks, one per (32-key half sb, 16-key step t) = block 2 sb + t; a block
// holds 128 channel rows of 16 keys (32 B), padded by 32 B so the four blocks start in
// different banks. Inside a row the two 16-byte halves are swapped on bit 2 of the row.
// K stage: 64 key rows of 128 B; 16-byte unit u of row r is stored at u ^ k_swz(r).
constexpr int VROW = 32;
constexpr int VBLK = DV * VROW + 32;          // 4128
constexpr int VSTAGE = 4 * VBLK;              // 16512
constexpr int KSTAGE = BC * D * 2;            // 8192
constexpr int V_BASE = 0;
constexpr int K1_BASE = NBUF * VSTAGE;        // 49536
constexpr int K2_BASE = K1_BASE + NBUF * KSTAGE;
constexpr int LDS_BYTES = K2_BASE + NBUF * KSTAGE;  // 98688
static_assert(K1_BASE % 16 == 0 && K2_BASE % 16 == 0, "16-byte aligned regions");

__device__ __forceinline__ int k_swz(int row) { return (row & 3) | ((row >> 1) & 4); }

// Physical key (0..31 within a 32-key sub-tile) held in score register j by lane half h.
__device__ __forceinline__ int key_of(int j, int h) { return 16 * (j >> 3) + 8 * h + (j & 7); }
// K row loaded into MFMA operand row m: swaps bits 2 and 3.
__device__ __forceinline__ int perm_row(int m) {
  return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}

struct StageRegs {
  u32x4 k1[2], k2[2], v[4];
};

// Tile loads are raw buffer loads through a resource descriptor that starts at the
// stage's first key and covers the rows that remain below N: rows at or beyond N read as
// zero in hardware (their scores are masked by the causal predicate, key > query for
// every stored row). The per-thread offsets are constant, so a stage costs no vector ALU
// work for addressing.
constexpr int kBufFlags = 0x00020000;  // raw 32-bit buffer, no swizzle

struct HeadRsrc {
  __amdgpu_buffer_rsrc_t k1, k2, v;
};

// k0: first key of the stage; kvo / vvo: this thread's constant byte offsets in a K / V
// tile. The descriptors cover the head's N rows, so rows at or beyond N read as zero.
__device__ __forceinline__ void load_stage(StageRegs& r, const HeadRsrc& rs, int k0, int kvo,
                                           int vvo) {
  // K: 16-byte chunk c = tid + 256 t of the 64 x 128-byte tile (row c / 8, unit c % 8).
  const int ko = kvo + k0 * (D * 2);
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    r.k1[t] = __builtin_amdgcn_raw_buffer_load_b128(rs.k1, ko + 4096 * t, 0, 0);
    r.k2[t] = __builtin_amdgcn_raw_buffer_load_b128(rs.k2, ko + 4096 * t, 0, 0);
  }
  // V: thread (kg = tid % 16, dg = tid / 16) takes keys 4kg..4kg+3, channels 8dg..8dg+7.
  const int vo = vvo + k0 * (DV * 2);
#pragma unroll
  for (int t = 0; t < 4; ++t) r.v[t] = __builtin_amdgcn_raw_buffer_load_b128(rs.v, vo + 256 * t, 0, 0);
}

// kw / kw2: this thread's K1 / K2 write address in ring slot 0 (chunk tid; chunk
// tid + 256 is 32 rows further); vw0 / vw1: its V^T write address for channels c < 4 and
// c >= 4 of its 8 (the 16-byte half flips with bit 2 of the channel row).
__device__ __forceinline__ void store_stage(const StageRegs& r, char* __restrict__ lds,
                                            int buf, int kw, int kw2, int vw0, int vw1) {
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    *reinterpret_cast<u32x4*>(lds + kw + buf * KSTAGE + 4096 * t) = r.k1[t];
    *reinterpret_cast<u32x4*>(lds + kw2 + buf * KSTAGE + 4096 * t) = r.k2[t];
  }
  // Transpose 4 keys x 8 channels to 8 channel rows of 4 keys (8 bytes each). The 16
  // lanes sharing dg write 16 different 8-byte slots of one row position: no conflicts.
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    // channel c of keys (4kg, 4kg+1) and (4kg+2, 4kg+3), low half = earlier key
    const uint32_t x0 = r.v[0][c >> 1], x1 = r.v[1][c >> 1];
    const uint32_t x2 = r.v[2][c >> 1], x3 = r.v[3][c >> 1];
    const uint32_t lo = (c & 1) ? ((x0 >> 16) | (x1 & 0xffff0000u)) : ((x0 & 0xffffu) | (x1 << 16));
    const uint32_t hi = (c & 1) ? ((x2 >> 16) | (x3 & 0xffff0000u)) : ((x2 & 0xffffu) | (x3 << 16));
    u32x2 w = {lo, hi};
    *reinterpret_cast<u32x2*>(lds + (c < 4 ? vw0 : vw1) + buf * VSTAGE + c * VROW) = w;
  }
}

__device__ __forceinline__ bf16x8 lds_read8(const char* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}

// ---------------------------------------------------------------------------------
// The softmax uses a lazily updated row maximum: m only moves when a new score exceeds
// it by more than kTau (in log2 units), so the accumulators are rescaled rarely; until
// then p = exp2(s c - m) <= 2^kTau. The final O = acc / l and the log-sum-exp
// m + log2(l) do not depend on which m was used.
constexpr float kTau = 8.0f;

struct Scores {
  f32x16 s1, s2;
};

// S^T = K Q^T for both maps (8 MFMAs). kaddr: per-lane LDS byte addresses of the K1
// operand rows for the 4 channel blocks; koff: stage and sub-tile byte offset.
__device__ __forceinline__ void qk_tile(Scores& S, const char* lds, const int* kaddr, int koff,
                                        const bf16x8* qf1, const bf16x8* qf2) {
#pragma unroll
  for (int j = 0; j < 16; ++j) S.s1[j] = S.s2[j] = 0.f;
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    const char* p = lds + kaddr[kb] + koff;
    S.s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_read8(p), qf1[kb], S.s1, 0, 0, 0);
    S.s2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_read8(p + (K2_BASE - K1_BASE)),
                                                   qf2[kb], S.s2, 0, 0, 0);
  }
}

__device__ __forceinline__ float max16(const f32x16& s) {
  float a = fmaxf(s[0], s[1]);
#pragma unroll
  for (int j = 2; j < 16; j += 2) a = fmaxf(a, fmaxf(s[j], s[j + 1]));
  return a;
}

// Row maxima of a fresh score tile (scaled, log2 domain), merged across lane halves.
__device__ __forceinline__ void tile_max(const Scores& S, float c, float& t1, float& t2) {
  float a = max16(S.s1), b = max16(S.s2);
  a = fmaxf(a, __shfl_xor(a, 32));
  b = fmaxf(b, __shfl_xor(b, 32));
  t1 = a * c;
  t2 = b * c;
}

// p = exp2(s c - m) for 16 scores; returns the bf16 operands of the two PV k-steps and
// adds the fp32 weights to l.
__device__ __forceinline__ void exp_tile(const f32x16& s, float c, float m, float& l,
                                         bf16x8& pa, bf16x8& pb) {
  f32x8 x, y;
  float sa = 0.f, sb = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    x[e] = fast_exp2(fmaf(s[e], c, -m));
    y[e] = fast_exp2(fmaf(s[8 + e], c, -m));
    sa += x[e];
    sb += y[e];
  }
  l += sa + sb;
  pa = __builtin_convertvector(x, bf16x8);
  pb = __builtin_convertvector(y, bf16x8);
}

// O^T += V^T P^T for both maps (16 MFMAs). vaddr: per-lane V^T byte address; voff: stage
// and sub-tile byte offset.
__device__ __forceinline__ void pv_tile(f32x16* acc1, f32x16* acc2, const char* lds, int vaddr,
                                        int voff, const bf16x8& p1a, const bf16x8& p1b,
                                        const bf16x8& p2a, const bf16x8& p2b) {
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const char* p = lds + vaddr + voff + b * 32 * VROW;
    const bf16x8 va = lds_read8(p);
    const bf16x8 vb = lds_read8(p + VBLK);
    acc1[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, p1a, acc1[b], 0, 0, 0);
    acc2[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, p2a, acc2[b], 0, 0, 0);
    acc1[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vb, p1b, acc1[b], 0, 0, 0);
    acc2[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vb, p2b, acc2[b], 0, 0, 0);
  }
}

// Causal predicate on a sub-tile starting at key ks: key > query -> -inf.
__device__ __forceinline__ void mask_tile(Scores& S, int ks, int q, int h) {
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    if (ks + key_of(j, h) > q) {
      S.s1[j] = -INFINITY;
      S.s2[j] = -INFINITY;
    }
  }
}

// Lazy max update for the next tile. The branch is taken when some row of the wave grew
// by more than kTau, but each row moves its own maximum only on its own trigger (the
// others multiply by exactly 1), so every row's result depends on its own scores only.
__device__ __forceinline__ void maybe_rescale(float t1, float t2, float& m1, float& m2,
                                              float& l1, float& l2, f32x16* acc1,
                                              f32x16* acc2) {
  const bool n1 = t1 > m1 + kTau, n2 = t2 > m2 + kTau;
  if (__builtin_expect(__any(n1 || n2), 0)) {
    const float a1 = n1 ? fast_exp2(m1 - t1) : 1.0f;
    const float a2 = n2 ? fast_exp2(m2 - t2) : 1.0f;
    m1 = n1 ? t1 : m1;
    m2 = n2 ? t2 : m2;
    l1 *= a1;
    l2 *= a2;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        acc1[b][j] *= a1;
        acc2[b][j] *= a2;
      }
    }
  }
}

using NoMask = std::integral_constant<bool, false>;
using Mask = std::integral_constant<bool, true>;

__global__ void __launch_bounds__(NT, 1) fwd_bf16_kernel(
    const bf16_t* __restrict__ q1, const bf16_t* __restrict__ q2,
    const bf16_t* __restrict__ k1, const bf16_t* __restrict__ k2,
    const bf16_t* __restrict__ v, const diffattn_lambda_state* __restrict__ lamst,
    const float* __restrict__ rms_w, bf16_t* __restrict__ out, float* __restrict__ sv_lse1,
    float* __restrict__ sv_lse2, float* __restrict__ sv_o1, float* __restrict__ sv_o2,
    float* __restrict__ sv_rstd, int BH, int H, int N, int nqb, float eps) {
  extern __shared__ __attribute__((aligned(16))) char lds[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int m = lane & 31;
  const int h = lane >> 5;

  // Longest-first over query tiles; consecutive ids walk the heads.
  const int bid = blockIdx.x;
  const int bh = bid % BH;
  const int qb = nqb - 1 - bid / BH;
  const int q0 = qb * BR;
  const int q0w = q0 + 32 * wv;
  const int64_t hoff = static_cast<int64_t>(bh) * N;

  const bf16_t* Q1 = q1 + hoff * D;
  const bf16_t* Q2 = q2 + hoff * D;
  const bf16_t* K1 = k1 + hoff * D;
  const bf16_t* K2 = k2 + hoff * D;
  const bf16_t* V = v + hoff * DV;

  // Q^T operand: lane holds query q0w + m, channels 16 kb + 8 h .. + 7.
  bf16x8 qf1[4], qf2[4];
  {
    const int q = min(q0w + m, N - 1);
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      qf1[kb] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(Q1 + q * D + 16 * kb + 8 * h));
      qf2[kb] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(Q2 + q * D + 16 * kb + 8 * h));
    }
  }
  // Per-lane LDS operand addresses (bytes).
  int kaddr[4];
  {
    const int kr = perm_row(m);
    const int ks = k_swz(kr);
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) kaddr[kb] = K1_BASE + kr * 128 + 16 * ((2 * kb + h) ^ ks);
  }
  int vaddr = V_BASE + m * VROW + 16 * (h ^ ((m >> 2) & 1));
  HeadRsrc rs;
  rs.k1 = __builtin_amdgcn_make_buffer_rsrc((void*)K1, 0, N * D * 2, kBufFlags);
  rs.k2 = __builtin_amdgcn_make_buffer_rsrc((void*)K2, 0, N * D * 2, kBufFlags);
  rs.v = __builtin_amdgcn_make_buffer_rsrc((void*)V, 0, N * DV * 2, kBufFlags);
  // Tile load offsets and LDS write addresses of this thread (see load/store_stage).
  const int kvo = 16 * tid;
  const int kgi = tid & 15, dgi = tid >> 4;
  const int vvo = 4 * kgi * DV * 2 + 16 * dgi;
  int kw, kw2, vw0, vw1;
  {
    const int row = tid >> 3, u = tid & 7;
    kw = K1_BASE + row * 128 + 16 * (u ^ k_swz(row));
    kw2 = kw + (K2_BASE - K1_BASE);
    const int blk = kgi >> 2, uu = (kgi >> 1) & 1, half = kgi & 1;
    const int vb = V_BASE + blk * VBLK + 8 * half + 8 * dgi * VROW;
    vw0 = vb + 16 * uu;
    vw1 = vb + 16 * (uu ^ 1);
  }

  const float c = kLog2e / 8.0f;  // log2(e) / sqrt(64)
  float m1 = -INFINITY, m2 = -INFINITY, l1 = 0.f, l2 = 0.f;
  f32x16 acc1[4], acc2[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) {
#pragma unroll
    for (int j = 0; j < 16; ++j) acc1[b][j] = acc2[b][j] = 0.f;
  }

  const int kend = min(N, q0 + BR);
  const int n_stages = (kend + BC - 1) / BC;
  const int n_full = q0 / BC;  // stages whose keys are all < q0: no mask for any row
  const int qrow = q0w + m;

  // One pipeline step: QK^T of the next sub-tile (K operand bases kb + byte offset
  // kofs) while the current tile's exponentials are formed, then PV of the current tile
  // (V^T base vb + byte offset vofs) while the next tile's row maxima are taken.
  auto step = [&](auto mask_tag, Scores& cur, Scores& nxt, const int* kb, int kofs, int vb,
                  int vofs, int nt) __attribute__((always_inline)) {
    constexpr bool kMask = decltype(mask_tag)::value;
    qk_tile(nxt, lds, kb, kofs, qf1, qf2);
    bf16x8 p1a, p1b, p2a, p2b;
    exp_tile(cur.s1, c, m1, l1, p1a, p1b);
    exp_tile(cur.s2, c, m2, l2, p2a, p2b);
    if (kMask) mask_tile(nxt, 32 * nt, qrow, h);
    pv_tile(acc1, acc2, lds, vb, vofs, p1a, p1b, p2a, p2b);
    float t1, t2;
    tile_max(nxt, c, t1, t2);
    maybe_rescale(t1, t2, m1, m2, l1, l2, acc1, acc2);
  };
  // The per-lane LDS bases follow the ring: kcur / vcur address ring slot s % 3 (the
  // stage being consumed) and kw.. the slot (s + 1) % 3 being filled; each advances by
  // one slot per stage, wrapping after three.
  int kcur[4] = {kaddr[0], kaddr[1], kaddr[2], kaddr[3]};
  int vcur = vaddr;
  kw += KSTAGE;
  kw2 += KSTAGE;
  vw0 += VSTAGE;
  vw1 += VSTAGE;
  int slot = 0;
  // Stage s: sub-tiles 2s (in A) and 2s+1, and the QK^T of sub-tile 2s+2 (stage s+1).
  // Stage s+1 was fetched into registers when stage s opened; it is written to its slot
  // here, opened at the barrier, and stage s+2 is fetched.
  Scores A, B;
  StageRegs regs;
  auto stage = [&](auto mask_tag, int s) __attribute__((always_inline)) {
    const int kstep = slot == 2 ? -2 * KSTAGE : KSTAGE;
    const int vstep = slot == 2 ? -2 * VSTAGE : VSTAGE;
    const int wk = slot == 1 ? -2 * KSTAGE : KSTAGE;   // the filled slot is one ahead
    const int wv = slot == 1 ? -2 * VSTAGE : VSTAGE;
    int knext[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) knext[i] = kcur[i] + kstep;
    step(mask_tag, A, B, kcur, 32 * 128, vcur, 0, 2 * s + 1);
    store_stage(regs, lds, 0, kw, kw2, vw0, vw1);
    __syncthreads();
    if (s + 2 < n_stages) load_stage(regs, rs, (s + 2) * BC, kvo, vvo);
    step(mask_tag, B, A, knext, 0, vcur, 2 * VBLK, 2 * s + 2);
#pragma unroll
    for (int i = 0; i < 4; ++i) kcur[i] = knext[i];
    vcur += vstep;
    kw += wk;
    kw2 += wk;
    vw0 += wv;
    vw1 += wv;
    slot = slot == 2 ? 0 : slot + 1;
  };

  // Prologue: stage 0 resident, stage 1 in flight, scores and max of sub-tile 0.
  load_stage(regs, rs, 0, kvo, vvo);
  store_stage(regs, lds, 0, kw - KSTAGE, kw2 - KSTAGE, vw0 - VSTAGE, vw1 - VSTAGE);
  __syncthreads();
  if (n_stages > 1) load_stage(regs, rs, BC, kvo, vvo);
  qk_tile(A, lds, kcur, 0, qf1, qf2);
  if (n_full == 0) mask_tile(A, 0, qrow, h);
  {
    float t1, t2;
    tile_max(A, c, t1, t2);
    maybe_rescale(t1, t2, m1, m2, l1, l2, acc1, acc2);
  }
  int s = 0;
  for (; s + 1 < n_full; ++s) stage(NoMask{}, s);   // stages wholly below the query tile
  for (; s + 1 < n_stages; ++s) stage(Mask{}, s);   // at most two touching the diagonal
  {
    // Last stage: sub-tiles 2s and 2s+1, nothing further to fetch.
    step(Mask{}, A, B, kcur, 32 * 128, vcur, 0, 2 * s + 1);
    bf16x8 p1a, p1b, p2a, p2b;
    exp_tile(B.s1, c, m1, l1, p1a, p1b);
    exp_tile(B.s2, c, m2, l2, p2a, p2b);
    pv_tile(acc1, acc2, lds, vcur, 2 * VBLK, p1a, p1b, p2a, p2b);
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
  if (qrow < N) {
    const int hh = bh % H;
    bf16_t* Y = out + (hoff + qrow) * DV;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
#pragma unroll
      for (int jg = 0; jg < 4; ++jg) {
        const int col = 32 * b + 8 * jg + 4 * h;
        f32x4 w = {1.f, 1.f, 1.f, 1.f};
        if (rms_w) w = *reinterpret_cast<const f32x4*>(rms_w + hh * DV + col);
        float y[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float o = acc1[b][4 * jg + e] - lam * acc2[b][4 * jg + e];
          y[e] = g * (w[e] * (o * rstd));
        }
        u32x2 pk = {pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
        *reinterpret_cast<u32x2*>(Y + col) = pk;
        if (sv_o1) {
          f32x4 a = {acc1[b][4 * jg], acc1[b][4 * jg + 1], acc1[b][4 * jg + 2], acc1[b][4 * jg + 3]};
          f32x4 bb = {acc2[b][4 * jg], acc2[b][4 * jg + 1], acc2[b][4 * jg + 2], acc2[b][4 * jg + 3]};
          *reinterpret_cast<f32x4*>(sv_o1 + (hoff + qrow) * DV + col) = a;
          *reinterpret_cast<f32x4*>(sv_o2 + (hoff + qrow) * DV + col) = bb;
        }
      }
    }
    if (sv_lse1 && h == 0) {
      // lse_k = ln(sum_j exp(S_kj)) = (m_k + log2 l_k) * ln 2, m_k in the scaled log2 domain.
      sv_lse1[hoff + qrow] = (m1 + __log2f(l1)) * kLn2;
      sv_lse2[hoff + qrow] = (m2 + __log2f(l2)) * kLn2;
      sv_rstd[hoff + qrow] = rstd;
    }
  }
}

}  // namespace fwdbf16

hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t s) {
  using namespace fwdbf16;
  const int64_t BH = a.B * a.H;
  const int nqb = static_cast<int>((a.N + BR - 1) / BR);
  const int64_t nblk = BH * nqb;
  static bool attr_done = false;
  if (!attr_done) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&fwd_bf16_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, LDS_BYTES);
    if (e != hipSuccess) return e;
    attr_done = true;
  }
  const diffattn_saved& sv = a.saved;
  hipLaunchKernelGGL(fwd_bf16_kernel, dim3(static_cast<unsigned>(nblk)), dim3(NT), LDS_BYTES, s,
                     static_cast<const bf16_t*>(a.q1), static_cast<const bf16_t*>(a.q2),
                     static_cast<const bf16_t*>(a.k1), static_cast<const bf16_t*>(a.k2),
                     static_cast<const bf16_t*>(a.v), a.lam, a.rms_weight,
                     static_cast<bf16_t*>(a.out), a.training ? sv.lse1 : nullptr,
                     a.training ? sv.lse2 : nullptr, a.training ? sv.o1 : nullptr,
                     a.training ? sv.o2 : nullptr, a.training ? sv.rstd : nullptr,
                     static_cast<int>(BH), static_cast<int>(a.H), static_cast<int>(a.N), nqb,
                     a.eps);
  return hipGetLastError();
}

}  // namespace diffattn
