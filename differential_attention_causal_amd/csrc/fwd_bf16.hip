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
// Work decomposition: one workgroup = 4 wavefronts = 128 query rows of one (b, h); two
// workgroups per CU, so each SIMD runs two wavefronts from different workgroups and one
// wave's softmax (vector ALU) overlaps the other's matrix-core work without the two
// being held in step by a shared barrier.
//  * each wavefront owns 32 query rows and computes the transposed score tile
//    S^T = K Q^T (32 keys x 32 queries) with v_mfma_f32_32x32x16_bf16, so each lane
//    holds 16 scores of ONE query; the row max needs one exchange with lane ^ 32;
//  * the key rows fed to the MFMA are permuted (bits 2 and 3 of the row swapped) so that
//    the score registers are directly the B operand of O^T += V^T P^T;
//  * K1, K2 and V tiles of 64 keys go from HBM straight into LDS (buffer loads with the
//    LDS as destination, double buffered, one barrier per tile). Rows at or beyond N read
//    as zero. The V^T operand comes out of the row-major V tile with the transposing LDS
//    read ds_read_b64_tr_b16: in each group of 16 lanes, lane 4a+b receives element b of
//    the 8 bytes that lanes 4j+a (j = 0..3) addressed; so lane 4j+a of group G points at
//    key 8(G/2)+j, channels 32 blk + 16(G%2) + 4a .. +3, and every MFMA lane ends up with
//    8 consecutive keys of one channel;
//  * LDS swizzles keep every operand read free of bank conflicts; operand addresses are a
//    per-lane base plus compile-time offsets;
//  * the running max moves lazily (see maybe_rescale), so the accumulators are rescaled
//    only a handful of times per row;
//  * sub-tiles wholly below a wave's rows run without mask code; the diagonal sub-tile
//    applies the causal predicate key <= query as an integer compare; later ones are
//    skipped;
//  * workgroups run longest-first (the last query tiles have the most keys), and
//    consecutive workgroup ids take different heads so that the tiles of one head land on
//    the same XCD (ids are dealt to the 8 XCDs round-robin) and share its L2.
#include "common.h"
#include "launch.h"

namespace diffattn {
namespace fwdbf16 {

#define LDS_AS __attribute__((address_space(3)))

constexpr int D = 64;
constexpr int DV = 128;
#ifndef DIFFATTN_FWD_WAVES
#define DIFFATTN_FWD_WAVES 4
#endif
// Wavefronts per workgroup. With 4, two workgroups share each CU (two waves per SIMD from
// different workgroups, so their barriers do not keep them in step).
constexpr int NW = DIFFATTN_FWD_WAVES;
constexpr int NT = 64 * NW;   // threads per workgroup
constexpr int BR = 32 * NW;   // query rows per workgroup
#ifndef DIFFATTN_FWD_TILE
#define DIFFATTN_FWD_TILE 64
#endif
constexpr int BC = DIFFATTN_FWD_TILE;  // keys per LDS tile (one barrier per tile)

// LDS slot (bytes): K1 [BC keys][128 B] | K2 [BC keys][128 B] | V in 4 regions of 32
// channels, [BC keys][64 B] each. Two slots.
constexpr int KTILE = BC * 128;
constexpr int VREG = BC * 64;
constexpr int K1_OFF = 0;
constexpr int K2_OFF = KTILE;
constexpr int V_OFF = 2 * KTILE;
constexpr int SLOT = 2 * KTILE + 4 * VREG;
constexpr int LDS_BYTES = 2 * SLOT;
constexpr int KBLK = BC / (8 * NW);   // 1 KB K1 (and K2) blocks per wave per tile
constexpr int VBLK = BC / (4 * NW);   // 1 KB V blocks per wave per tile
static_assert(BC % 64 == 0, "tile of 64-key multiples");

// K rows: 16-byte unit u stored at u ^ k_swz(row). Bits (b0 ^ b2, b1, b3): the 16 rows a
// group of 16 operand lanes reads land in 16 different bank slots of 256 bytes, and any 8
// of them in 8 slots of 128 bytes.
__device__ __forceinline__ int k_swz(int row) {
  return ((row ^ (row >> 2)) & 1) | (row & 2) | ((row >> 1) & 4);
}
// V rows (64 B, four 16-byte chunks): chunk c stored at c ^ v_swz(row).
__device__ __forceinline__ int v_swz(int row) { return 2 * ((row >> 1) & 1); }

// Physical key (0..31 within a 32-key sub-tile) held in score register j by lane half h.
__device__ __forceinline__ int key_of(int j, int h) { return 16 * (j >> 3) + 8 * h + (j & 7); }
// K row loaded into MFMA operand row m: swaps bits 2 and 3.
__device__ __forceinline__ int perm_row(int m) {
  return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}

constexpr int kBufFlags = 0x00020000;  // raw 32-bit buffer, no swizzle

// Per-thread DMA source offsets (bytes, for tile key 0). K1 (and K2) block i holds key
// rows 8i .. 8i+7; wave w moves blocks w + NW r. V block i holds rows 16 (i % (BC/16)) ..
// +15 of region i / (BC/16); wave w moves blocks w + NW r. The swizzles depend only on
// the low row bits, which the blocks of one wave share.
struct DmaPlan {
  int k[KBLK];
  int v[VBLK];
};

__device__ __forceinline__ DmaPlan dma_plan(int wv, int lane) {
  DmaPlan p;
#pragma unroll
  for (int r = 0; r < KBLK; ++r) {
    const int row = 8 * (wv + NW * r) + (lane >> 3), pu = lane & 7;
    p.k[r] = row * (D * 2) + 16 * (pu ^ k_swz(row));
  }
#pragma unroll
  for (int r = 0; r < VBLK; ++r) {
    const int i = wv + NW * r;
    const int region = i / (BC / 16);
    const int row = 16 * (i % (BC / 16)) + (lane >> 2), pc = lane & 3;
    p.v[r] = row * (DV * 2) + 64 * region + 16 * (pc ^ v_swz(row));
  }
  return p;
}

struct HeadRsrc {
  __amdgpu_buffer_rsrc_t k1, k2, v;
};

// Issues this wave's share of tile k0 into LDS slot `slot` (lane l's 16 bytes land at
// block base + 16 l).
__device__ __forceinline__ void dma_tile(const HeadRsrc& rs, const DmaPlan& p, char* lds,
                                         int slot, int k0, int wv) {
  LDS_AS char* base = (LDS_AS char*)(lds) + slot * SLOT;
#pragma unroll
  for (int r = 0; r < KBLK; ++r) {
    const int ko = p.k[r] + k0 * (D * 2);
    LDS_AS char* dst = base + 1024 * (wv + NW * r);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs.k1, (LDS_AS void*)(dst + K1_OFF), 16, ko, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs.k2, (LDS_AS void*)(dst + K2_OFF), 16, ko, 0, 0, 0);
  }
#pragma unroll
  for (int r = 0; r < VBLK; ++r) {
    LDS_AS char* dst = base + V_OFF + 1024 * (wv + NW * r);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs.v, (LDS_AS void*)(dst), 16, p.v[r] + k0 * (DV * 2), 0, 0, 0);
  }
}

__device__ __forceinline__ bf16x8 lds_read8(const char* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}

// The V^T operand reads are issued as inline assembly: the compiler cannot tell that a
// transposing LDS read does not overlap the tile being fetched into the other LDS slot,
// and would otherwise wait for that fetch before every read. Their completion is awaited
// explicitly (vt_wait) before the PV products, tied to the registers they fill.
template <int OFF>
__device__ __forceinline__ u32x2 ds_read_tr16(int addr) {
  u32x2 r;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "n"(OFF));
  return r;
}

// The 16 reads of one sub-tile: for region b and k-step t, keys e = 0..3 of the lane's 8
// and (4 rows further) e = 4..7.
struct VtRegs {
  u32x2 r[4][2][2];
};

template <int B, int T>
__device__ __forceinline__ void vt_issue_bt(VtRegs& v, int addr) {
  v.r[B][T][0] = ds_read_tr16<V_OFF + VREG * B + 1024 * T>(addr);
  v.r[B][T][1] = ds_read_tr16<V_OFF + VREG * B + 1024 * T + 4 * 64>(addr);
}

__device__ __forceinline__ void vt_issue(VtRegs& v, int addr) {
  vt_issue_bt<0, 0>(v, addr); vt_issue_bt<0, 1>(v, addr);
  vt_issue_bt<1, 0>(v, addr); vt_issue_bt<1, 1>(v, addr);
  vt_issue_bt<2, 0>(v, addr); vt_issue_bt<2, 1>(v, addr);
  vt_issue_bt<3, 0>(v, addr); vt_issue_bt<3, 1>(v, addr);
}

__device__ __forceinline__ void vt_wait(VtRegs& v) {
  asm volatile("s_waitcnt lgkmcnt(0)"
               : "+v"(v.r[0][0][0]), "+v"(v.r[0][0][1]), "+v"(v.r[0][1][0]), "+v"(v.r[0][1][1]),
                 "+v"(v.r[1][0][0]), "+v"(v.r[1][0][1]), "+v"(v.r[1][1][0]), "+v"(v.r[1][1][1]),
                 "+v"(v.r[2][0][0]), "+v"(v.r[2][0][1]), "+v"(v.r[2][1][0]), "+v"(v.r[2][1][1]),
                 "+v"(v.r[3][0][0]), "+v"(v.r[3][0][1]), "+v"(v.r[3][1][0]), "+v"(v.r[3][1][1]));
}

__device__ __forceinline__ bf16x8 vt_operand(const VtRegs& v, int b, int t) {
  const u32x4 x = {v.r[b][t][0][0], v.r[b][t][0][1], v.r[b][t][1][0], v.r[b][t][1][1]};
  return __builtin_bit_cast(bf16x8, x);
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
// operand rows for the 4 channel blocks (slot 0, sub-tile 0); koff: slot and sub-tile.
__device__ __forceinline__ void qk_tile(Scores& S, const char* lds, const int* kaddr, int koff,
                                        const bf16x8* qf1, const bf16x8* qf2) {
#pragma unroll
  for (int j = 0; j < 16; ++j) S.s1[j] = S.s2[j] = 0.f;
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    const char* p = lds + kaddr[kb] + koff;
    S.s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_read8(p + K1_OFF), qf1[kb], S.s1, 0, 0, 0);
    S.s2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_read8(p + K2_OFF), qf2[kb], S.s2, 0, 0, 0);
  }
}

__device__ __forceinline__ float max16(const f32x16& s) {
  float a = fmaxf(s[0], s[1]);
#pragma unroll
  for (int j = 2; j < 16; j += 2) a = fmaxf(a, fmaxf(s[j], s[j + 1]));
  return a;
}

// max(x[l], x[l ^ 32]): v_permlane32_swap exchanges the upper half of its first operand
// with the lower half of its second, so with x in both the two results hold x[l] and
// x[l ^ 32] in every lane.
__device__ __forceinline__ float max_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Row maxima of a score tile (scaled, log2 domain), merged across lane halves.
__device__ __forceinline__ void tile_max(const Scores& S, float c, float& t1, float& t2) {
  float a = max16(S.s1), b = max16(S.s2);
  a = max_halves(a);
  b = max_halves(b);
  t1 = a * c;
  t2 = b * c;
}

// p = exp2(s c - m) for 16 scores; returns the bf16 operands of the two PV k-steps and
// adds their sum to l. The sum is taken over the bf16-rounded weights, the same values
// the PV product multiplies, two per v_dot2 against (1, 1).
__device__ __forceinline__ void exp_tile(const f32x16& s, float c, float m, float& l,
                                         bf16x8& pa, bf16x8& pb) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  f32x8 x, y;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    x[e] = fast_exp2(fmaf(s[e], c, -m));
    y[e] = fast_exp2(fmaf(s[8 + e], c, -m));
  }
  pa = __builtin_convertvector(x, bf16x8);
  pb = __builtin_convertvector(y, bf16x8);
  const bf16x2 one = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
  float sa = l, sb = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const bf16x2 a2 = {pa[2 * e], pa[2 * e + 1]};
    const bf16x2 b2 = {pb[2 * e], pb[2 * e + 1]};
    sa = __builtin_amdgcn_fdot2_f32_bf16(a2, one, sa, false);
    sb = __builtin_amdgcn_fdot2_f32_bf16(b2, one, sb, false);
  }
  l = sa + sb;
}

// O^T += V^T P^T for both maps (16 MFMAs), from the V^T operands already read.
__device__ __forceinline__ void pv_tile(f32x16* acc1, f32x16* acc2, const VtRegs& vt,
                                        const bf16x8& p1a, const bf16x8& p1b,
                                        const bf16x8& p2a, const bf16x8& p2b) {
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const bf16x8 va = vt_operand(vt, b, 0);
    const bf16x8 vb = vt_operand(vt, b, 1);
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

// Lazy max update. The branch is taken when some row of the wave grew by more than
// kTau, but each row moves its own maximum only on its own trigger (the others multiply
// by exactly 1), so every row's result depends on its own scores only.
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

__global__ void __launch_bounds__(NT, 8 / NW) fwd_bf16_kernel(
    const bf16_t* __restrict__ q1, const bf16_t* __restrict__ q2,
    const bf16_t* __restrict__ k1, const bf16_t* __restrict__ k2,
    const bf16_t* __restrict__ v, const diffattn_lambda_state* __restrict__ lamst,
    const float* __restrict__ rms_w, bf16_t* __restrict__ out, float* __restrict__ sv_lse1,
    float* __restrict__ sv_lse2, float* __restrict__ sv_o1, float* __restrict__ sv_o2,
    float* __restrict__ sv_rstd, int BH, int H, int N, int nqb, float eps) {
  __shared__ __attribute__((aligned(16))) char lds[LDS_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
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
  HeadRsrc rs;
  rs.k1 = __builtin_amdgcn_make_buffer_rsrc((void*)(k1 + hoff * D), 0, N * D * 2, kBufFlags);
  rs.k2 = __builtin_amdgcn_make_buffer_rsrc((void*)(k2 + hoff * D), 0, N * D * 2, kBufFlags);
  rs.v = __builtin_amdgcn_make_buffer_rsrc((void*)(v + hoff * DV), 0, N * DV * 2, kBufFlags);
  const DmaPlan plan = dma_plan(wv, lane);

  const int kend = min(N, q0 + BR);
  const int n_tiles = (kend + BC - 1) / BC;
  dma_tile(rs, plan, lds, 0, 0, wv);

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
  // Per-lane LDS operand addresses (bytes, slot 0, sub-tile 0).
  int kaddr[4];
  {
    const int kr = perm_row(m);
    const int ks = k_swz(kr);
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) kaddr[kb] = kr * 128 + 16 * ((2 * kb + h) ^ ks);
  }
  int vaddr;
  {
    const int G = lane >> 4, j = (lane >> 2) & 3, a = lane & 3;
    const int row = 8 * (G >> 1) + j;                 // + 32 sb + 16 t + 4 (second read)
    const int cp = 2 * (G & 1) + (a >> 1);
    vaddr = row * 64 + 16 * (cp ^ v_swz(row)) + 8 * (a & 1);
  }

  // LDS-relative byte address of the array, for the operands given to inline assembly.
  const int lds_base = static_cast<int>(reinterpret_cast<uintptr_t>((LDS_AS char*)lds));
  const float c = kLog2e / 8.0f;  // log2(e) / sqrt(64)
  float m1 = -INFINITY, m2 = -INFINITY, l1 = 0.f, l2 = 0.f;
  f32x16 acc1[4], acc2[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) {
#pragma unroll
    for (int j = 0; j < 16; ++j) acc1[b][j] = acc2[b][j] = 0.f;
  }
  const int qrow = q0w + m;
  // Sub-tiles (32 keys) below this wave's rows need no mask; sub-tile `diag` holds the
  // diagonal; later ones are skipped.
  const int diag = q0w / 32;

  // One loop over 32-key sub-tiles with a single copy of the body. The operand bases
  // follow the tile: sub-tile jt lives in slot (jt / 2) % 2 at half jt % 2.
  constexpr int SPT = BC / 32;  // sub-tiles per tile
  const int n_sub = min(SPT * n_tiles, diag + 1);
  int koff = 0, voff = 0;
  for (int jt = 0; jt < SPT * n_tiles; ++jt) {
    const int t = jt / SPT;
    if (jt % SPT == 0) {
      // Tile t resident: each wave waits for its own fetch, then all meet; the other slot
      // is then free for tile t + 1.
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      if (t + 1 < n_tiles) dma_tile(rs, plan, lds, (t + 1) & 1, (t + 1) * BC, wv);
    }
    if (jt < n_sub) {
      Scores S;
      qk_tile(S, lds, kaddr, koff, qf1, qf2);
      VtRegs vt;
      vt_issue(vt, lds_base + vaddr + voff);
      if (jt == diag) mask_tile(S, 32 * jt, qrow, h);
      float t1, t2;
      tile_max(S, c, t1, t2);
      maybe_rescale(t1, t2, m1, m2, l1, l2, acc1, acc2);
      bf16x8 p1a, p1b, p2a, p2b;
      exp_tile(S.s1, c, m1, l1, p1a, p1b);
      exp_tile(S.s2, c, m2, l2, p2a, p2b);
      vt_wait(vt);
      pv_tile(acc1, acc2, vt, p1a, p1b, p2a, p2b);
    }
    // next sub-tile: slot (jt + 1) / SPT % 2, position (jt + 1) % SPT within the tile
    const int nt = (jt + 1) / SPT, ns = (jt + 1) % SPT;
    koff = (nt & 1) * SLOT + ns * (32 * 128);
    voff = (nt & 1) * SLOT + ns * (32 * 64);
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
  const diffattn_saved& sv = a.saved;
  hipLaunchKernelGGL(fwd_bf16_kernel, dim3(static_cast<unsigned>(nblk)), dim3(NT), 0, s,
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
