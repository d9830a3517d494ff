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
// Work decomposition: one workgroup = 4 wavefronts = 256 query rows of one (b, h), one
// workgroup per CU and one wavefront per SIMD. A wavefront owns 64 query rows as two
// groups of 32; its four accumulators (2 maps x 2 groups, 128 x 32 fp32 each) live in
// the accumulation registers, everything else in the vector registers. When the blocks
// are few (short sequences), a workgroup takes 128 rows instead, one group of 32 per
// wavefront, which halves the longest key walk of a wavefront.
//  * Transposed score tiles S^T = K Q^T (32 keys x 32 queries per group) with
//    v_mfma_f32_32x32x16_bf16: each lane holds 16 scores of one query of each group, and
//    the key rows fed to the MFMA are permuted (bits 2 and 3 swapped) so that the score
//    registers, packed to bf16, are directly the B operand of O^T += V^T P^T. The two
//    groups share every K and V^T operand read from LDS.
//  * Software pipeline over 32-key sub-tiles j, in two half-steps whose matrix work and
//    vector work are independent, so the wavefront issues one map's softmax between the
//    other map's MFMAs:
//      X(j): MFMA  S2(j) = K2 Q2^T,  acc2 += V^T(j-1) P2(j-1)^T
//            VALU  softmax of S1(j) -> P1(j)
//      Y(j): MFMA  S1(j+1) = K1 Q1^T, acc1 += V^T(j) P1(j)^T
//            VALU  softmax of S2(j) -> P2(j)
//    A map's rescale (when its running max moved) happens between its half-steps, after
//    the last product into that accumulator and before the next.
//    With one group per wavefront the fast pass steps over whole 64-key tiles instead:
//    the tile's two 32-key halves fill the places of the two groups in the same
//    half-step schedule (two score tiles per map and half-step, twice the products
//    between dependent instructions), sharing the wavefront's one set of rows, Q
//    operands and accumulators. Products and row sums keep their key order, so the
//    result is the same bit for bit as on 32-key sub-tiles.
//  * Query rows are dealt to lanes with stride 4 NG (row 4 NG m + NG w + g of the
//    workgroup's rows for lane column m, wavefront w, group g; NG groups per wavefront),
//    so every wavefront and group sees the same key range: sub-tiles below the
//    workgroup's first row run without mask code and the 4 NG sub-tiles of the diagonal
//    block apply the integer predicate key <= query.
//  * K1, K2 and V tiles of 64 keys go from HBM straight into LDS (buffer loads with the
//    LDS as destination) in a ring of 4 slots, two tiles ahead, one barrier per tile.
//    Rows at or beyond N read as zero. V^T comes out of the row-major V tile with the
//    transposing read ds_read_b64_tr_b16; LDS swizzles keep every operand read free of
//    bank conflicts.
//  * No running row maximum on the fast path: each row's reference m is the exact maximum
//    of its first sub-tile, and the loop never branches. A row whose normaliser ends above
//    2^48 (kBad) is flagged; a second launch (the fixup pass) redoes only flagged blocks
//    on the checked path, where a row's partial sum above kThr moves its m to the exact
//    maximum and rescales. The decisions are per row, so every row's result depends on
//    its own scores only.
//  * Workgroups run longest-first, and consecutive workgroup ids take different heads so
//    that the tiles of one head land on the same XCD (ids are dealt to the 8 XCDs
//    round-robin) and share its L2.
#include "common.h"
#include "launch.h"

namespace diffattn {
namespace fwdbf16 {

#define LDS_AS __attribute__((address_space(3)))

constexpr int D = 64;
constexpr int DV = 128;
constexpr int NW = 4;          // wavefronts per workgroup (one per SIMD)
constexpr int NT = 64 * NW;    // threads per workgroup
constexpr int BR = 64 * NW;    // query rows per workgroup with two query groups per wave
constexpr int BC = 64;         // keys per LDS tile
constexpr int NSLOT = 4;       // LDS ring depth (tiles)

// LDS slot (bytes): K1 [BC keys][128 B] | K2 [BC keys][128 B] | V in 4 regions of 32
// channels, [BC keys][64 B] each.
constexpr int KTILE = BC * 128;
constexpr int VREG = BC * 64;
constexpr int K1_OFF = 0;
constexpr int K2_OFF = KTILE;
constexpr int V_OFF = 2 * KTILE;
constexpr int SLOT = 2 * KTILE + 4 * VREG;
constexpr int LDS_BYTES = NSLOT * SLOT;
constexpr int KBLK = BC / (8 * NW);   // 1 KB K1 (and K2) blocks per wave per tile
constexpr int VBLK = BC / (4 * NW);   // 1 KB V blocks per wave per tile
constexpr int DMA_PER_TILE = 2 * KBLK + VBLK;   // buffer loads per wave per tile
static_assert(DMA_PER_TILE == 8, "vmcnt immediates below assume 8 loads per tile");

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


// Issues this wave's share of tile `t` (keys t BC ..) into its ring slot; lane l's 16
// bytes land at block base + 16 l. K1 (and K2) block i holds key rows 8i .. 8i+7, V
// block i rows 16 (i % (BC/16)) .. +15 of region i / (BC/16); wave w moves blocks
// w + NW r. The source offsets are recomputed per tile (they would otherwise hold six
// vector registers through the loop).
struct HeadRsrc {
  u32x4 k1, k2, v;
};
// Buffer resource words (raw 32-bit buffer, no swizzle) for `bytes` bytes at `base`.
__device__ __forceinline__ u32x4 rsrc_words(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const u32x4 r = {static_cast<uint32_t>(a), static_cast<uint32_t>(a >> 32) & 0xffffu, bytes,
                   0x00020000u};
  return r;
}
// 16 bytes per lane from the buffer (offset voff) into LDS at m0 + 16 lane. Issued as
// assembly: the compiler would otherwise make every later LDS read wait for it. (m0 is
// reserved by the compiler and used by nothing else in this kernel.)
__device__ __forceinline__ void dma16(const u32x4& rs, uint32_t m0, int voff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(m0), "v"(voff), "s"(rs));
}

__device__ __forceinline__ void dma_tile(const HeadRsrc& rs, char* lds, int t, int wv, int lane) {
  const uint32_t base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((LDS_AS char*)lds)) +
                        (t % NSLOT) * SLOT;
  const int k0 = t * BC;
#pragma unroll
  for (int r = 0; r < KBLK; ++r) {
    const int row = 8 * (wv + NW * r) + (lane >> 3), pu = lane & 7;
    const int ko = (k0 + row) * (D * 2) + 16 * (pu ^ k_swz(row));
    const uint32_t dst = base + 1024 * (wv + NW * r);
    dma16(rs.k1, dst + K1_OFF, ko);
    dma16(rs.k2, dst + K2_OFF, ko);
  }
#pragma unroll
  for (int r = 0; r < VBLK; ++r) {
    const int i = wv + NW * r;
    const int region = i / (BC / 16);
    const int row = 16 * (i % (BC / 16)) + (lane >> 2), pc = lane & 3;
    const int vo = (k0 + row) * (DV * 2) + 64 * region + 16 * (pc ^ v_swz(row));
    dma16(rs.v, base + V_OFF + 1024 * i, vo);
  }
}

// Tile t resident in LDS for every wave: this wave's own loads of tile t are complete
// (only tile t + 1's, issued later, may still be in flight), then all waves meet.
__device__ __forceinline__ void tile_barrier(bool next_in_flight) {
  if (next_in_flight) {
    asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
  } else {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
  asm volatile("s_barrier" ::: "memory");
}

// ---------------------------------------------------------------------------------
// LDS operand reads are ordinary loads: the compiler tracks their completion and places
// the waits (reads issued as assembly would complete after the compiler believes their
// registers hold the data, and it may copy or reuse those registers meanwhile). The
// tile fills are assembly (dma16), so the compiler does not order these reads behind
// them; the tile barrier orders them instead.
template <int OFF>
__device__ __forceinline__ u32x4 ds_read_b128(int addr) {
  return *reinterpret_cast<const LDS_AS u32x4*>((LDS_AS char*)nullptr + addr + OFF);
}
typedef short s16x4 __attribute__((ext_vector_type(4)));
template <int OFF>
__device__ __forceinline__ u32x2 ds_read_tr16(int addr) {
  const s16x4 v =
      __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)((LDS_AS char*)nullptr + addr + OFF));
  return __builtin_bit_cast(u32x2, v);
}

// K operand of one map for one 32-key sub-tile: 4 channel blocks of 16.
struct KOps {
  u32x4 r[4];
};
template <int MAP_OFF>
__device__ __forceinline__ void k_issue(KOps& k, const int* kaddr, int off) {
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) k.r[kb] = ds_read_b128<MAP_OFF>(kaddr[kb] + off);
}
__device__ __forceinline__ bf16x8 k_operand(const KOps& k, int kb) {
  return __builtin_bit_cast(bf16x8, k.r[kb]);
}

// V^T operand of one k-step (16 keys) of a sub-tile: for region b, keys e = 0..3 of the
// lane's 8 and (4 rows further) e = 4..7.
struct VtHalf {
  u32x2 r[4][2];
};
template <int B, int T>
__device__ __forceinline__ void vt_issue_b(VtHalf& v, int addr) {
  v.r[B][0] = ds_read_tr16<V_OFF + VREG * B + 1024 * T>(addr);
  v.r[B][1] = ds_read_tr16<V_OFF + VREG * B + 1024 * T + 4 * 64>(addr);
}
template <int T>
__device__ __forceinline__ void vt_issue(VtHalf& v, int addr) {
  vt_issue_b<0, T>(v, addr); vt_issue_b<1, T>(v, addr);
  vt_issue_b<2, T>(v, addr); vt_issue_b<3, T>(v, addr);
}
__device__ __forceinline__ bf16x8 vt_operand(const VtHalf& v, int b) {
  const u32x4 x = {v.r[b][0][0], v.r[b][0][1], v.r[b][1][0], v.r[b][1][1]};
  return __builtin_bit_cast(bf16x8, x);
}

// ---------------------------------------------------------------------------------
// Softmax with a lazily moved reference m per row (scaled log2 domain): the weights of a
// sub-tile are p = exp2(s c - m) with the m the row already has, and the row's partial
// sum of them (its lane's 16 keys) is checked afterwards. Only when that partial exceeds
// kThr (always on the row's first sub-tile, while m is still kMInit) does the row take
// the slow path: m moves to the row's exact maximum if that is larger, the row's weights
// are recomputed, and its accumulator and normaliser are rescaled. Otherwise every
// weight is at most kThr. The decision and its effect are per row, so each row's result
// depends on its own scores only; the final O = acc / l and the log-sum-exp m + log2(l)
// do not depend on which m was used.
constexpr float kThr = 256.0f;
// Initial reference: finite, so that the first sub-tile's weights are +inf for visible
// keys (forcing the slow path) and exactly 0 for masked ones, and no NaN ever arises (the
// library is built assuming no NaNs, so the threshold test could not see one).
constexpr float kMInit = -1e30f;

// Per map and group: reference m, this lane's normaliser l (its 16 keys of each sub-tile)
// and the sub-tile's partial sum lp (added to l once the sub-tile is settled). The fast
// pass instead keeps two running sums, l and l2 (the first and last 8 of the lane's 16
// keys of every sub-tile), with no per-sub-tile partial; the normaliser is l + l2.
struct RowState {
  float m, l, lp, l2;
};

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

// Causal predicate on a sub-tile starting at key ks for query q: key > query -> -inf.
__device__ __forceinline__ void mask_scores(f32x16& s, int ks, int q, int h) {
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    if (ks + key_of(j, h) > q) s[j] = -INFINITY;
  }
}

// p = exp2(s c - m) for the 16 scores, packed to the bf16 operands of the two PV k-steps;
// returns their float32 sum (the row's partial normaliser, summed as in the fast loop).
__device__ __forceinline__ float exp_pack(const f32x16& s, float c, float m, bf16x8& pa,
                                          bf16x8& pb) {
  f32x8 x, y;
  float sum = 0.f;
#pragma unroll
  for (int e = 0; e < 8; e += 2) {
    x[e] = fast_exp2(fmaf(s[e], c, -m));
    x[e + 1] = fast_exp2(fmaf(s[e + 1], c, -m));
    sum += x[e] + x[e + 1];
  }
#pragma unroll
  for (int e = 0; e < 8; e += 2) {
    y[e] = fast_exp2(fmaf(s[8 + e], c, -m));
    y[e + 1] = fast_exp2(fmaf(s[9 + e], c, -m));
    sum += y[e] + y[e + 1];
  }
  pa = __builtin_convertvector(x, bf16x8);
  pb = __builtin_convertvector(y, bf16x8);
  return sum;
}

__device__ __forceinline__ bool over(float lp) { return !(lp <= kThr); }

// Fast path bound: a row keeps the reference m of its first sub-tile for the whole key
// range. Its normaliser (the sum of all its weights, so also a bound on every weight) may
// grow up to 2^48: the weights, their products with V and the accumulated sums then stay
// far inside float range, and their relative precision does not depend on the scale. A
// row whose normaliser ends above kBad (including +inf) is flagged for the fixup pass.
// The check runs once per row, after the loop.
constexpr float kBad = 281474976710656.0f;   // 2^48

// Accumulator registers pass through one vector register to be scaled (read, multiply,
// write back), so the rare slow path needs almost no vector registers of its own.
__device__ __forceinline__ float scale_acc(float x, float a) {
  float t;
  asm volatile("v_accvgpr_read_b32 %1, %0\n\t"
               "v_mul_f32 %1, %1, %2\n\t"
               "v_accvgpr_write_b32 %0, %1"
               : "+a"(x), "=&v"(t)
               : "v"(a));
  return x;
}

// Slow path for one group (see above): rows whose partial sum is over the threshold
// move m to their exact maximum when it is larger, recompute their weights and partial
// sum, and rescale their accumulator column and normaliser. Other rows keep everything
// (a = 1, their weights unchanged).
__device__ __forceinline__ void settle_row(const f32x16& s, float c, RowState& st, bf16x8& pa,
                                           bf16x8& pb, f32x16 (&acc)[4]) {
  const auto tr = __builtin_amdgcn_permlane32_swap(over(st.lp), over(st.lp), false, false);
  const bool trig = (tr[0] | tr[1]) != 0;
  const float t = max_halves(max16(s)) * c;
  const float mn = (trig && t > st.m) ? t : st.m;
  const float a = (mn == st.m) ? 1.0f : fast_exp2(st.m - mn);
  bf16x8 na, nb;
  const float nlp = exp_pack(s, c, mn, na, nb);
  if (trig) {
    pa = na;
    pb = nb;
    st.lp = nlp;
  }
  st.m = mn;
  st.l *= a;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[b][j] = scale_acc(acc[b][j], a);
  }
}

// S^T = K Q^T for one map and the NG query groups of a wave (4 NG MFMAs sharing the K
// operands). The score products are written as assembly so that their results stay in
// vector registers while the accumulator products (compiler-visible, below) keep theirs
// in the accumulation registers. Their consumers are fenced by s_guard. Destinations are
// early-clobber outputs: a product may not overwrite its own operands.
template <int NG>
__device__ __forceinline__ void qk(f32x16 (&S)[NG], const KOps& k, const bf16x8 (&q)[NG][4]) {
  const bf16x8 a0 = k_operand(k, 0);
#pragma unroll
  for (int g = 0; g < NG; ++g)
    asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(S[g]) : "v"(a0), "v"(q[g][0]));
#pragma unroll
  for (int kb = 1; kb < 4; ++kb) {
    const bf16x8 a = k_operand(k, kb);
#pragma unroll
    for (int g = 0; g < NG; ++g)
      asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(S[g]) : "v"(a), "v"(q[g][kb]));
  }
}
// One score product; FIRST starts the accumulation from zero. The destination must not
// share registers with the operands (early clobber): the product writes it while the
// operands are still being read.
__device__ __forceinline__ void qk_one(f32x16& S, const bf16x8& a, const bf16x8& q, bool first) {
  if (first) {
    asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(S) : "v"(a), "v"(q));
  } else {
    asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(S) : "v"(a), "v"(q));
  }
}
// Wait states between the last score product and any vector access to the scores (more
// than the 8-pass MFMA's result latency); every consumer depends on this statement.
__device__ __forceinline__ void s_guard(f32x16 (&S)[2]) {
  asm volatile("s_nop 7\n\ts_nop 4" : "+v"(S[0]), "+v"(S[1]));
}
__device__ __forceinline__ void s_guard(f32x16 (&S)[1]) {
  asm volatile("s_nop 7\n\ts_nop 4" : "+v"(S[0]));
}
// Orders the consumers of S after its products without waiting (the products are known
// to be complete).
__device__ __forceinline__ void s_anchor(f32x16 (&S)[2]) {
  asm volatile("" : "+v"(S[0]), "+v"(S[1]));
}

// Product order of a half-step's 12 NG slots: 8 NG accumulator products and 4 NG score
// products. With two query groups (NG = 2) the score products sit in the middle (X: slots
// 8..15; Y: the even slots 6..20), so the next half-step reads their results without
// wait states; they start 4 slots or more after their K operands are read (slot 2). With
// one group (NG = 1) they take the even slots 4..10, one accumulator product between two
// of them (each depends on the one before), and the next half-step waits for them
// (s_guard). qk_slot: the score product at slot k (kb = q / NG, group q % NG), or -1;
// pv_index: the accumulator product at slot k, in issue order (k-step t = pv / (4 NG),
// region (pv % (4 NG)) / NG, group pv % NG).
template <int NG, bool IS_X>
__host__ __device__ constexpr int qk_slot(int k) {
  if (NG == 1) return (k >= 4 && k <= 10 && (k & 1) == 0) ? (k - 4) / 2 : -1;
  if (IS_X) return (k >= 8 && k < 16) ? k - 8 : -1;
  return (k >= 6 && k <= 20 && (k & 1) == 0) ? (k - 6) / 2 : -1;
}
template <int NG, bool IS_X>
__host__ __device__ constexpr int pv_index(int k) {
  int n = 0;
  for (int i = 0; i < k; ++i) n += qk_slot<NG, IS_X>(i) < 0 ? 1 : 0;
  return n;
}
static_assert(pv_index<2, false>(24) == 16 && pv_index<2, true>(24) == 16, "16 products");
static_assert(pv_index<1, false>(12) == 8 && pv_index<1, true>(12) == 8, "8 products");
// X half-steps refill V^T region b of k-step t behind the slot of the last accumulator
// product that reads it. NG = 2: t = 0 behind slots 8..11 (its products are slots 0..7),
// t = 1 behind slots 18, 20, 22 and 23 (its products are slots 16..23, two per region).
// NG = 1: t = 0 behind slots 4..7 (its products are slots 0..3), t = 1 behind slots 6, 8,
// 10 and 11 (its products are slots 5, 7, 9 and 11).
template <int NG>
__host__ __device__ constexpr int vt_read_slot(int t, int b) {
  if (NG == 1) return t == 0 ? 4 + b : (b < 3 ? 6 + 2 * b : 11);
  return t == 0 ? 8 + b : (b < 3 ? 18 + 2 * b : 23);
}
// Slot of the first step of softmax pair pr (16 pairs over 24 slots with two groups, 8
// over 12 with one); its five steps take that slot and the four after it.
template <int NG>
__host__ __device__ constexpr int pair_start(int pr) { return NG == 2 ? (pr * 5) / 4 : pr; }
static_assert(pair_start<2>(15) + 4 < 24 && pair_start<1>(7) + 4 < 12, "pairs end in time");

// Keeps the accumulators in the accumulation registers across the loop.
__device__ __forceinline__ void acc_pin(f32x16 (&acc)[2][4]) {
  asm volatile(""
               : "+a"(acc[0][0]), "+a"(acc[0][1]), "+a"(acc[0][2]), "+a"(acc[0][3]),
                 "+a"(acc[1][0]), "+a"(acc[1][1]), "+a"(acc[1][2]), "+a"(acc[1][3]));
}
__device__ __forceinline__ void acc_pin(f32x16 (&acc)[1][4]) {
  asm volatile("" : "+a"(acc[0][0]), "+a"(acc[0][1]), "+a"(acc[0][2]), "+a"(acc[0][3]));
}

template <bool B>
struct Flag {
  static constexpr bool value = B;
};
template <int N>
struct Int {
  static constexpr int value = N;
};
// Calls f(Int<I>{}) for I = A .. B-1, in order, each with a compile-time index.
template <int A, int B, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (A < B) {
    f(Int<A>{});
    static_for<A + 1, B>(f);
  }
}

// LDS byte offsets of sub-tile j's K rows and V rows relative to slot 0, sub-tile 0.
__device__ __forceinline__ int k_off(int j) { return ((j >> 1) % NSLOT) * SLOT + (j & 1) * (32 * 128); }
__device__ __forceinline__ int v_off(int j) { return ((j >> 1) % NSLOT) * SLOT + (j & 1) * (32 * 64); }

// SAFE = false: the fast pass (every row block). SAFE = true: the fixup pass, which
// returns at once unless the fast pass flagged a row of its block in `flags` (4 NG words
// per block, block (b h, qb) at words 4 NG (bh nqb + qb) ..: bit m of word NG w + g is the
// row of lane column m, group g of wave w), and then redoes the block on the checked path
// and rewrites exactly the flagged rows. NG: query groups of 32 rows per wave (2: 256-row
// blocks; 1: 128-row blocks, see fwd_bf16_groups). With one group the fast pass does that
// fixup itself, in the same launch, and the SAFE instance is not used.
template <bool SAFE, int NG>
__global__ void __launch_bounds__(NT, 1) fwd_bf16_kernel(
    const bf16_t* __restrict__ q1, const bf16_t* __restrict__ q2,
    const bf16_t* __restrict__ k1, const bf16_t* __restrict__ k2,
    const bf16_t* __restrict__ v, const diffattn_lambda_state* __restrict__ lamst,
    const float* __restrict__ rms_w, bf16_t* __restrict__ out, float* __restrict__ sv_lse1,
    float* __restrict__ sv_lse2, float* __restrict__ sv_o1, float* __restrict__ sv_o2,
    float* __restrict__ sv_rstd, uint32_t* __restrict__ flags, int BH, int H, int N, int nqb,
    float eps, int out_bnh, int G) {
  extern __shared__ __attribute__((aligned(16))) char lds[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int m = lane & 31;
  const int h = lane >> 5;

  // Longest-first over query blocks; consecutive ids walk the heads.
  const int bid = blockIdx.x;
  const int bh = bid % BH;
  const int qb = nqb - 1 - bid / BH;
  constexpr int RB = 32 * NW * NG;   // query rows per workgroup
  constexpr int FW = NW * NG;        // row-flag words per block
  const int q0 = qb * RB;
  // Workgroup row of lane column m, group g of this wave: rows are dealt with stride
  // NW NG, so every wave and group sees the same key range.
  auto row_of = [&](int g) __attribute__((always_inline)) { return q0 + FW * m + NG * wv + g; };
  const int64_t hoff = static_cast<int64_t>(bh) * N;

  // K/V head of this query head (grouped-query attention: G query heads per K/V head).
  const int64_t kvoff = (static_cast<int64_t>(bh / H) * (H / G) + (bh % H) / G) * N;
  HeadRsrc rs;
  rs.k1 = rsrc_words(k1 + kvoff * D, N * D * 2);
  rs.k2 = rsrc_words(k2 + kvoff * D, N * D * 2);
  rs.v = rsrc_words(v + kvoff * DV, N * DV * 2);

  // Every wave walks the same sub-tiles: keys 0 .. q0 + RB - 1 (rows beyond N are
  // zero-filled and masked). The first jd are wholly below the block's first row.
  const int n_sub = (q0 + RB) / 32;
  const int n_tiles = n_sub / 2;
  const int jd = q0 / 32;

  // Queries of this lane: group g holds workgroup row 8 m + 2 wv + g.
  bf16x8 qf1[NG][4], qf2[NG][4];
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    const int q = min(row_of(g), N - 1);
    const bf16_t* Q1 = q1 + (hoff + q) * D;
    const bf16_t* Q2 = q2 + (hoff + q) * D;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      qf1[g][kb] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(Q1 + 16 * kb + 8 * h));
      qf2[g][kb] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(Q2 + 16 * kb + 8 * h));
    }
  }

  // LDS-relative byte addresses of the operands (slot 0, sub-tile 0).
  const int lds_base = static_cast<int>(reinterpret_cast<uintptr_t>((LDS_AS char*)lds));
  int ka[4];
  {
    const int kr = perm_row(m);
    const int ks = k_swz(kr);
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) ka[kb] = lds_base + kr * 128 + 16 * ((2 * kb + h) ^ ks);
  }
  int va;
  {
    const int G = lane >> 4, j = (lane >> 2) & 3, a = lane & 3;
    const int row = 8 * (G >> 1) + j;
    const int cp = 2 * (G & 1) + (a >> 1);
    va = lds_base + row * 64 + 16 * (cp ^ v_swz(row)) + 8 * (a & 1);
  }

  const float c = kLog2e / 8.0f;  // log2(e) / sqrt(64)
  RowState st1[NG], st2[NG];
  f32x16 acc1[NG][4], acc2[NG][4];
  f32x16 S1[NG], S2[NG];
  bf16x8 P1[NG][2], P2[NG][2];
  // V^T operands of the sub-tile the next PV products use.
  VtHalf vt[2];
  // Per group: this lane's row left the fast path's bound on some sub-tile (fast pass),
  // or was flagged by it (fixup pass).
  uint32_t bad[NG] = {};
  if constexpr (SAFE) {
    const uint32_t* f = flags + FW * (static_cast<int64_t>(bh) * nqb + qb);
    uint32_t any = 0;
#pragma unroll
    for (int i = 0; i < FW; ++i) any |= f[i];
    if (__builtin_amdgcn_readfirstlane(any) == 0) return;
#pragma unroll
    for (int g = 0; g < NG; ++g) bad[g] = (f[NG * wv + g] >> m) & 1u;
  }

  // One half-step, in a fixed order: 24 products (16 accumulator products acc += V^T P^T
  // and 8 score products S_next = K Q^T in the middle, see qk_slot), each followed by a
  // slice of the softmax of
  // S_cur (sub-tile j, for accumulator acc_cur), software-pipelined over pairs of scores
  // started every 1.25 slots: fma (scale, subtract m), one exp2, the other exp2, pack to
  // bf16, row sum. At most two transcendentals fall behind one product, and no v_dot2
  // (which does not co-execute with the matrix core); each step's results are anchored
  // so the compiler cannot gather the steps of many slots in one place. The matrix core
  // thus always has a product queued while the vector unit works. CHECK (fixup pass):
  // the sub-tile's row sums are tested against kThr and the rare slow path may follow;
  // otherwise (fast pass) the weights go straight into the running row sums, nothing is
  // tested inside the loop and it has no branch at all. IS_X: the X half-step, which
  // also prefetches V^T(j) (used by Y(j) and again by X(j + 1)); the Y half-step of an
  // odd sub-tile holds the tile barrier.
  auto half = [&](auto masked, auto is_x, auto check, int j, f32x16 (&acc)[NG][4],
                  const bf16x8 (&Pin)[NG][2], f32x16 (&S_next)[NG], const bf16x8 (&qf)[NG][4],
                  int k_sub, f32x16 (&S_cur)[NG], const bf16x8 (&qf_cur)[NG][4],
                  RowState (&st)[NG], bf16x8 (&Pout)[NG][2], f32x16 (&acc_cur)[NG][4])
      __attribute__((always_inline)) {
    constexpr bool MASKED = decltype(masked)::value;
    constexpr bool IS_X = decltype(is_x)::value;
    constexpr bool CHECK = decltype(check)::value;
    constexpr int KN_OFF = IS_X ? K2_OFF : K1_OFF;   // map of S_next
    constexpr int KC_OFF = IS_X ? K1_OFF : K2_OFF;   // map of S_cur
    KOps kop;
    float y[32];
    // Packed weights as separate 32-bit words: kept in a u32x4 and updated element by
    // element, the dot products below were compiled to read element 0 each time.
    uint32_t pw[NG][2][4];
    // Row sums: the sub-tile's partial (fixup pass), or the running sums (fast pass).
    float ssum[NG][2];
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      ssum[g][0] = CHECK ? 0.f : st[g].l;
      ssum[g][1] = CHECK ? 0.f : st[g].l2;
    }
    bool slow = false;
    auto slot = [&](auto kc) __attribute__((always_inline)) {
      constexpr int k = decltype(kc)::value;
      // ---- the k-th product (score product q or accumulator product pv, see qk_slot)
      constexpr int q = qk_slot<NG, IS_X>(k);
      if constexpr (q < 0) {
        constexpr int pv = pv_index<NG, IS_X>(k);
        constexpr int t = pv / (4 * NG), b = (pv % (4 * NG)) / NG, g = pv % NG;
        acc[g][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vt_operand(vt[t], b), Pin[g][t],
                                                             acc[g][b], 0, 0, 0);
      } else {
        constexpr int kb = q / NG, g = q % NG;
        qk_one(S_next[g], k_operand(kop, kb), qf[g][kb], kb == 0);
      }
      __builtin_amdgcn_sched_barrier(0);
      // ---- work placed behind it
      // S_cur came from the previous half-step's score products, the last of them 3 or
      // more slots before that half-step ended: more than the result latency.
      if constexpr (k == 0) {
        if constexpr (NG == 2) {
          s_anchor(S_cur);
        } else {
          s_guard(S_cur);
        }
      }
      if constexpr (k == 2) k_issue<KN_OFF>(kop, ka, k_off(k_sub));
      static_for<0, 8 * NG>([&](auto pc) __attribute__((always_inline)) {
        constexpr int pr = decltype(pc)::value;
        constexpr int sa = pair_start<NG>(pr);
        constexpr int g = pr >> 3, e = 2 * (pr & 7);
        if constexpr (k == sa) {          // scale and subtract the reference
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            float sv = S_cur[g][e + i];
            if (MASKED && 32 * j + key_of(e + i, h) > row_of(g)) sv = -INFINITY;
            y[16 * g + e + i] = fmaf(sv, c, -st[g].m);
          }
          asm volatile("" : "+v"(y[16 * g + e]), "+v"(y[16 * g + e + 1]));
        }
        if constexpr (k == sa + 1) {      // exp2 of the first
          y[16 * g + e] = fast_exp2(y[16 * g + e]);
          asm volatile("" : "+v"(y[16 * g + e]));
        }
        if constexpr (k == sa + 2) {      // exp2 of the second
          y[16 * g + e + 1] = fast_exp2(y[16 * g + e + 1]);
          asm volatile("" : "+v"(y[16 * g + e + 1]));
        }
        if constexpr (k == sa + 3) {      // pack to bf16
          pw[g][e >> 3][(e & 7) >> 1] = pack_bf16x2(y[16 * g + e], y[16 * g + e + 1]);
          asm volatile("" : "+v"(pw[g][e >> 3][(e & 7) >> 1]));
        }
        if constexpr (k == sa + 4) {      // row sum
          ssum[g][e >> 3] += y[16 * g + e] + y[16 * g + e + 1];
          asm volatile("" : "+v"(ssum[g][e >> 3]));
        }
      });
      // V^T(j) for Y(j) and X(j + 1): two transposing reads per slot (they do not overlap
      // the matrix core well when bunched), each behind the last accumulator product that
      // reads the registers it refills (vt_read_slot).
      if constexpr (IS_X) {
        static_for<0, 8>([&](auto ic) __attribute__((always_inline)) {
          constexpr int t = decltype(ic)::value >> 2, b = decltype(ic)::value & 3;
          if constexpr (k == vt_read_slot<NG>(t, b)) vt_issue_b<b, t>(vt[t], va + v_off(j));
        });
      }
      __builtin_amdgcn_sched_barrier(0);
    };
    slot(Int<0>{});
    slot(Int<1>{});
    if (!IS_X && (j & 1) && ((j + 1) >> 1) < n_tiles) {
      // tile of sub-tile j + 1 resident before its K1 rows are read (slot 2)
      const int u = (j + 1) >> 1;
      tile_barrier(u + 1 < n_tiles);
      if (u + 2 < n_tiles) dma_tile(rs, lds, u + 2, wv, lane);
    }
    static_for<2, 12 * NG>(slot);
    if constexpr (CHECK) {
#pragma unroll
      for (int g = 0; g < NG; ++g) st[g].lp = ssum[g][0] + ssum[g][1];
      bool o = false;
#pragma unroll
      for (int g = 0; g < NG; ++g) o = o || over(st[g].lp);
      slow = __any(o);
    } else {
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        st[g].l = ssum[g][0];
        st[g].l2 = ssum[g][1];
      }
    }
#pragma unroll
    for (int g = 0; g < NG; ++g) {
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const u32x4 w4 = {pw[g][hf][0], pw[g][hf][1], pw[g][hf][2], pw[g][hf][3]};
        Pout[g][hf] = __builtin_bit_cast(bf16x8, w4);
      }
    }
    if constexpr (CHECK) {
      if (__builtin_expect(slow, 0)) {
        // Slow path: S_cur again from its K rows (still resident) and Q.
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        KOps kc;
        k_issue<KC_OFF>(kc, ka, k_off(j));
        f32x16 Sr[NG];
        qk(Sr, kc, qf_cur);
        s_guard(Sr);
#pragma unroll
        for (int g = 0; g < NG; ++g) {
          if (MASKED) mask_scores(Sr[g], 32 * j, row_of(g), h);
          settle_row(Sr[g], c, st[g], Pout[g][0], Pout[g][1], acc_cur[g]);
        }
      }
    }
    if constexpr (CHECK) {
#pragma unroll
      for (int g = 0; g < NG; ++g) st[g].l += st[g].lp;
    }
  };

  auto step = [&](int j, auto masked, auto check) __attribute__((always_inline)) {
    DIFFATTN_DEBUG_BARRIER();   // every wave runs the same sub-tiles
    // X(j): acc2 += V^T(j-1) P2(j-1); S2(j); softmax of S1(j) -> P1.
    half(masked, Flag<true>{}, check, j, acc2, P2, S2, qf2, j, S1, qf1, st1, P1, acc1);
    // Y(j): acc1 += V^T(j) P1(j); S1(j+1); softmax of S2(j) -> P2.
    half(masked, Flag<false>{}, check, j, acc1, P1, S1, qf1, j + 1, S2, qf2, st2, P2, acc2);
  };

  // The key loop over every sub-tile, from loading tile 0 to the last product. The fast
  // pass takes each row's reference m from the exact maximum of its first sub-tile (both
  // maps' first score tiles are formed here once for that) and never branches; the fixup
  // (CHECK) checks every sub-tile.
  auto run = [&](auto check) __attribute__((always_inline)) {
    constexpr bool CHECK = decltype(check)::value;
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      st1[g] = RowState{kMInit, 0.f, 0.f, 0.f};
      st2[g] = RowState{kMInit, 0.f, 0.f, 0.f};
#pragma unroll
      for (int b = 0; b < 4; ++b) {
#pragma unroll
        for (int j = 0; j < 16; ++j) acc1[g][b][j] = acc2[g][b][j] = 0.f;
      }
    }
    acc_pin(acc1);
    acc_pin(acc2);
    // Tiles 0 and 1 on their way, tile 0 resident, tile 2 on its way; S1(0).
    dma_tile(rs, lds, 0, wv, lane);
    if (n_tiles > 1) dma_tile(rs, lds, 1, wv, lane);
    tile_barrier(n_tiles > 1);
    if (n_tiles > 2) dma_tile(rs, lds, 2, wv, lane);
    {
      KOps kop;
      k_issue<K1_OFF>(kop, ka, k_off(0));
      qk(S1, kop, qf1);
    }
    if constexpr (!CHECK) {
      // Reference m of both maps: exact row maxima of sub-tile 0 (masked where the block
      // starts at key 0).
      KOps kop;
      k_issue<K2_OFF>(kop, ka, k_off(0));
      f32x16 T2[NG];
      qk(T2, kop, qf2);
      s_guard(S1);
      s_guard(T2);
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        f32x16 a = S1[g], b = T2[g];
        if (jd == 0) {
          mask_scores(a, 0, row_of(g), h);
          mask_scores(b, 0, row_of(g), h);
        }
        st1[g].m = max_halves(max16(a)) * c;
        st2[g].m = max_halves(max16(b)) * c;
      }
    }
#pragma unroll
    for (int g = 0; g < NG; ++g) P2[g][0] = P2[g][1] = bf16x8{};
    // X(0) multiplies tile 0's V (finite) by P2 = 0.
    vt_issue<0>(vt[0], va + v_off(0));
    vt_issue<1>(vt[1], va + v_off(0));
    for (int j = 0; j < jd; ++j) step(j, Flag<false>{}, check);
    for (int j = jd; j < n_sub; ++j) step(j, Flag<true>{}, check);
    if constexpr (!CHECK) {
      // Rows whose normaliser left the fast path's bound (either lane half of the row).
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        st1[g].l += st1[g].l2;
        st2[g].l += st2[g].l2;
        bad[g] = static_cast<uint32_t>(st1[g].l > kBad || st2[g].l > kBad);
      }
    }
    // Drain: acc2 += V^T(last) P2(last); vt holds V^T(last).
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int b = 0; b < 4; ++b) {
#pragma unroll
        for (int g = 0; g < NG; ++g)
          acc2[g][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vt_operand(vt[t], b), P2[g][t],
                                                               acc2[g][b], 0, 0, 0);
      }
    }
  };

  // One group per wave (128-row blocks), fast pass: 64-key steps. The two 32-key halves s
  // of tile j take the part the two query groups take with NG = 2 (same slot order: 16
  // accumulator products and 8 score products per half-step, 16 softmax pairs), but they
  // share the wave's 32 rows: one Q operand set, one accumulator set, one row state. Each
  // step carries twice the independent work of a 32-key sub-tile, which covers the
  // latencies a 32-key step leaves exposed. Products, row-sum additions and the reference
  // maximum (the first 32 keys) come in the same key order as on 32-key sub-tiles, so
  // the results are the same bit for bit.
  // Accumulator product pv of a half-step: key half pv / 8, k-step (pv / 4) % 2, region
  // pv % 4 (key order within each accumulator).
  auto half_kh = [&](auto masked, auto is_x, int j, f32x16 (&acc)[4],
                     const bf16x8 (&Pin)[2][2], f32x16 (&S_next)[2], const bf16x8 (&qf)[4],
                     int k_step, f32x16 (&S_cur)[2], RowState& st, bf16x8 (&Pout)[2][2],
                     VtHalf (&vk)[2][2]) __attribute__((always_inline)) {
    constexpr bool MASKED = decltype(masked)::value;
    constexpr bool IS_X = decltype(is_x)::value;
    constexpr int KN_OFF = IS_X ? K2_OFF : K1_OFF;   // map of S_next
    KOps kop[2];
    float y[32];
    uint32_t pw[2][2][4];
    float ssum[2] = {st.l, st.l2};
    auto slot = [&](auto kc) __attribute__((always_inline)) {
      constexpr int k = decltype(kc)::value;
      constexpr int q = qk_slot<2, IS_X>(k);
      if constexpr (q < 0) {
        constexpr int pv = pv_index<2, IS_X>(k);
        constexpr int s = pv / 8, t = (pv / 4) % 2, b = pv % 4;
        acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vt_operand(vk[s][t], b), Pin[s][t],
                                                         acc[b], 0, 0, 0);
        // X refills the operand it just consumed with V^T(j), which Y(j) and X(j + 1) use.
        if constexpr (IS_X) vt_issue_b<b, t>(vk[s][t], va + v_off(2 * j + s));
      } else {
        constexpr int kb = q / 2, s = q % 2;
        qk_one(S_next[s], k_operand(kop[s], kb), qf[kb], kb == 0);
      }
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (k == 0) s_anchor(S_cur);
      if constexpr (k == 2) {
        k_issue<KN_OFF>(kop[0], ka, k_off(2 * k_step));
        k_issue<KN_OFF>(kop[1], ka, k_off(2 * k_step + 1));
      }
      static_for<0, 16>([&](auto pc) __attribute__((always_inline)) {
        constexpr int pr = decltype(pc)::value;
        constexpr int sa = pair_start<2>(pr);
        constexpr int s = pr >> 3, e = 2 * (pr & 7);
        if constexpr (k == sa) {          // scale and subtract the reference
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            float sv = S_cur[s][e + i];
            if (MASKED && 64 * j + 32 * s + key_of(e + i, h) > row_of(0)) sv = -INFINITY;
            y[16 * s + e + i] = fmaf(sv, c, -st.m);
          }
          asm volatile("" : "+v"(y[16 * s + e]), "+v"(y[16 * s + e + 1]));
        }
        if constexpr (k == sa + 1) {      // exp2 of the first
          y[16 * s + e] = fast_exp2(y[16 * s + e]);
          asm volatile("" : "+v"(y[16 * s + e]));
        }
        if constexpr (k == sa + 2) {      // exp2 of the second
          y[16 * s + e + 1] = fast_exp2(y[16 * s + e + 1]);
          asm volatile("" : "+v"(y[16 * s + e + 1]));
        }
        if constexpr (k == sa + 3) {      // pack to bf16
          pw[s][e >> 3][(e & 7) >> 1] = pack_bf16x2(y[16 * s + e], y[16 * s + e + 1]);
          asm volatile("" : "+v"(pw[s][e >> 3][(e & 7) >> 1]));
        }
        if constexpr (k == sa + 4) {      // row sum
          ssum[e >> 3] += y[16 * s + e] + y[16 * s + e + 1];
          asm volatile("" : "+v"(ssum[e >> 3]));
        }
      });
      __builtin_amdgcn_sched_barrier(0);
    };
    slot(Int<0>{});
    slot(Int<1>{});
    if (!IS_X && j + 1 < n_tiles) {
      // tile j + 1 resident before its K1 rows are read (slot 2)
      tile_barrier(j + 2 < n_tiles);
      if (j + 3 < n_tiles) dma_tile(rs, lds, j + 3, wv, lane);
    }
    static_for<2, 24>(slot);
    st.l = ssum[0];
    st.l2 = ssum[1];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const u32x4 w4 = {pw[s][hf][0], pw[s][hf][1], pw[s][hf][2], pw[s][hf][3]};
        Pout[s][hf] = __builtin_bit_cast(bf16x8, w4);
      }
    }
  };

  auto run_kh = [&]() __attribute__((always_inline)) {
    st1[0] = RowState{kMInit, 0.f, 0.f, 0.f};
    st2[0] = RowState{kMInit, 0.f, 0.f, 0.f};
#pragma unroll
    for (int b = 0; b < 4; ++b) {
#pragma unroll
      for (int i = 0; i < 16; ++i) acc1[0][b][i] = acc2[0][b][i] = 0.f;
    }
    acc_pin(acc1);
    acc_pin(acc2);
    f32x16 SA[2], SB[2];           // scores of the two key halves, maps 1 and 2
    bf16x8 PA[2][2], PB[2][2];     // packed weights [half][k-step]
    VtHalf vk[2][2];               // V^T of the current tile [half][k-step]
    dma_tile(rs, lds, 0, wv, lane);
    if (n_tiles > 1) dma_tile(rs, lds, 1, wv, lane);
    tile_barrier(n_tiles > 1);
    if (n_tiles > 2) dma_tile(rs, lds, 2, wv, lane);
    {
      KOps k0, k1;
      k_issue<K1_OFF>(k0, ka, k_off(0));
      k_issue<K1_OFF>(k1, ka, k_off(1));
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        qk_one(SA[0], k_operand(k0, kb), qf1[0][kb], kb == 0);
        qk_one(SA[1], k_operand(k1, kb), qf1[0][kb], kb == 0);
      }
    }
    {
      // Reference m of both maps: exact row maxima of the first 32 keys (masked where the
      // block starts at key 0).
      KOps kop;
      k_issue<K2_OFF>(kop, ka, k_off(0));
      f32x16 T2[1];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) qk_one(T2[0], k_operand(kop, kb), qf2[0][kb], kb == 0);
      s_guard(SA);
      s_guard(T2);
      f32x16 a = SA[0], b = T2[0];
      if (jd == 0) {
        mask_scores(a, 0, row_of(0), h);
        mask_scores(b, 0, row_of(0), h);
      }
      st1[0].m = max_halves(max16(a)) * c;
      st2[0].m = max_halves(max16(b)) * c;
    }
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      PB[s][0] = PB[s][1] = bf16x8{};
      // X(0) multiplies tile 0's V (finite) by P2 = 0.
      vt_issue<0>(vk[s][0], va + v_off(s));
      vt_issue<1>(vk[s][1], va + v_off(s));
    }
    auto step_kh = [&](int jj, auto msk) __attribute__((always_inline)) {
      DIFFATTN_DEBUG_BARRIER();   // every wave runs the same steps
      // X(j): acc2 += V^T(j-1) P2(j-1); S2(j); softmax of S1(j) -> P1.
      half_kh(msk, Flag<true>{}, jj, acc2[0], PB, SB, qf2[0], jj, SA, st1[0], PA, vk);
      // Y(j): acc1 += V^T(j) P1(j); S1(j+1); softmax of S2(j) -> P2.
      half_kh(msk, Flag<false>{}, jj, acc1[0], PA, SA, qf1[0], jj + 1, SB, st2[0], PB, vk);
    };
    for (int jj = 0; jj < jd / 2; ++jj) step_kh(jj, Flag<false>{});
    for (int jj = jd / 2; jj < n_tiles; ++jj) step_kh(jj, Flag<true>{});
    st1[0].l += st1[0].l2;
    st2[0].l += st2[0].l2;
    bad[0] = static_cast<uint32_t>(st1[0].l > kBad || st2[0].l > kBad);
    // Drain: acc2 += V^T(last) P2(last).
#pragma unroll
    for (int s = 0; s < 2; ++s) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int b = 0; b < 4; ++b)
          acc2[0][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vt_operand(vk[s][t], b),
                                                               PB[s][t], acc2[0][b], 0, 0, 0);
      }
    }
  };

  // Epilogue per group: combine the lane halves' normalisers, form O, RMSNorm, scale,
  // store. ONLY_BAD: only rows whose flag is set (after the safe re-run). The lane holds
  // 64 of its row's 128 channels: 32 b + 8 jg + 4 h + e for region b, chunk jg, e < 4.
  // O = acc1 / l1 - lambda acc2 / l2 is formed once and kept in vector registers, which
  // the loop no longer needs; Y = O times one per-row factor (1 - lambda_init) rstd,
  // times w when given.
  // The fast pass stages its Y rows in LDS and stores them as whole rows. Each wave has
  // 8 NG KiB there (32 NG rows of 256 B) in the two ring slots after the last tile's slot:
  // once a wave has passed the last tile barrier, every wave is past its last read of any
  // slot but the last tile's, and no tile load is in flight.
  constexpr int STAGE_W = 32 * NG * DV * 2;   // bytes per wave
  constexpr int WPS = SLOT / STAGE_W;         // waves per slot
  static_assert(NW <= 2 * WPS, "the staging areas fit two ring slots");
  const int stage = lds_base + ((n_tiles + wv / WPS) % NSLOT) * SLOT + (wv % WPS) * STAGE_W;
  const float lam = lamst->lambda_f;
  const float gsc = lamst->one_minus_init_f;
  const int hh = bh % H;
  auto epilogue = [&](auto only_bad) __attribute__((always_inline)) {
  constexpr bool STAGED = !decltype(only_bad)::value;
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    const bool row_bad = (bad[g] | static_cast<uint32_t>(__shfl_xor(static_cast<int>(bad[g]), 32))) != 0;
    float l1 = st1[g].l + __shfl_xor(st1[g].l, 32);
    float l2 = st2[g].l + __shfl_xor(st2[g].l, 32);
    const float il1 = 1.0f / l1, il2 = 1.0f / l2;
    const float c2 = lam * il2;
    float o[64];
    float ss[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int b = 0; b < 4; ++b) {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        // Two rounded products (not contracted into one fused multiply-add), then their
        // difference: identical maps with lambda = 1 give exactly zero, as in exact
        // arithmetic.
#pragma clang fp contract(off)
        const float x = acc1[g][b][j] * il1 - acc2[g][b][j] * c2;
        o[16 * b + j] = x;
        ss[j & 3] = fmaf(x, x, ss[j & 3]);
      }
    }
    float sst = (ss[0] + ss[1]) + (ss[2] + ss[3]);
    sst += __shfl_xor(sst, 32);
    const float rstd = 1.0f / sqrtf(sst * (1.0f / DV) + eps);
    const float sc = gsc * rstd;
    const int qr = row_of(g);
    if constexpr (STAGED) {
      // Row 2 m + g of the wave's staging area; its 16-byte unit u (channels 8 u .. 8 u + 7)
      // sits at u ^ (m % 16), so the 32 rows one write touches spread over the banks.
      const int sr = stage + (NG * m + g) * (DV * 2) + 8 * h;
      const float* W = rms_w ? rms_w + hh * DV + 4 * h : nullptr;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int b = i >> 2, jg = i & 3;
        const float* x = o + 16 * b + 4 * jg;
        f32x4 y = {sc * x[0], sc * x[1], sc * x[2], sc * x[3]};
        if (W) {
          const f32x4 wv4 = *reinterpret_cast<const f32x4*>(W + 8 * i);
          y = f32x4{sc * (wv4[0] * x[0]), sc * (wv4[1] * x[1]), sc * (wv4[2] * x[2]),
                    sc * (wv4[3] * x[3])};
        }
        const u32x2 pk = {pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
        *reinterpret_cast<LDS_AS u32x2*>((LDS_AS char*)nullptr + sr + 16 * ((4 * b + jg) ^ (m & 15))) = pk;
      }
    }
    if (qr < N && (STAGED || row_bad)) {
      // Y row of (b, h, qr): [B, H, N, 2d], or [B, N, H, 2d] with out_bnh.
      const int64_t yrow = out_bnh ? (static_cast<int64_t>(bh / H) * N + qr) * H + hh : hoff + qr;
      bf16_t* Y = out + yrow * DV + 4 * h;
      if (STAGED) {
      } else if (rms_w) {
        const float* W = rms_w + hh * DV + 4 * h;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int b = i >> 2, jg = i & 3;
          const float* x = o + 16 * b + 4 * jg;
          const f32x4 wv4 = *reinterpret_cast<const f32x4*>(W + 8 * i);
          const u32x2 pk = {pack_bf16x2(sc * (wv4[0] * x[0]), sc * (wv4[1] * x[1])),
                            pack_bf16x2(sc * (wv4[2] * x[2]), sc * (wv4[3] * x[3]))};
          *reinterpret_cast<u32x2*>(Y + 8 * i) = pk;
        }
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int b = i >> 2, jg = i & 3;
          const float* x = o + 16 * b + 4 * jg;
          const u32x2 pk = {pack_bf16x2(sc * x[0], sc * x[1]), pack_bf16x2(sc * x[2], sc * x[3])};
          *reinterpret_cast<u32x2*>(Y + 8 * i) = pk;
        }
      }
      if (sv_o1) {
        // Training saves: O1 = acc1 / l1, O2 = acc2 / l2, the log-sum-exps and rstd.
        float* S1 = sv_o1 + (hoff + qr) * DV + 4 * h;
        float* S2 = sv_o2 + (hoff + qr) * DV + 4 * h;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int b = i >> 2, jg = i & 3;
          const f32x4 a = {acc1[g][b][4 * jg] * il1, acc1[g][b][4 * jg + 1] * il1,
                           acc1[g][b][4 * jg + 2] * il1, acc1[g][b][4 * jg + 3] * il1};
          const f32x4 bb = {acc2[g][b][4 * jg] * il2, acc2[g][b][4 * jg + 1] * il2,
                            acc2[g][b][4 * jg + 2] * il2, acc2[g][b][4 * jg + 3] * il2};
          *reinterpret_cast<f32x4*>(S1 + 8 * i) = a;
          *reinterpret_cast<f32x4*>(S2 + 8 * i) = bb;
        }
        if (h == 0) {
          // lse_k = ln(sum_j exp(S_kj)) = (m_k + log2 l_k) ln 2, m_k in the scaled log2
          // domain.
          sv_lse1[hoff + qr] = (st1[g].m + __log2f(l1)) * kLn2;
          sv_lse2[hoff + qr] = (st2[g].m + __log2f(l2)) * kLn2;
          sv_rstd[hoff + qr] = rstd;
        }
      }
    }
  }
  if constexpr (STAGED) {
    // The wave's 32 NG rows as whole rows: 4 rows of 256 B per instruction, 16 B per lane.
#pragma unroll
    for (int i = 0; i < 8 * NG; ++i) {
      const int r = 4 * i + (lane >> 4), c = lane & 15;
      const int rm = r / NG, rg = r % NG;   // lane column and group of staged row r
      const u32x4 v = *reinterpret_cast<const LDS_AS u32x4*>(
          (LDS_AS char*)nullptr + stage + r * (DV * 2) + 16 * (c ^ (rm & 15)));
      const int qr = q0 + FW * rm + NG * wv + rg;
      if (qr < N) {
        const int64_t yrow = out_bnh ? (static_cast<int64_t>(bh / H) * N + qr) * H + hh : hoff + qr;
        *reinterpret_cast<u32x4*>(out + yrow * DV + 8 * c) = v;
      }
    }
  }
  };

  if constexpr (!SAFE) {
    if constexpr (NG == 1) {
      run_kh();
    } else {
      run(Flag<false>{});
    }
    epilogue(Flag<false>{});
    // Row flags of this block: bit m of word NG wv + g for the row of lane column m and
    // group g.
    uint32_t mask[NG];
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      const uint64_t bal = __ballot(bad[g] != 0);
      mask[g] = static_cast<uint32_t>(bal) | static_cast<uint32_t>(bal >> 32);
      if (lane == 0) flags[FW * (static_cast<int64_t>(bh) * nqb + qb) + NG * wv + g] = mask[g];
    }
    if constexpr (NG == 1) {
      // One-group blocks redo a flagged block here rather than in a second launch, which
      // costs more than the rare fixup itself on the small problems that use them. The
      // waves share their flags through LDS; the barrier also ends every wave's reads of
      // the staging slots.
      __shared__ uint32_t wave_flags[NW];
      if (lane == 0) wave_flags[wv] = mask[0];
      __syncthreads();
      uint32_t any = 0;
#pragma unroll
      for (int i = 0; i < NW; ++i) any |= wave_flags[i];
      if (__builtin_amdgcn_readfirstlane(any) != 0) {
        bad[0] = (mask[0] >> m) & 1u;
        // The fast pass's stores of the flagged rows land before the rewrite.
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        run(Flag<true>{});
        epilogue(Flag<true>{});
      }
    }
  } else {
    run(Flag<true>{});
    epilogue(Flag<true>{});
  }
}

}  // namespace fwdbf16

// Query groups per wave: one (128-row blocks) when the 256-row blocks would not fill
// the chip twice over. Every wave of a block walks all keys up to the block's end, so a
// wave's longest walk is half as long with 32 rows per wave; with few blocks per compute
// unit that walk, not the total work, sets the time. With more blocks the hardware's
// longest-first dispatch already balances the compute units, and two groups per wave
// share every K and V^T operand read.
constexpr int64_t kFwdOneGroupMaxBlocks = 384;
int fwd_bf16_groups(int64_t B, int64_t H, int64_t N) {
  const int64_t blocks256 = B * H * ((N + fwdbf16::BR - 1) / fwdbf16::BR);
  return blocks256 <= kFwdOneGroupMaxBlocks ? 1 : 2;
}

template <int NG>
static hipError_t launch_fwd_bf16_ng(const FwdArgs& a, hipStream_t s) {
  using namespace fwdbf16;
  static std::atomic<uint64_t> attr_done{0};
  const hipError_t ea = once_per_device(attr_done, [] {
    hipError_t r = hipFuncSetAttribute(reinterpret_cast<const void*>(fwd_bf16_kernel<false, NG>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, LDS_BYTES);
    if (NG == 2 && r == hipSuccess)
      r = hipFuncSetAttribute(reinterpret_cast<const void*>(fwd_bf16_kernel<true, 2>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, LDS_BYTES);
    return r;
  });
  if (ea != hipSuccess) return ea;
  constexpr int RB = 32 * NW * NG;
  const int64_t BH = a.B * a.H;
  const int nqb = static_cast<int>((a.N + RB - 1) / RB);
  const int64_t nblk = BH * nqb;
  const diffattn_saved& sv = a.saved;
  uint32_t* flags = static_cast<uint32_t*>(a.workspace);
  auto launch = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(nblk)), dim3(NT), LDS_BYTES, s,
                       static_cast<const bf16_t*>(a.q1), static_cast<const bf16_t*>(a.q2),
                       static_cast<const bf16_t*>(a.k1), static_cast<const bf16_t*>(a.k2),
                       static_cast<const bf16_t*>(a.v), a.lam, a.rms_weight,
                       static_cast<bf16_t*>(a.out), a.training ? sv.lse1 : nullptr,
                       a.training ? sv.lse2 : nullptr, a.training ? sv.o1 : nullptr,
                       a.training ? sv.o2 : nullptr, a.training ? sv.rstd : nullptr, flags,
                       static_cast<int>(BH), static_cast<int>(a.H), static_cast<int>(a.N), nqb,
                       a.eps, a.out_bnh ? 1 : 0, a.G);
    return hipGetLastError();
  };
  hipError_t e = launch(fwd_bf16_kernel<false, NG>);
  // One-group blocks fix their flagged rows in the same launch.
  if (e != hipSuccess || NG == 1) return e;
  return launch(fwd_bf16_kernel<true, 2>);
}

hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t s) {
  return fwd_bf16_groups(a.B, a.H, a.N) == 1 ? launch_fwd_bf16_ng<1>(a, s)
                                             : launch_fwd_bf16_ng<2>(a, s);
}

size_t fwd_bf16_workspace_bytes(int64_t B, int64_t H, int64_t N) {
  // Row flags: 8 words per 256-row block, or 4 per 128-row block (no more words in all).
  const int64_t nqb = (N + fwdbf16::BR - 1) / fwdbf16::BR;
  return static_cast<size_t>(B * H * nqb) * 8 * sizeof(uint32_t);
}

}  // namespace diffattn
