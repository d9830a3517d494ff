// The projections on either side of DiffAttn, as bf16 MFMA GEMMs (float32 accumulation).
//
// The input embeddings X are projected into two queries, two keys and one value per head
// (Q1, Q2 from W_Q; K1, K2 from W_K; V from W_V), and the per-head outputs, concatenated
// over heads, are projected back to the model width by W_O (intoai.pub, "Moving On To The
// Differential Transformer" and "Differential Attention With Multiple Heads";
// pt.news.hada.io, "Estrutura multi-head e arquitetura completa").
//
// One kernel computes C = A B^T for A [M, K] and B [Nc, K], both row-major with K
// contiguous (B is a weight in the [out_features, in_features] layout), and writes C in
// bf16 (round to nearest even) through one of two epilogues:
//   plain  C row-major [M, Nc] (the W_O projection into [B, N, d_model]);
//   qkv    the fused [(H + 2 Hkv) 2d, d_model] weight's columns scattered into Q1, Q2
//          [B, H, N, d], K1, K2 [B, Hkv, N, d] and V [B, Hkv, N, 2d] (Hkv < H: grouped-
//          query attention): column h 2d + j d + c of the query block is channel c of
//          Q_(j+1) in head h, likewise for the key block; column h 2d + c of the value
//          block is channel c of V in head h. Row b N + i is token i of sequence b.
//
// Tiling: a 256-thread workgroup (4 waves, 2 x 2, one per SIMD) computes a 256 x 256
// tile of C in K-steps of 64; each wave holds a 128 x 128 sub-tile as 4 x 4 accumulators
// of the 32x32x16 bf16 MFMA (256 accumulation registers, so they live in the AGPRs). Per
// 16-deep step a wave reads 4 A and 4 B operands from LDS for 16 products: half an LDS
// read per product, which keeps the LDS well below its bandwidth. A and B K-slabs
// (32 KiB each) are copied global -> LDS by the buffer unit (buffer_load ... lds),
// double-buffered, one barrier per K-step. A slab's 16 loads per wave go out four at a
// time: after the barrier that frees its stage, then at the start of each of the next
// K-step's first three 16-deep steps, where the matrix core still has products queued
// (sixteen at once stalled the wave's issue). The finished tile is rounded to bf16 and
// staged through LDS, so that every lane stores 16 contiguous bytes. Tiles are ordered in
// groups of four 256-row panels (so the 32 tiles one XCD runs at a time share A and B
// slabs in its L2), and each XCD is given a contiguous range of that order.
#include "common.h"
#include "launch.h"

namespace diffattn {
namespace gemm {

#define LDS_AS __attribute__((address_space(3)))

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int NT = 256, NWAVE = 4;
constexpr int WT = 128;                    // wave sub-tile: WT x WT
constexpr int SLAB = BM * BK * 2;          // bytes of one A (or B) K-slab: 32 KiB
constexpr int STAGE = 2 * SLAB;            // A slab then B slab
constexpr int LDS_BYTES = 2 * STAGE;       // two stages: 128 KiB
constexpr int GROUP_M = 4;                 // 256-row panels per tile group
static_assert(BM == BN, "A and B slabs share one layout");

// Slab rows are 128 bytes (64 bf16 of K); the 16-byte unit u of row r is stored at
// u ^ swz(r). The 32 rows that one operand read touches (lanes 0..31, then 32..63) then
// fall into distinct bank groups: bits (b0 ^ b2, b1, b3) of the row pick the unit, so any
// 8 consecutive rows use 8 different 16-byte slots of a 128-byte line and any 16 use 16
// different slots of 256 bytes.
__device__ __forceinline__ int swz(int row) {
  return ((row ^ (row >> 2)) & 1) | (row & 2) | ((row >> 1) & 4);
}

// Buffer resource words (raw buffer, no swizzle) covering `bytes` bytes at `base`: loads
// past the end return zeros, which pads the M and Nc tails of a tile.
__device__ __forceinline__ u32x4 rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const u32x4 r = {static_cast<uint32_t>(a), static_cast<uint32_t>(a >> 32) & 0xffffu, bytes,
                   0x00020000u};
  return r;
}

// 16 bytes per lane from the buffer at byte offset voff into LDS at m0 + 16 lane. Issued
// as assembly so the compiler does not make later LDS reads wait on it; the K-step
// barrier orders the two. (m0 is used by nothing else in this kernel.)
__device__ __forceinline__ void dma16(const u32x4& rs, uint32_t m0, int voff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(m0), "v"(voff), "s"(rs));
}

// This wave's share of one K-slab: 32 transfers of 1 KiB (8 rows each) per slab, eight
// per wave. Lane l of transfer t fills 16-byte slot l of its KiB: row 8 t + l / 8, stored
// unit l % 8, which holds K unit (l % 8) ^ swz(row) of that row.
__device__ __forceinline__ void load_slab(const u32x4& rs, uint32_t dst, int k0, int row_bytes,
                                          int wv, int lane) {
#pragma unroll
  for (int r = 0; r < 32 / NWAVE; ++r) {
    const int t = wv + NWAVE * r;
    const int row = 8 * t + (lane >> 3);
    const int unit = (lane & 7) ^ swz(row);
    dma16(rs, dst + 1024 * t, row * row_bytes + k0 * 2 + 16 * unit);
  }
}

// Transfers R0 .. R0 + RN - 1 of this wave's eight (see load_slab).
template <int R0, int RN>
__device__ __forceinline__ void load_part(const u32x4& rs, uint32_t dst, int k0, int row_bytes,
                                          int wv, int lane) {
#pragma unroll
  for (int r = R0; r < R0 + RN; ++r) {
    const int t = wv + NWAVE * r;
    const int row = 8 * t + (lane >> 3);
    const int unit = (lane & 7) ^ swz(row);
    dma16(rs, dst + 1024 * t, row * row_bytes + k0 * 2 + 16 * unit);
  }
}

__device__ __forceinline__ bf16x8 lds_operand(uint32_t slab, int row, int unit) {
  const int addr = static_cast<int>(slab) + row * 128 + 16 * (unit ^ swz(row));
  return *reinterpret_cast<const LDS_AS bf16x8*>((LDS_AS char*)nullptr + addr);
}

struct QkvOut {
  bf16_t *q1, *q2, *k1, *k2, *v;
  uint32_t n;    // tokens per sequence
  int h;         // query heads
  int hkv;       // key / value heads
  int d;         // width of Q1 / K1 (V is 2d)
};

// Column block [n, n + 32) of the fused projection (never straddling a head half, as d
// is a multiple of 32): its destination tensor, offset by head and channel, its row
// stride (width) and the heads of that tensor; row (b, i) then sits (b heads N + i) rows
// further.
__device__ __forceinline__ bf16_t* qkv_column(const QkvOut& o, int n, int& width, int& heads) {
  const int d2 = 2 * o.d;
  const int q_cols = d2 * o.h, kv_cols = d2 * o.hkv;
  const int which = n < q_cols ? 0 : (n < q_cols + kv_cols ? 1 : 2);
  const int hc = n - (which == 0 ? 0 : (which == 1 ? q_cols : q_cols + kv_cols));
  const int head = hc / d2, within = hc - head * d2;
  const int64_t head_off = static_cast<int64_t>(head) * o.n;
  heads = which == 0 ? o.h : o.hkv;
  if (which == 2) {
    width = d2;
    return o.v + head_off * width + within;
  }
  const int half = within >= o.d;
  width = o.d;
  bf16_t* base = which == 0 ? (half ? o.q2 : o.q1) : (half ? o.k2 : o.k1);
  return base + head_off * width + (within - half * o.d);
}

template <bool QKV>
__global__ void __launch_bounds__(NT, 1)
    gemm_bf16_kernel(const bf16_t* __restrict__ A, const bf16_t* __restrict__ Bw,
                     bf16_t* __restrict__ C, QkvOut qo, int64_t M, int Nc, int K) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (LDS bases in SGPRs)
  const int wm = wv >> 1, wn = wv & 1;

  // Tile of this workgroup: XCD x (= block id mod 8) takes a contiguous range of the
  // grouped tile order.
  const int m_tiles = static_cast<int>((M + BM - 1) / BM), n_tiles = (Nc + BN - 1) / BN;
  const int T = m_tiles * n_tiles;
  const int id = blockIdx.x, x = id & 7, q = T >> 3, rem = T & 7;
  const int t = x * q + (x < rem ? x : rem) + (id >> 3);
  const int per_group = GROUP_M * n_tiles;
  const int g = t / per_group, in_g = t - g * per_group;
  const int gm = min(GROUP_M, m_tiles - g * GROUP_M);
  const int mt = g * GROUP_M + in_g % gm, nt = in_g / gm;
  const int64_t m0 = static_cast<int64_t>(mt) * BM;
  const int n0 = nt * BN;

  const int64_t a_rows = min<int64_t>(BM, M - m0);
  const int b_rows = min(BN, Nc - n0);
  const u32x4 ra = rsrc(A + m0 * K, static_cast<uint32_t>(a_rows * K * 2));
  const u32x4 rb = rsrc(Bw + static_cast<int64_t>(n0) * K, static_cast<uint32_t>(b_rows) * K * 2);
  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((LDS_AS char*)smem));

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  const int KT = K / BK;
  const int r32 = lane & 31, hi = lane >> 5;
  // Operands of one 16-deep step: A rows 128 wm + 32 i + r32, B rows 128 wn + 32 j + r32.
  auto read_ops = [&](bf16x8 (&a)[4], bf16x8 (&b)[4], uint32_t stage, int kk)
                      __attribute__((always_inline)) {
    const int unit = 2 * kk + hi;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      a[i] = lds_operand(stage, WT * wm + 32 * i + r32, unit);
      b[i] = lds_operand(stage + SLAB, WT * wn + 32 * i + r32, unit);
    }
  };
  auto products = [&](const bf16x8 (&a)[4], const bf16x8 (&b)[4], int first, int count)
                      __attribute__((always_inline)) {
#pragma unroll
    for (int t = first; t < first + count; ++t)
      acc[t >> 2][t & 3] =
          __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[t >> 2], b[t & 3], acc[t >> 2][t & 3], 0, 0, 0);
  };
  // One read issued after each of the first 8 products (the reads of the next step run
  // while the matrix core works), then the remaining products.
  auto interleave = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // one LDS read
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
  };

  // Slabs 0 and 1 in flight; slab 0 landed for every wave; step 0's operands read.
  load_slab(ra, lds0, 0, K * 2, wv, lane);
  load_slab(rb, lds0 + SLAB, 0, K * 2, wv, lane);
  if (KT > 1) {
    load_slab(ra, lds0 + STAGE, BK, K * 2, wv, lane);
    load_slab(rb, lds0 + STAGE + SLAB, BK, K * 2, wv, lane);
    asm volatile("s_waitcnt vmcnt(16)\n\ts_barrier" ::: "memory");
  } else {
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
  }
  bf16x8 fa[2][4], fb[2][4];
  read_ops(fa[0], fb[0], lds0, 0);
  for (int kt = 0; kt < KT; ++kt) {
    DIFFATTN_DEBUG_BARRIER();   // every wave runs the same K-steps
    const uint32_t cur = lds0 + (kt & 1) * STAGE;
    // The rest of slab kt + 1, a quarter per step (its first quarter went out after the
    // previous K-step's barrier), into the stage this K-step does not read.
    const bool rest = kt >= 1 && kt + 1 < KT;
    const uint32_t nst = lds0 + ((kt + 1) & 1) * STAGE;
    const int nk0 = (kt + 1) * BK;
    if (rest) load_part<4, 4>(ra, nst, nk0, K * 2, wv, lane);
    read_ops(fa[1], fb[1], cur, 1);
    products(fa[0], fb[0], 0, 16);
    interleave();
    if (rest) load_part<0, 4>(rb, nst + SLAB, nk0, K * 2, wv, lane);
    read_ops(fa[0], fb[0], cur, 2);
    products(fa[1], fb[1], 0, 16);
    interleave();
    if (rest) load_part<4, 4>(rb, nst + SLAB, nk0, K * 2, wv, lane);
    read_ops(fa[1], fb[1], cur, 3);
    products(fa[0], fb[0], 0, 16);
    interleave();
    // Last step of slab kt. Its operands are in registers once the first product has
    // issued; then slab kt + 1 (sent one K-step ago) must have landed for every wave, and
    // every wave is done reading slab kt, so its stage can take slab kt + 2.
    products(fa[1], fb[1], 0, 4);
    if (kt + 1 < KT) {
      asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
      // The remaining products stay below the barrier: they consume these registers.
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) asm volatile("" : "+a"(acc[i][j]));
      if (kt + 2 < KT) load_part<0, 4>(ra, cur, (kt + 2) * BK, K * 2, wv, lane);
      read_ops(fa[0], fb[0], lds0 + ((kt + 1) & 1) * STAGE, 0);
    }
    products(fa[1], fb[1], 4, 12);
  }

  // Epilogue. Accumulator element e of block (i, j) is row 8 (e / 4) + 4 hi + e % 4,
  // column r32 of the block. Each wave rounds its 128 x 128 sub-tile to bf16 into its own
  // 32 KiB of LDS (rows of 256 bytes; the 16-byte unit u of row r at u ^ (r & 15)), then
  // stores it back row by row, 16 bytes per lane.
  asm volatile("s_barrier" ::: "memory");   // every wave is done with the last slab
  LDS_AS char* const stage = (LDS_AS char*)smem + wv * (WT * WT * 2);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int r = 32 * i + 8 * (e >> 2) + 4 * hi + (e & 3);
        const int c = 32 * j + r32;
        const int u = (c >> 3) ^ (r & 15);
        *reinterpret_cast<LDS_AS bf16_t*>(stage + r * 256 + 16 * u + 2 * (c & 7)) =
            f32_to_bf16(acc[i][j][e]);
      }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // this wave's staging writes done
  // Each pass stores 4 rows: lane l takes unit l % 16 of row 4 pass + l / 16.
  const int u = lane & 15;
  const int n = n0 + WT * wn + 8 * u;              // first column of this lane's 16 bytes
  const bool col_ok = n < Nc;                       // Nc is a multiple of 8
  int width = Nc, heads = 1;
  bf16_t* col = C + n;
  if (QKV) col = (col_ok ? qkv_column(qo, n & ~31, width, heads) : qo.q1) + (n & 31);
  const int64_t mrow0 = m0 + WT * wm;
#pragma unroll 4
  for (int pass = 0; pass < WT / 4; ++pass) {
    const int r = 4 * pass + (lane >> 4);
    const int64_t m = mrow0 + r;
    const u32x4 val = *reinterpret_cast<const LDS_AS u32x4*>(stage + r * 256 + 16 * (u ^ (r & 15)));
    if (m >= M || !col_ok) continue;
    int64_t row = m;
    if (QKV) {   // m = b N + i  ->  (b heads + 0) N + i; the head is in col
      const uint32_t b = static_cast<uint32_t>(m) / qo.n;
      row = static_cast<int64_t>(b) * (heads - 1) * qo.n + m;
    }
    *reinterpret_cast<u32x4*>(col + row * width) = val;
  }
}

template <bool QKV>
hipError_t launch(const bf16_t* A, const bf16_t* B, bf16_t* C, const QkvOut& qo, int64_t M,
                  int Nc, int K, hipStream_t s) {
  static std::atomic<uint64_t> attr_done{0};   // one word per instantiation
  const hipError_t ea = once_per_device(attr_done, [] {
    return hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_bf16_kernel<QKV>),
                               hipFuncAttributeMaxDynamicSharedMemorySize, LDS_BYTES);
  });
  if (ea != hipSuccess) return ea;
  const int64_t tiles = ((M + BM - 1) / BM) * ((Nc + BN - 1) / BN);
  hipLaunchKernelGGL(gemm_bf16_kernel<QKV>, dim3(static_cast<unsigned>(tiles)), dim3(NT),
                     LDS_BYTES, s, A, B, C, qo, M, Nc, K);
  return hipGetLastError();
}

}  // namespace gemm

hipError_t launch_qkv_proj_bf16(const QkvProjArgs& a, hipStream_t s) {
  gemm::QkvOut qo{static_cast<bf16_t*>(a.q1), static_cast<bf16_t*>(a.q2),
                  static_cast<bf16_t*>(a.k1), static_cast<bf16_t*>(a.k2),
                  static_cast<bf16_t*>(a.v),  static_cast<uint32_t>(a.N), static_cast<int>(a.H),
                  static_cast<int>(a.Hkv), a.d};
  const int nc = static_cast<int>(2 * a.d * (a.H + 2 * a.Hkv));
  return gemm::launch<true>(static_cast<const bf16_t*>(a.x), static_cast<const bf16_t*>(a.w),
                            nullptr, qo, a.B * a.N, nc, static_cast<int>(a.d_model), s);
}

hipError_t launch_out_proj_bf16(const OutProjArgs& a, hipStream_t s) {
  gemm::QkvOut none{};
  return gemm::launch<false>(static_cast<const bf16_t*>(a.attn), static_cast<const bf16_t*>(a.w),
                             static_cast<bf16_t*>(a.y), none, a.M, static_cast<int>(a.d_model),
                             static_cast<int>(a.k), s);
}

}  // namespace diffattn
