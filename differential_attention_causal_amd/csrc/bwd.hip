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
//         (the kernels form A2 (D2 - dP) per score; lambda scales dK2 and dQ2 once, at
//          their stores)
//   dK_k = s dS_k^T Q_k                                   (bwd_dkdv_kernel)
//   dQ_k = s dS_k K_k                                     (bwd_dq_kernel)
//   dlambda = -sum over rows of D2; lambda = exp(lq1.lk1) - exp(lq2.lk2) + lambda_init gives
//   dlq1 = dlambda e^a lk1, dlk1 = dlambda e^a lq1, dlq2 = -dlambda e^b lk2,
//   dlk2 = -dlambda e^b lq2                               (lambda_grad_kernel)
//   dw_h = (1 - lambda_init) sum over (b, i) of dout O r  (bwd_pre_kernel partials,
//                                                          rms_weight_grad_kernel)
// A_k is recomputed from the log-sum-exps the forward saved: A_k = exp(S_k - lse_k).
//
// Two matrix-core kernels, no atomics (deterministic). Both have the same shape:
//  * Each wavefront owns 32 rows (keys in bwd_dkdv_kernel, queries in bwd_dq_kernel). A
//    dK/dV workgroup is 4 wavefronts, one per SIMD; a dQ workgroup is 8, two per SIMD (the
//    dQ kernel fits in half the register file, so each SIMD interleaves two waves). The operands that belong to the owned
//    rows stay in the accumulation registers for the whole kernel (as the B operand of the
//    score and dP products), next to the gradient accumulators.
//  * The other side (query tiles for dK/dV, key tiles for dQ) streams through LDS in tiles
//    of 64 rows: buffer loads with LDS as the destination fill a ring of 4 slots, two
//    tiles ahead, with one barrier per tile. One swizzled layout per tensor serves both
//    the row reads (ds_read_b128, A operand of S = Q K^T and dP = G V^T) and the
//    transposing reads (ds_read_b64_tr_b16, A operand of dV^T = G^T P and dK^T = Q^T dS).
//  * Per 32 x 32 sub-tile j the work is A(j): score and dP products; B(j): weights and
//    score gradients on the vector ALUs; C(j): the gradient products. They are
//    software-pipelined: one half-step issues the products of A(j+1) and C(j-1), one per
//    fixed slot, with the vector work of B(j) placed between them, so the matrix cores
//    always have work queued while the vector unit computes.
#include "common.h"
#include "launch.h"

namespace diffattn {
namespace bwd {

#define LDS_AS __attribute__((address_space(3)))

constexpr int D = 64;
constexpr int DV = 128;
constexpr int NW = 4;            // wavefronts per workgroup
constexpr int NT = 64 * NW;
constexpr int BW = 32 * NW;      // rows owned by a workgroup
// The dQ kernel: 8 wavefronts (two per SIMD, so that one hides the other's latencies),
// 32 query rows each.
constexpr int NWQ = 8;
constexpr int NTQ = 64 * NWQ;
constexpr int BWQ = 32 * NWQ;
constexpr int TB = 64;           // rows per streamed tile
constexpr int NSLOT = 4;         // LDS ring depth
constexpr int REG = TB * 64;     // one 32-channel region of a tile: [64 rows][64 B]

// dK/dV slot: Q1 (2 regions) | Q2 (2) | G (4) | per-row vector (lse1, lse2, D1, D2).
constexpr int KV_Q1 = 0;
constexpr int KV_Q2 = 2 * REG;
constexpr int KV_G = 4 * REG;
constexpr int KV_VEC = 8 * REG;
constexpr int KV_SLOT = KV_VEC + TB * 16;
constexpr int KV_LDS = NSLOT * KV_SLOT;
// dQ slot: K1 (2 regions) | K2 (2) | V (4).
constexpr int Q_K1 = 0;
constexpr int Q_K2 = 2 * REG;
constexpr int Q_V = 4 * REG;
constexpr int Q_SLOT = 8 * REG;
constexpr int Q_LDS = NSLOT * Q_SLOT;
// Per-wave regions of the result staging (the stores through LDS), inside the ring.
constexpr int KV_STAGE = 32 * (2 * DV + 16) + 2 * 32 * (2 * D + 16);
constexpr int Q_STAGE = 2 * 32 * (2 * D + 16);
static_assert(NW * KV_STAGE <= KV_LDS && NWQ * Q_STAGE <= Q_LDS, "staging exceeds the ring");

// Tile layout: a W-channel bf16 tensor is stored as W/32 regions of [64 rows][64 B]; the
// 16-byte chunk c of row r sits at position c ^ sw(r). With sw, the 16 operand rows that a
// group of 16 lanes reads with ds_read_b128 fall into 16 different 16-byte bank groups
// (and any 8 of them into 8), and the 4-row, 2-chunk footprint of a transposing read of 16
// lanes into 8.
__device__ __forceinline__ int sw(int r) { return 2 * (((r >> 1) ^ (r >> 2)) & 1) + ((r >> 3) & 1); }
// Operand row m of a score product reads tile row perm_row(m) (bits 2 and 3 swapped), so
// that output register j of lane half h holds row idx_of(j, h): 8 consecutive rows per 8
// registers, the layout of a B operand whose contraction runs over those rows.
__device__ __forceinline__ int perm_row(int m) {
  return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}
__host__ __device__ constexpr int idx_of(int j, int h) { return 16 * (j >> 3) + 8 * h + (j & 7); }

// ---------------------------------------------------------------------------- helpers
template <bool B>
struct Flag {
  static constexpr bool value = B;
};
template <int N>
struct Int {
  static constexpr int value = N;
};
template <int A, int B, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (A < B) {
    f(Int<A>{});
    static_for<A + 1, B>(f);
  }
}

// Buffer resource words (raw 32-bit buffer, no swizzle) for `bytes` bytes at `base`.
__device__ __forceinline__ u32x4 rsrc_words(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const u32x4 r = {static_cast<uint32_t>(a), static_cast<uint32_t>(a >> 32) & 0xffffu, bytes,
                   0x00020000u};
  return r;
}
// 16 bytes per lane from the buffer (offset voff) into LDS at m0 + 16 lane. Issued as
// assembly: the compiler would otherwise make every later LDS read wait for it. (m0 is
// reserved by the compiler and used by nothing else in these kernels.)
__device__ __forceinline__ void dma16(const u32x4& rs, uint32_t m0, int voff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(m0), "v"(voff), "s"(rs));
}
// One 1 KiB block (rows 16 (b % 4) .. +15 of region b / 4) of the W-channel tile whose
// first row is t0, into LDS byte address dst + 1024 b; lane l's 16 bytes land at
// dst + 1024 b + 16 l.
template <int W>
__device__ __forceinline__ void dma_rows(const u32x4& rs, uint32_t dst, int t0, int b, int lane) {
  const int region = b >> 2, row = 16 * (b & 3) + (lane >> 2), p = lane & 3;
  const int off = (t0 + row) * (W * 2) + 64 * region + 16 * (p ^ sw(row));
  dma16(rs, dst + 1024 * b, off);
}
// Workgroup barrier that also keeps the compiler from moving LDS reads across it.
__device__ __forceinline__ void barrier() { asm volatile("s_barrier" ::: "memory"); }

// Result rows leave through LDS. A lane's accumulator holds 4 consecutive channels of
// one row (8 bytes), and 32 rows per store instruction cost the memory pipeline about as
// much per row as a whole line: the wave instead writes its 32 rows of a W-channel result
// into LDS, row pitch 2 W + 16 bytes (the 8-byte writes of 32 rows and the 16-byte reads
// along rows both meet no bank conflict), and copies them out as 16-byte pieces of
// contiguous rows, 1 KiB per instruction.
template <int W>
constexpr int stage_pitch() { return 2 * W + 16; }
template <int W>
constexpr int stage_bytes() { return 32 * stage_pitch<W>(); }
// Lane (m, h): channels 32 b + 8 jg + 4 h .. + 3 of row m.
template <int W>
__device__ __forceinline__ void stage_put(int base, int m, int h, int b, int jg, u32x2 v) {
  *reinterpret_cast<LDS_AS u32x2*>((LDS_AS char*)nullptr + base + m * stage_pitch<W>() +
                                   2 * (32 * b + 8 * jg + 4 * h)) = v;
}
// The 32 staged rows to dst (row pitch W elements); rows from `valid` on are not written.
// Every lane of the wave has put its values (the wave's LDS accesses complete in order).
template <int W>
__device__ __forceinline__ void stage_flush(int base, bf16_t* dst, int valid, int lane) {
  constexpr int LPR = 2 * W / 16;   // lanes per row
  constexpr int RPI = 64 / LPR;     // rows per instruction
  asm volatile("" ::: "memory");
#pragma unroll
  for (int i = 0; i < 32 / RPI; ++i) {
    const int r = RPI * i + lane / LPR, cb = 16 * (lane % LPR);
    const u32x4 x = *reinterpret_cast<const LDS_AS u32x4*>(
        (LDS_AS char*)nullptr + base + r * stage_pitch<W>() + cb);
    if (r < valid) *reinterpret_cast<u32x4*>(reinterpret_cast<char*>(dst + r * W) + cb) = x;
  }
}

template <int N>
__device__ __forceinline__ void vm_wait() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// LDS operand reads are ordinary loads: the compiler tracks their completion and inserts
// the waits. The tile loads that fill the ring are issued as assembly (below), so the
// compiler does not order these reads behind them; the tile barrier orders them instead.
template <int OFF>
__device__ __forceinline__ u32x4 rd128(int a) {
  return *reinterpret_cast<const LDS_AS u32x4*>((LDS_AS char*)nullptr + a + OFF);
}
typedef short s16x4 __attribute__((ext_vector_type(4)));
template <int OFF>
__device__ __forceinline__ u32x2 rdtr(int a) {
  const s16x4 v =
      __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)((LDS_AS char*)nullptr + a + OFF));
  return __builtin_bit_cast(u32x2, v);
}
__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& x) { return __builtin_bit_cast(bf16x8, x); }
__device__ __forceinline__ bf16x8 tr_operand(const u32x2& lo, const u32x2& hi) {
  const u32x4 x = {lo[0], lo[1], hi[0], hi[1]};
  return __builtin_bit_cast(bf16x8, x);
}
__device__ __forceinline__ bf16x8 words(const uint32_t (&w)[8], int ks) {
  const u32x4 x = {w[4 * ks], w[4 * ks + 1], w[4 * ks + 2], w[4 * ks + 3]};
  return __builtin_bit_cast(bf16x8, x);
}

// Score / dP product with its B operand in the accumulation registers; the result stays
// in vector registers for the vector ALU. Destinations are early-clobber (a product may
// not overwrite its own operands); consumers are fenced by s_guard.
__device__ __forceinline__ void mm_first(f32x16& d, const bf16x8& a, const bf16x8& b) {
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "a"(b));
}
__device__ __forceinline__ void mm_acc(f32x16& d, const bf16x8& a, const bf16x8& b) {
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "a"(b));
}
// Wait states between the last product into a buffer and the first vector read of it.
__device__ __forceinline__ void s_guard(f32x16& a) { asm volatile("s_nop 7\n\ts_nop 4" : "+v"(a)); }
__device__ __forceinline__ void s_guard3(f32x16& a, f32x16& b, f32x16& c) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 4" : "+v"(a), "+v"(b), "+v"(c));
}
// Anchors: the values are complete at this point of the instruction stream. Without them
// the vector work of a slot may be moved away from the products it is meant to overlap.
template <typename A>
__device__ __forceinline__ void anchor(A& a) {
  asm volatile("" : "+v"(a));
}
template <typename A, typename B>
__device__ __forceinline__ void anchor(A& a, B& b) {
  asm volatile("" : "+v"(a), "+v"(b));
}
template <typename A, typename B, typename C>
__device__ __forceinline__ void anchor(A& a, B& b, C& c) {
  asm volatile("" : "+v"(a), "+v"(b), "+v"(c));
}
template <typename A, typename B, typename C, typename E>
__device__ __forceinline__ void anchor(A& a, B& b, C& c, E& e) {
  asm volatile("" : "+v"(a), "+v"(b), "+v"(c), "+v"(e));
}
template <typename A, typename B, typename C, typename E, typename F>
__device__ __forceinline__ void anchor(A& a, B& b, C& c, E& e, F& f) {
  asm volatile("" : "+v"(a), "+v"(b), "+v"(c), "+v"(e), "+v"(f));
}
// Keeps a value in the accumulation registers.
template <typename T>
__device__ __forceinline__ void pin_a(T& x) {
  asm volatile("" : "+a"(x));
}
__device__ __forceinline__ f32x16 mfma(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// LDS read schedules (reads issued per slot of a half-step, the same in every half-step;
// reads for the first slots of the next half-step are issued at the end of this one).
// Waits are computed from them: lgkmcnt(n) with n = reads issued after the awaited one
// up to the wait (at most 15, which only waits longer).
struct KvSched {   // dK/dV: 32 slots, C products in 0..15, A products in 16..31
  static constexpr int SLOTS = 32, LT = 4, LA = 5;
  static constexpr int ntr(int k) { return (k <= 15 - LT || k >= SLOTS - LT) ? 2 : 0; }
  static constexpr int nrow(int k) { return (k >= 16 - LA && k <= 31 - LA) ? 1 : 0; }
  static constexpr int nvec(int k) { return (k % 4 == 1) ? 2 : 0; }
  static constexpr int n(int k) { return ntr(k) + nrow(k) + nvec(k); }
  static constexpr int between(int a, int b) {   // reads in slots [a, b), a may be < 0
    int s = 0;
    for (int k = a; k < b; ++k) s += n((k + SLOTS) % SLOTS);
    return s;
  }
  static constexpr int cap(int x) { return x > 15 ? 15 : x; }
  static constexpr int wait_c(int i) {     // C product i at slot i
    const int t = i - LT, tt = (t + SLOTS) % SLOTS;
    return cap(nrow(tt) + nvec(tt) + between(t + 1, i));
  }
  static constexpr int wait_a(int i) {     // A product i at slot 16 + i
    const int t = 16 + i - LA;
    return cap(nvec(t) + between(t + 1, 16 + i));
  }
  static constexpr int wait_v(int pr) {    // vector of pair pr, used at slot 4 pr
    return cap(between(4 * pr - 3 + 1, 4 * pr + 1));
  }
};
struct QSched {    // dQ: 24 slots, C products in 0..7, A products in 8..23
  static constexpr int SLOTS = 24, LT = 3, LA = 4;
  static constexpr int ntr(int k) { return (k <= 7 - LT || k >= SLOTS - LT) ? 2 : 0; }
  static constexpr int nrow(int k) { return (k >= 8 - LA && k <= 23 - LA) ? 1 : 0; }
  static constexpr int n(int k) { return ntr(k) + nrow(k); }
  static constexpr int between(int a, int b) {
    int s = 0;
    for (int k = a; k < b; ++k) s += n((k + SLOTS) % SLOTS);
    return s;
  }
  static constexpr int cap(int x) { return x > 15 ? 15 : x; }
  static constexpr int wait_c(int i) {
    const int t = i - LT, tt = (t + SLOTS) % SLOTS;
    return cap(nrow(tt) + between(t + 1, i));
  }
  static constexpr int wait_a(int i) {
    const int t = 8 + i - LA;
    return cap(between(t + 1, 8 + i));
  }
};

// A products of a sub-tile, in slot order: (S1, S2, dP) for k-steps 0..3, then dP 4..7.
// Returns 0 = S1, 1 = S2, 2 = dP, and the k-step.
__host__ __device__ constexpr int a_kind(int i) { return i < 12 ? i % 3 : 2; }
__host__ __device__ constexpr int a_kb(int i) { return i < 12 ? i / 3 : i - 8; }

// A product i of a sub-tile: destination buffer and resident B operand by kind.
template <int KIND, int KB>
__device__ __forceinline__ void a_product(f32x16& s1, f32x16& s2, f32x16& dp, const bf16x8& a,
                                          const bf16x8 (&b1)[4], const bf16x8 (&b2)[4],
                                          const bf16x8 (&bv)[8]) {
  f32x16& d = KIND == 0 ? s1 : (KIND == 1 ? s2 : dp);
  const bf16x8& b = KIND == 0 ? b1[KB & 3] : (KIND == 1 ? b2[KB & 3] : bv[KB]);
  if constexpr (KB == 0) mm_first(d, a, b);
  else mm_acc(d, a, b);
}

// ------------------------------------------------------------------------ bwd_pre
// 64 rows per workgroup, 8 at a time, 32 threads per row, 4 channels per thread.
// Writes G (float32 to d_attn, bf16 to gb), the per-row vector (lse1 log2 e, lse2 log2 e,
// D1, D2) the main kernels read, and one partial sum of D2 per workgroup.
// Workgroup blk covers rows n0 .. n0 + 63 (n0 = 64 (blk % nchunk)) of head bh = blk / nchunk,
// 8 rows at a time, 32 lanes per row with 4 channels each. Besides G, the bf16 copy of G
// and the per-row vector, it writes part[blk] = the sum of D2 over its rows and
// pw[blk] = its rows' share of the RMSNorm weight gradient (2d floats), both summed in a
// fixed order.
__global__ void __launch_bounds__(256) bwd_pre_kernel(
    const float* __restrict__ o1, const float* __restrict__ o2, const float* __restrict__ rstd,
    const float* __restrict__ lse1, const float* __restrict__ lse2,
    const bf16_t* __restrict__ dout, const diffattn_lambda_state* __restrict__ lamst,
    const float* __restrict__ rms_w, float* __restrict__ d_attn, bf16_t* __restrict__ gb,
    f32x4* __restrict__ vec, float* __restrict__ part, f32x4* __restrict__ pw, int64_t N,
    int64_t H, int64_t nchunk, int dout_bnh) {
  __shared__ float red[8];
  __shared__ f32x4 redw[8][32];
  const int tid = threadIdx.x;
  const int t = tid & 31;
  const float lam = lamst->lambda_f;
  const float gsc = lamst->one_minus_init_f;
  const int64_t blk = blockIdx.x;
  const int64_t bh = blk / nchunk;
  const int64_t n0 = (blk - bh * nchunk) * 64;
  const int64_t hh = bh % H, bb = bh / H;
  float d2 = 0.f;
  f32x4 dw = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
  for (int it = 0; it < 8; ++it) {
    const int64_t n = n0 + 8 * it + (tid >> 5);
    if (n >= N) break;
    const int64_t r = bh * N + n;
    const int64_t yr = dout_bnh ? (bb * N + n) * H + hh : r;   // dout row in its layout
    // O1, O2 and dY are read once: non-temporal loads keep them out of the caches.
    const f32x4 a = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(o1 + r * DV + 4 * t));
    const f32x4 b = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(o2 + r * DV + 4 * t));
    const u32x2 dy = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(dout + yr * DV + 4 * t));
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
      dw[e] = fmaf(gsc * dyv[e], o[e] * rs, dw[e]);
    }
#pragma unroll
    for (int off = 16; off > 0; off >>= 1) go += __shfl_xor(go, off);
    const float k3 = rs * rs * rs * go * (1.0f / DV);
    // The D_k used in dS pair with dP = G V^T, which the products form from the
    // bf16-rounded G, so they are formed from the same rounded values: for a row that sees
    // one key dP - D_k is then zero up to summation order, as it is exactly. dlambda =
    // -sum D2 is summed from the float32 G, where that rounding would swamp rows whose D2
    // is a near-cancellation.
    f32x4 G;
    float dd1 = 0.f, dd2 = 0.f, dd2f = 0.f;
    u32x2 gp;
#pragma unroll
    for (int e = 0; e < 4; ++e) G[e] = rs * g[e] - o[e] * k3;
    gp[0] = pack_bf16x2(G[0], G[1]);
    gp[1] = pack_bf16x2(G[2], G[3]);
    const float gr[4] = {__uint_as_float(gp[0] << 16), __uint_as_float(gp[0] & 0xffff0000u),
                         __uint_as_float(gp[1] << 16), __uint_as_float(gp[1] & 0xffff0000u)};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      dd1 = fmaf(gr[e], a[e], dd1);
      dd2 = fmaf(gr[e], b[e], dd2);
      dd2f = fmaf(G[e], b[e], dd2f);
    }
#pragma unroll
    for (int off = 16; off > 0; off >>= 1) {
      dd1 += __shfl_xor(dd1, off);
      dd2 += __shfl_xor(dd2, off);
      dd2f += __shfl_xor(dd2f, off);
    }
    *reinterpret_cast<f32x4*>(d_attn + r * DV + 4 * t) = G;
    *reinterpret_cast<u32x2*>(gb + r * DV + 4 * t) = gp;
    if (t == 0) {
      const f32x4 vv = {lse1[r] * kLog2e, lse2[r] * kLog2e, dd1, dd2};
      vec[r] = vv;
    }
    d2 += dd2f;
  }
  if (t == 0) red[tid >> 5] = d2;
  redw[tid >> 5][t] = dw;
  __syncthreads();
  if (tid == 0) {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) s += red[i];
    part[blk] = s;   // sum of D2 (float32 G) over this block's rows
  }
  if (tid < 32) {
    f32x4 s = redw[0][tid];
#pragma unroll
    for (int i = 1; i < 8; ++i) s += redw[i][tid];
    pw[blk * 32 + tid] = s;   // channels 4 tid .. 4 tid + 3
  }
}

// d_rms_weight[h, c] = the sum of head h's partials over (b, chunk), in float64 and in a
// fixed order: thread group g (of 32) sums partials q = g, g + 32, ... (q = b nchunk +
// chunk), then the 32 group sums are added in order. Workgroup (h, 8-channel slice),
// thread 8 g + channel.
constexpr int WG_GROUPS = 32, WG_CH = 8;
__global__ void __launch_bounds__(WG_GROUPS * WG_CH) rms_weight_grad_kernel(
    const float* __restrict__ pw, int64_t B, int64_t H, int64_t nchunk, float* __restrict__ dw) {
  __shared__ double red[WG_GROUPS][WG_CH];
  const int64_t h = blockIdx.x;
  const int c = blockIdx.y * WG_CH + threadIdx.x % WG_CH, g = threadIdx.x / WG_CH;
  const int64_t nq = B * nchunk;
  double s = 0.0;
#pragma unroll 4
  for (int64_t q = g; q < nq; q += WG_GROUPS) {
    const int64_t b = q / nchunk, k = q - b * nchunk;
    s += static_cast<double>(pw[((b * H + h) * nchunk + k) * DV + c]);
  }
  red[g][threadIdx.x % WG_CH] = s;
  __syncthreads();
  if (g == 0) {
    double t = red[0][threadIdx.x];
#pragma unroll
    for (int i = 1; i < WG_GROUPS; ++i) t += red[i][threadIdx.x];
    dw[h * DV + c] = static_cast<float>(t);
  }
}

// ------------------------------------------------------------------------ lambda grads
__global__ void __launch_bounds__(1024) lambda_grad_kernel(
    const float* __restrict__ part, int64_t nparts, const diffattn_lambda_state* __restrict__ lamst,
    const float* __restrict__ lq1, const float* __restrict__ lk1, const float* __restrict__ lq2,
    const float* __restrict__ lk2, float* __restrict__ dlq1, float* __restrict__ dlk1,
    float* __restrict__ dlq2, float* __restrict__ dlk2, int d) {
  __shared__ double red[1024];
  const int tid = threadIdx.x;
  double s = 0.0;
  for (int64_t i = tid; i < nparts; i += 1024) s += static_cast<double>(part[i]);
  red[tid] = s;
  __syncthreads();
  for (int off = 512; off > 0; off >>= 1) {
    if (tid < off) red[tid] += red[tid + off];
    __syncthreads();
  }
  const double dlam = -red[0];
  const double ea = lamst->exp_a, eb = lamst->exp_b;
  for (int i = tid; i < d; i += 1024) {
    dlq1[i] = static_cast<float>(dlam * ea * static_cast<double>(lk1[i]));
    dlk1[i] = static_cast<float>(dlam * ea * static_cast<double>(lq1[i]));
    dlq2[i] = static_cast<float>(-dlam * eb * static_cast<double>(lk2[i]));
    dlk2[i] = static_cast<float>(-dlam * eb * static_cast<double>(lq2[i]));
  }
}

// Per-lane byte offsets inside a tile slot (before the slot base).
struct LaneAddr {
  int rb[2];   // row reads: operand row perm_row(m), chunk h (k-step even) or 2 + h (odd)
  int tb[2];   // transposing reads: rows 0..3 / 8..11 (lo) and 4 rows further (hi)
};
__device__ __forceinline__ LaneAddr lane_addr(int lane) {
  LaneAddr a;
  const int m = lane & 31, h = lane >> 5;
  const int pr = perm_row(m);
  a.rb[0] = pr * 64 + 16 * (h ^ sw(pr));
  a.rb[1] = pr * 64 + 16 * ((2 + h) ^ sw(pr));
  const int G = lane >> 4, jj = (lane >> 2) & 3, al = lane & 3;
  const int row = 8 * (G >> 1) + jj;
  const int cp = 2 * (G & 1) + (al >> 1);
  a.tb[0] = row * 64 + 16 * (cp ^ sw(row)) + 8 * (al & 1);
  a.tb[1] = (row + 4) * 64 + 16 * (cp ^ sw(row + 4)) + 8 * (al & 1);
  return a;
}

// ------------------------------------------------------------------------ dK, dV
// C products of a half-step (slot order): dV^T regions 0..3, dK1^T 0..1, dK2^T 0..1 for
// k-step 0, then the same for k-step 1. Tensor 0 = G, 1 = Q1, 2 = Q2.
__host__ __device__ constexpr int kvc_t(int i) { return (i & 7) < 4 ? 0 : ((i & 7) < 6 ? 1 : 2); }
__host__ __device__ constexpr int kvc_b(int i) { return (i & 7) < 4 ? (i & 7) : ((i & 7) < 6 ? (i & 7) - 4 : (i & 7) - 6); }
__host__ __device__ constexpr int kvc_ks(int i) { return i >> 3; }
__host__ __device__ constexpr int kv_toff(int t) { return t == 0 ? KV_G : (t == 1 ? KV_Q1 : KV_Q2); }

struct KvRsrc {
  u32x4 q1, q2, g, vec;
};

// This wave's share of tile `tile` (rows t0 ..) into its ring slot: blocks w, w + 4 of
// Q1 and Q2, w + 4 i of G; wave 0 also moves the 64 per-row vectors (1 KiB).
__device__ __forceinline__ void kv_dma(const KvRsrc& rs, uint32_t lds, int tile, int t0,
                                       int wv, int lane) {
  const uint32_t base = lds + (tile % NSLOT) * KV_SLOT;
  dma_rows<D>(rs.q1, base + KV_Q1, t0, wv, lane);
  dma_rows<D>(rs.q1, base + KV_Q1, t0, wv + 4, lane);
  dma_rows<D>(rs.q2, base + KV_Q2, t0, wv, lane);
  dma_rows<D>(rs.q2, base + KV_Q2, t0, wv + 4, lane);
#pragma unroll
  for (int i = 0; i < 4; ++i) dma_rows<DV>(rs.g, base + KV_G, t0, wv + 4 * i, lane);
  if (wv == 0)
    dma16(rs.vec, base + KV_VEC, (t0 + lane) * 16);
}
// Tile resident for every wave: this wave's loads of it are complete (the next tile's
// may still be in flight: 9 loads for wave 0, 8 for the others), then all waves meet.
__device__ __forceinline__ void kv_tile_barrier(bool next_in_flight, bool w0) {
  if (next_in_flight) {
    if (w0) vm_wait<9>();
    else vm_wait<8>();
  } else {
    vm_wait<0>();
  }
  barrier();
}

__global__ void __launch_bounds__(NT, 1) bwd_dkdv_kernel(
    const bf16_t* __restrict__ q1, const bf16_t* __restrict__ q2, const bf16_t* __restrict__ k1,
    const bf16_t* __restrict__ k2, const bf16_t* __restrict__ v, const bf16_t* __restrict__ gb,
    const f32x4* __restrict__ vec, const diffattn_lambda_state* __restrict__ lamst,
    bf16_t* __restrict__ dk1, bf16_t* __restrict__ dk2, bf16_t* __restrict__ dv, int BHK, int N,
    int G) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  using Sc = KvSched;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int m = lane & 31, h = lane >> 5;
  const int bid = blockIdx.x;
  // K/V head bhk (of B x Hkv); with grouped-query attention its G query heads are the
  // consecutive heads bhk G .. bhk G + G - 1, and their contributions to dK and dV add up
  // in the accumulators.
  const int bhk = bid % BHK;
  const int k0 = (bid / BHK) * BW;     // early key blocks see the most queries: first
  const int key = k0 + 32 * wv + m;
  const int64_t ho = static_cast<int64_t>(bhk) * N;   // K/V rows of this head
  KvRsrc rs;
  // Query tiles from the block's first key on: rows beyond N read as zero (and then
  // contribute nothing: their Q and G rows are zero).
  const int qt0 = k0 / TB;
  const int nT = (N + TB - 1) / TB - qt0;
  const uint32_t ldsu = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((LDS_AS char*)lds));
  const int lds0 = static_cast<int>(ldsu);

  // Tiles 0..2 of query head g on their way into the ring.
  auto start_head = [&](int g) {
    const int64_t qo = (static_cast<int64_t>(bhk) * G + g) * N;   // query head bhk G + g
    rs.q1 = rsrc_words(q1 + qo * D, N * D * 2);
    rs.q2 = rsrc_words(q2 + qo * D, N * D * 2);
    rs.g = rsrc_words(gb + qo * DV, N * DV * 2);
    rs.vec = rsrc_words(vec + qo, N * 16);
    kv_dma(rs, ldsu, 0, qt0 * TB, wv, lane);
    if (nT > 1) kv_dma(rs, ldsu, 1, (qt0 + 1) * TB, wv, lane);
    if (nT > 2) kv_dma(rs, ldsu, 2, (qt0 + 2) * TB, wv, lane);
  };
  // The first head's tiles travel together with the resident loads below.
  start_head(0);

  // Resident B operands (K^T and V^T columns of this lane's key), in the accumulation
  // registers.
  bf16x8 kr1[4], kr2[4], vr[8];
  {
    const bool ok = key < N;
    const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const u32x4 a = ok ? *reinterpret_cast<const u32x4*>(k1 + (ho + key) * D + 16 * i + 8 * h) : z;
      const u32x4 b = ok ? *reinterpret_cast<const u32x4*>(k2 + (ho + key) * D + 16 * i + 8 * h) : z;
      kr1[i] = as_bf16x8(a);
      kr2[i] = as_bf16x8(b);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const u32x4 a = ok ? *reinterpret_cast<const u32x4*>(v + (ho + key) * DV + 16 * i + 8 * h) : z;
      vr[i] = as_bf16x8(a);
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    pin_a(kr1[i]);
    pin_a(kr2[i]);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) pin_a(vr[i]);

  f32x16 adv[4], adk1[2], adk2[2];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
#pragma unroll
    for (int b = 0; b < 4; ++b) adv[b][j] = 0.f;
#pragma unroll
    for (int b = 0; b < 2; ++b) adk1[b][j] = adk2[b][j] = 0.f;
  }
#pragma unroll
  for (int b = 0; b < 4; ++b) pin_a(adv[b]);
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    pin_a(adk1[b]);
    pin_a(adk2[b]);
  }

  const LaneAddr la = lane_addr(lane);
  const int vb = 128 * h;   // per-row vectors of rows 8 h ..
  auto slot_of = [&](int j) { return lds0 + ((j >> 1) & (NSLOT - 1)) * KV_SLOT; };
#pragma clang loop unroll(disable)
  for (int g = 0; g < G; ++g) {
  // Every wave is done with the previous query head's tiles before the ring refills.
  if (g > 0) {
    barrier();
    start_head(g);
  }
  const float lam = lamst->lambda_f;
  const float c = kLog2e / 8.0f;   // log2(e) / sqrt(64)
  // Causal test: key > query for register e of sub-tile j  <=>  idx_of(e, 0) > kq - 32 j.
  const int kq = 32 * wv + m - 8 * h;

  // Pipeline state. Buffers by sub-tile parity: scores and dP (A -> B), packed P - lambda
  // P2, dS1, dS2 (B -> C). Per pair of score registers (by pair parity): the values its
  // later steps need.
  f32x16 S1[2], S2[2], dP[2];
  uint32_t pcw[2][8], g1w[2][8], g2w[2][8];
  float p1[2][2], p2[2][2], y1[2][2], y2[2][2], u[2][2], ww[2][2], dd2[2][2];
  u32x4 vecr[2][2];   // per-row vectors of the pair's two rows
  u32x2 trl[16], trh[16];   // transposing reads of the C products of the half-step
  u32x4 rr[16];             // row reads of its A products

  // One half-step j: products of C(j-1) (slots 0..15) and A(j+1) (16..31); vector work of
  // B(j): pair pr of score registers takes steps 0..3 in slots 4 pr .. 4 pr + 3 and steps
  // 4..7 in the next four slots (pair 7's in slots 0..3 of the next half-step, alongside
  // pair 0 of the next sub-tile):
  //   0: scale and subtract lse (4 fma), exp2 of p1[0]   1: exp2 p1[1], dP - D1
  //   2: exp2 p2[0], causal mask of p1                   3: exp2 p2[1], mask p2, dS1, pack
  //   4: lambda p2                                       5: D2 - dP
  //   6: dS2, pack                                       7: P1 - lambda P2, pack
  auto half = [&](auto masked, auto parity, int j) __attribute__((always_inline)) {
    constexpr bool MASKED = decltype(masked)::value;
    constexpr int PA = decltype(parity)::value;   // j & 1
    constexpr int PN = 1 - PA;                    // (j +- 1) & 1
    const int baseA = slot_of(j + 1);
    const int baseC = slot_of(j > 0 ? j - 1 : 0);
    const int baseB = slot_of(j);
    const int aA0 = baseA + la.rb[0], aA1 = baseA + la.rb[1];
    const int aC0 = baseC + la.tb[0], aC1 = baseC + la.tb[1];
    const int aN0 = baseB + la.tb[0], aN1 = baseB + la.tb[1];
    const int aV = baseB + vb, aVn = baseA + vb;
    const int dq = kq - 32 * j;
    auto slot = [&](auto kc) __attribute__((always_inline)) {
      constexpr int k = decltype(kc)::value;
      // ---- the product of slot k
      if constexpr (k < 16) {
        constexpr int t = kvc_t(k), b = kvc_b(k), ks = kvc_ks(k);
        const bf16x8 a = tr_operand(trl[k], trh[k]);
        if constexpr (t == 0) adv[b] = mfma(a, words(pcw[PN], ks), adv[b]);
        if constexpr (t == 1) adk1[b] = mfma(a, words(g1w[PN], ks), adk1[b]);
        if constexpr (t == 2) adk2[b] = mfma(a, words(g2w[PN], ks), adk2[b]);
      } else {
        constexpr int i = k - 16, kind = a_kind(i), kb = a_kb(i);
        const bf16x8 a = as_bf16x8(rr[i]);
        a_product<kind, kb>(S1[PN], S2[PN], dP[PN], a, kr1, kr2, vr);
      }
      __builtin_amdgcn_sched_barrier(0);
      // ---- LDS reads issued in slot k (order: transposing, row, vectors)
      if constexpr (k <= 15 - Sc::LT) {   // C(j-1), product k + LT
        constexpr int i = k + Sc::LT, t = kvc_t(i), b = kvc_b(i), ks = kvc_ks(i);
        constexpr int off = kv_toff(t) + REG * b + 1024 * (2 * PN + ks);
        trl[i] = rdtr<off>(aC0);
        trh[i] = rdtr<off>(aC1);
      }
      if constexpr (k >= Sc::SLOTS - Sc::LT) {   // C(j) of the next half-step, product i
        constexpr int i = k - (Sc::SLOTS - Sc::LT), t = kvc_t(i), b = kvc_b(i), ks = kvc_ks(i);
        constexpr int off = kv_toff(t) + REG * b + 1024 * (2 * PA + ks);
        trl[i] = rdtr<off>(aN0);
        trh[i] = rdtr<off>(aN1);
      }
      if constexpr (Sc::nrow(k)) {        // A(j+1), product k + LA - 16
        constexpr int i = k + Sc::LA - 16, kind = a_kind(i), kb = a_kb(i);
        constexpr int toff = kind == 0 ? KV_Q1 : (kind == 1 ? KV_Q2 : KV_G);
        constexpr int off = toff + REG * (kb >> 1) + 2048 * PN;
        rr[i] = rd128<off>((kb & 1) ? aA1 : aA0);
      }
      if constexpr (k % 4 == 1) {         // vectors of pair (k + 3) / 4 of B(j), or pair 0
        constexpr int pr = ((k + 3) / 4) % 8;   // of B(j + 1) in the last slots
        constexpr int e = 2 * pr, P = (k == 29) ? PN : PA;
        constexpr int o0 = KV_VEC + 512 * P + 16 * idx_of(e, 0);
        if constexpr (k == 29) {
          vecr[0][0] = rd128<o0>(aVn);
          vecr[0][1] = rd128<o0 + 16>(aVn);
        } else {
          vecr[pr & 1][0] = rd128<o0>(aV);
          vecr[pr & 1][1] = rd128<o0 + 16>(aV);
        }
      }
      // ---- vector work
      if constexpr (k == 1) s_guard(dP[PA]);
      {   // steps 0..3 of pair k / 4 of B(j)
        constexpr int pr = k / 4, st = k % 4, q = pr & 1, e = 2 * pr;
        if constexpr (st == 0) {
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            y1[q][i] = fmaf(S1[PA][e + i], c, -__uint_as_float(vecr[q][i][0]));
            y2[q][i] = fmaf(S2[PA][e + i], c, -__uint_as_float(vecr[q][i][1]));
          }
          p1[q][0] = fast_exp2(y1[q][0]);
          anchor(y1[q][1], y2[q][0], y2[q][1], p1[q][0]);
        }
        if constexpr (st == 1) {
          p1[q][1] = fast_exp2(y1[q][1]);
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            u[q][i] = dP[PA][e + i] - __uint_as_float(vecr[q][i][2]);
            dd2[q][i] = __uint_as_float(vecr[q][i][3]);
          }
          anchor(p1[q][1], u[q][0], u[q][1], dd2[q][0], dd2[q][1]);
        }
        if constexpr (st == 2) {
          p2[q][0] = fast_exp2(y2[q][0]);
          if constexpr (MASKED) {
#pragma unroll
            for (int i = 0; i < 2; ++i)
              if (idx_of(e + i, 0) < dq) p1[q][i] = 0.f;
          }
          anchor(p2[q][0], p1[q][0], p1[q][1]);
        }
        if constexpr (st == 3) {
          p2[q][1] = fast_exp2(y2[q][1]);
          if constexpr (MASKED) {
#pragma unroll
            for (int i = 0; i < 2; ++i)
              if (idx_of(e + i, 0) < dq) p2[q][i] = 0.f;
          }
          g1w[PA][pr] = pack_bf16x2(p1[q][0] * u[q][0], p1[q][1] * u[q][1]);
          anchor(p2[q][0], p2[q][1], g1w[PA][pr]);
        }
      }
      {   // steps 4..7 of the previous pair (pair 7 of B(j-1) in slots 0..3)
        constexpr int pr = (k / 4 + 7) % 8, st = k % 4, q = pr & 1, e = 2 * pr;
        constexpr int P = (k < 4) ? PN : PA;
        if constexpr (st == 0) {
          ww[q][0] = dd2[q][0] - dP[P][e];
          ww[q][1] = dd2[q][1] - dP[P][e + 1];
          anchor(ww[q][0], ww[q][1]);
        }
        if constexpr (st == 1) {
          g2w[P][pr] = pack_bf16x2(p2[q][0] * ww[q][0], p2[q][1] * ww[q][1]);
          anchor(g2w[P][pr]);
        }
        if constexpr (st == 2) {
          pcw[P][pr] = pack_bf16x2(fmaf(-lam, p2[q][0], p1[q][0]), fmaf(-lam, p2[q][1], p1[q][1]));
          anchor(pcw[P][pr]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    };
    static_for<0, Sc::SLOTS>(slot);
  };

  // Prologue: tile 0 resident, A(0), and the state a previous half-step would leave:
  // P(-1) = 0 (so C(-1), which reads tile 0's data, adds zero; pair 7 of B(-1) yields
  // zeros), the transposing reads of C(-1)'s first products and the vectors of B(0)'s
  // first pair in flight, in the order of the steady state.
  if (nT > 2) {
    if (wv == 0) vm_wait<18>();
    else vm_wait<16>();
  } else if (nT > 1) {
    if (wv == 0) vm_wait<9>();
    else vm_wait<8>();
  } else {
    vm_wait<0>();
  }
  barrier();
  {
    const int b0 = slot_of(0);
    u32x4 r[16];
    static_for<0, 16>([&](auto ic) __attribute__((always_inline)) {
      constexpr int i = decltype(ic)::value, kind = a_kind(i), kb = a_kb(i);
      constexpr int toff = kind == 0 ? KV_Q1 : (kind == 1 ? KV_Q2 : KV_G);
      r[i] = rd128<toff + REG * (kb >> 1)>(b0 + la.rb[kb & 1]);
    });
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    static_for<0, 16>([&](auto ic) __attribute__((always_inline)) {
      constexpr int i = decltype(ic)::value, kind = a_kind(i), kb = a_kb(i);
      a_product<kind, kb>(S1[0], S2[0], dP[0], as_bf16x8(r[i]), kr1, kr2, vr);
    });
    s_guard3(S1[0], S2[0], dP[0]);   // the first half-step reads them at once
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) pcw[1][i] = g1w[1][i] = g2w[1][i] = 0u;
#pragma unroll
  for (int i = 0; i < 2; ++i) p1[1][i] = p2[1][i] = dd2[1][i] = 0.f;
#pragma unroll
  for (int e = 0; e < 16; ++e) dP[1][e] = 0.f;
  {
    const int b0 = slot_of(0);
    const int a0 = b0 + la.tb[0], a1 = b0 + la.tb[1], av = b0 + vb;
    static_for<0, Sc::LT>([&](auto ic) __attribute__((always_inline)) {
      constexpr int i = decltype(ic)::value, t = kvc_t(i), b = kvc_b(i), ks = kvc_ks(i);
      constexpr int off = kv_toff(t) + REG * b + 1024 * (2 + ks);
      trl[i] = rdtr<off>(a0);
      trh[i] = rdtr<off>(a1);
      if constexpr (Sc::SLOTS - Sc::LT + i == 29) {
        vecr[0][0] = rd128<KV_VEC + 16 * idx_of(0, 0)>(av);
        vecr[0][1] = rd128<KV_VEC + 16 * idx_of(1, 0)>(av);
      }
    });
  }

  // Trips: half-steps 2T (A(2T+1) from tile T) and 2T+1 (A(2T+2) from tile T+1, after
  // its barrier, which also frees tile T-1's slot for tile T+3). Sub-tiles 0..3 (the
  // first two tiles) hold the causal diagonal band of this block's keys.
  auto trip = [&](auto masked, int T) __attribute__((always_inline)) {
    DIFFATTN_DEBUG_BARRIER();   // every wave runs the same trips
    half(masked, Int<0>{}, 2 * T);
    if (T + 1 < nT) {
      kv_tile_barrier(T + 2 < nT, wv == 0);
      if (T + 3 < nT) kv_dma(rs, ldsu, T + 3, (qt0 + T + 3) * TB, wv, lane);
    }
    half(masked, Int<1>{}, 2 * T + 1);
  };
  const int nmask = nT < 2 ? nT : 2;
  for (int T = 0; T < nmask; ++T) trip(Flag<true>{}, T);
  for (int T = 2; T < nT; ++T) trip(Flag<false>{}, T);
  // The last half-step's score products (of a sub-tile that does not exist) are not
  // read; keep their registers until the products have written them.
  s_guard3(S1[0], S2[0], dP[0]);

  // Drain: C of the last sub-tile (parity 1) and the last steps of its pair 7.
  {
    const int jl = 2 * nT - 1;
    const int bl = slot_of(jl);
    const int a0 = bl + la.tb[0], a1 = bl + la.tb[1];
    {
      constexpr int q = 1, e = 14;
      ww[q][0] = dd2[q][0] - dP[1][e];
      ww[q][1] = dd2[q][1] - dP[1][e + 1];
      g2w[1][7] = pack_bf16x2(p2[q][0] * ww[q][0], p2[q][1] * ww[q][1]);
      pcw[1][7] = pack_bf16x2(fmaf(-lam, p2[q][0], p1[q][0]), fmaf(-lam, p2[q][1], p1[q][1]));
    }
    static_for<Sc::LT, 16>([&](auto ic) __attribute__((always_inline)) {
      constexpr int i = decltype(ic)::value, t = kvc_t(i), b = kvc_b(i), ks = kvc_ks(i);
      constexpr int off = kv_toff(t) + REG * b + 1024 * (2 + ks);
      trl[i] = rdtr<off>(a0);
      trh[i] = rdtr<off>(a1);
    });
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    static_for<0, 16>([&](auto ic) __attribute__((always_inline)) {
      constexpr int i = decltype(ic)::value, t = kvc_t(i), b = kvc_b(i), ks = kvc_ks(i);
      const bf16x8 a = tr_operand(trl[i], trh[i]);
      if constexpr (t == 0) adv[b] = mfma(a, words(pcw[1], ks), adv[b]);
      if constexpr (t == 1) adk1[b] = mfma(a, words(g1w[1], ks), adk1[b]);
      if constexpr (t == 2) adk2[b] = mfma(a, words(g2w[1], ks), adk2[b]);
    });
  }
  }   // query heads of the group

  // Stores: register j of block b holds channel 32 b + 8 (j / 4) + 4 h + j % 4 of the key.
  // Stores through LDS, in this wave's region of the ring once every wave is done with it
  // (no tile load is in flight after the last tile's barrier).
  barrier();
  {
    const float s = 0.125f;  // 1 / sqrt(64)
    // Map 2's score gradients were accumulated without their factor lambda (the same for
    // every score): dS2 = lambda P2 (D2 - dP).
    const float s2 = s * lamst->lambda_f;
    const int sv = lds0 + wv * KV_STAGE, sk1 = sv + stage_bytes<DV>(), sk2 = sk1 + stage_bytes<D>();
#pragma unroll
    for (int b = 0; b < 4; ++b) {
#pragma unroll
      for (int jg = 0; jg < 4; ++jg) {
        u32x2 pk = {pack_bf16x2(adv[b][4 * jg], adv[b][4 * jg + 1]),
                    pack_bf16x2(adv[b][4 * jg + 2], adv[b][4 * jg + 3])};
        stage_put<DV>(sv, m, h, b, jg, pk);
      }
    }
#pragma unroll
    for (int b = 0; b < 2; ++b) {
#pragma unroll
      for (int jg = 0; jg < 4; ++jg) {
        u32x2 pa = {pack_bf16x2(s * adk1[b][4 * jg], s * adk1[b][4 * jg + 1]),
                    pack_bf16x2(s * adk1[b][4 * jg + 2], s * adk1[b][4 * jg + 3])};
        u32x2 pb = {pack_bf16x2(s2 * adk2[b][4 * jg], s2 * adk2[b][4 * jg + 1]),
                    pack_bf16x2(s2 * adk2[b][4 * jg + 2], s2 * adk2[b][4 * jg + 3])};
        stage_put<D>(sk1, m, h, b, jg, pa);
        stage_put<D>(sk2, m, h, b, jg, pb);
      }
    }
    const int r0 = k0 + 32 * wv, valid = N - r0;
    stage_flush<DV>(sv, dv + (ho + r0) * DV, valid, lane);
    stage_flush<D>(sk1, dk1 + (ho + r0) * D, valid, lane);
    stage_flush<D>(sk2, dk2 + (ho + r0) * D, valid, lane);
  }
}

// ------------------------------------------------------------------------ dQ
// C products of a half-step (slot order): dQ1^T regions 0..1, dQ2^T 0..1 for k-step 0, then
// k-step 1. Map 0 = K1, 1 = K2.
__host__ __device__ constexpr int qc_map(int i) { return (i >> 1) & 1; }
__host__ __device__ constexpr int qc_b(int i) { return i & 1; }
__host__ __device__ constexpr int qc_ks(int i) { return i >> 2; }

struct QRsrc {
  u32x4 k1, k2, v;
};

// This wave's share of key tile `tile` (rows t0 ..): blocks w, w + 4 of K1 and K2, w + 4 i
// of V (8 loads).
// A tile is 32 blocks of 1 KiB (K1 8, K2 8, V 16); wave wv of the 8 moves K1 and K2 block
// wv and V blocks wv and wv + 8: four loads per wave per tile.
__device__ __forceinline__ void q_dma(const QRsrc& rs, uint32_t lds, int tile, int t0,
                                      int wv, int lane) {
  const uint32_t base = lds + (tile % NSLOT) * Q_SLOT;
  dma_rows<D>(rs.k1, base + Q_K1, t0, wv, lane);
  dma_rows<D>(rs.k2, base + Q_K2, t0, wv, lane);
  dma_rows<DV>(rs.v, base + Q_V, t0, wv, lane);
  dma_rows<DV>(rs.v, base + Q_V, t0, wv + 8, lane);
}
__device__ __forceinline__ void q_tile_barrier(bool next_in_flight) {
  if (next_in_flight) vm_wait<4>();
  else vm_wait<0>();
  barrier();
}

__global__ void __launch_bounds__(NTQ, 1) bwd_dq_kernel(
    const bf16_t* __restrict__ q1, const bf16_t* __restrict__ q2, const bf16_t* __restrict__ k1,
    const bf16_t* __restrict__ k2, const bf16_t* __restrict__ v, const bf16_t* __restrict__ gb,
    const f32x4* __restrict__ vec, const diffattn_lambda_state* __restrict__ lamst,
    bf16_t* __restrict__ dq1, bf16_t* __restrict__ dq2, int BH, int N, int nqb, int G) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  using Sc = QSched;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int m = lane & 31, h = lane >> 5;
  const int bid = blockIdx.x;
  const int bh = bid % BH;
  const int q0 = (nqb - 1 - bid / BH) * BWQ;   // late query blocks see the most keys: first
  const int q = q0 + 32 * wv + m;
  const bool qok = q < N;
  const int64_t ho = static_cast<int64_t>(bh) * N;

  QRsrc rs;
  // K/V head of this query head (G consecutive query heads share one).
  const int64_t kvo = static_cast<int64_t>(bh / G) * N;
  rs.k1 = rsrc_words(k1 + kvo * D, N * D * 2);
  rs.k2 = rsrc_words(k2 + kvo * D, N * D * 2);
  rs.v = rsrc_words(v + kvo * DV, N * DV * 2);
  // Key tiles 0 .. up to the block's last query (keys beyond N read as zero and are
  // masked: they follow every query).
  const int kend = min(N, q0 + BWQ);
  const int nT = (kend + TB - 1) / TB;
  const uint32_t ldsu = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((LDS_AS char*)lds));
  const int lds0 = static_cast<int>(ldsu);

  // Resident B operands (Q^T and G^T columns of this lane's query), in the accumulation
  // registers; the query's per-row vector in vector registers.
  bf16x8 qr1[4], qr2[4], gr[8];
  float L1 = 0.f, L2 = 0.f, D1 = 0.f, D2 = 0.f;
  {
    const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const u32x4 a = qok ? *reinterpret_cast<const u32x4*>(q1 + (ho + q) * D + 16 * i + 8 * h) : z;
      const u32x4 b = qok ? *reinterpret_cast<const u32x4*>(q2 + (ho + q) * D + 16 * i + 8 * h) : z;
      qr1[i] = as_bf16x8(a);
      qr2[i] = as_bf16x8(b);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const u32x4 a = qok ? *reinterpret_cast<const u32x4*>(gb + (ho + q) * DV + 16 * i + 8 * h) : z;
      gr[i] = as_bf16x8(a);
    }
    if (qok) {
      const f32x4 vv = vec[ho + q];
      L1 = vv[0];
      L2 = vv[1];
      D1 = vv[2];
      D2 = vv[3];
    }
  }
  q_dma(rs, ldsu, 0, 0, wv, lane);
  if (nT > 1) q_dma(rs, ldsu, 1, TB, wv, lane);
  if (nT > 2) q_dma(rs, ldsu, 2, 2 * TB, wv, lane);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    pin_a(qr1[i]);
    pin_a(qr2[i]);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) pin_a(gr[i]);

  f32x16 aq1[2], aq2[2];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
#pragma unroll
    for (int b = 0; b < 2; ++b) aq1[b][j] = aq2[b][j] = 0.f;
  }
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    pin_a(aq1[b]);
    pin_a(aq2[b]);
  }

  const LaneAddr la = lane_addr(lane);
  auto slot_of = [&](int j) { return lds0 + ((j >> 1) & (NSLOT - 1)) * Q_SLOT; };
  const float c = kLog2e / 8.0f;
  // Causal test: key > query for register e of sub-tile j  <=>  idx_of(e, 0) > qk - 32 j.
  const int qk = 32 * wv + m - 8 * h + q0;

  f32x16 S1[2], S2[2], dP[2];
  uint32_t g1w[2][8], g2w[2][8];
  float p1[2][2], p2[2][2], y1[2][2], y2[2][2], u[2][2], ww[2][2];
  u32x2 trl[8], trh[8];
  u32x4 rr[16];

  // One half-step j: products of C(j-1) (slots 0..7) and A(j+1) (8..23); vector work of
  // B(j): pair pr of score registers takes steps 0..2 in slots 3 pr .. 3 pr + 2 and steps
  // 3..5 in the next three (pair 7's in slots 0..2 of the next half-step):
  //   0: scale and subtract lse (4 fma), exp2 p1[0]
  //   1: exp2 p1[1], exp2 p2[0], dP - D1, causal mask of p1
  //   2: exp2 p2[1], mask p2, dS1, pack         3: lambda p2
  //   4: D2 - dP                                5: dS2, pack
  auto half = [&](auto masked, auto parity, int j) __attribute__((always_inline)) {
    constexpr bool MASKED = decltype(masked)::value;
    constexpr int PA = decltype(parity)::value;
    constexpr int PN = 1 - PA;
    const int baseA = slot_of(j + 1);
    const int baseC = slot_of(j > 0 ? j - 1 : 0);
    const int baseB = slot_of(j);
    const int aA0 = baseA + la.rb[0], aA1 = baseA + la.rb[1];
    const int aC0 = baseC + la.tb[0], aC1 = baseC + la.tb[1];
    const int aN0 = baseB + la.tb[0], aN1 = baseB + la.tb[1];
    const int dk = qk - 32 * j;
    auto slot = [&](auto kc) __attribute__((always_inline)) {
      constexpr int k = decltype(kc)::value;
      if constexpr (k < 8) {
        constexpr int mp = qc_map(k), b = qc_b(k), ks = qc_ks(k);
        const bf16x8 a = tr_operand(trl[k], trh[k]);
        if constexpr (mp == 0) aq1[b] = mfma(a, words(g1w[PN], ks), aq1[b]);
        else aq2[b] = mfma(a, words(g2w[PN], ks), aq2[b]);
      } else {
        constexpr int i = k - 8, kind = a_kind(i), kb = a_kb(i);
        const bf16x8 a = as_bf16x8(rr[i]);
        a_product<kind, kb>(S1[PN], S2[PN], dP[PN], a, qr1, qr2, gr);
      }
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (k <= 7 - Sc::LT) {   // C(j-1), product k + LT
        constexpr int i = k + Sc::LT, mp = qc_map(i), b = qc_b(i), ks = qc_ks(i);
        constexpr int off = (mp ? Q_K2 : Q_K1) + REG * b + 1024 * (2 * PN + ks);
        trl[i] = rdtr<off>(aC0);
        trh[i] = rdtr<off>(aC1);
      }
      if constexpr (k >= Sc::SLOTS - Sc::LT) {   // C(j) of the next half-step
        constexpr int i = k - (Sc::SLOTS - Sc::LT), mp = qc_map(i), b = qc_b(i), ks = qc_ks(i);
        constexpr int off = (mp ? Q_K2 : Q_K1) + REG * b + 1024 * (2 * PA + ks);
        trl[i] = rdtr<off>(aN0);
        trh[i] = rdtr<off>(aN1);
      }
      if constexpr (Sc::nrow(k)) {        // A(j+1), product k + LA - 8
        constexpr int i = k + Sc::LA - 8, kind = a_kind(i), kb = a_kb(i);
        constexpr int toff = kind == 0 ? Q_K1 : (kind == 1 ? Q_K2 : Q_V);
        constexpr int off = toff + REG * (kb >> 1) + 2048 * PN;
        rr[i] = rd128<off>((kb & 1) ? aA1 : aA0);
      }
      if constexpr (k == 1) s_guard(dP[PA]);
      {   // steps 0..2 of pair k / 3 of B(j)
        constexpr int pr = k / 3, st = k % 3, qq = pr & 1, e = 2 * pr;
        if constexpr (st == 0) {
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            y1[qq][i] = fmaf(S1[PA][e + i], c, -L1);
            y2[qq][i] = fmaf(S2[PA][e + i], c, -L2);
          }
          p1[qq][0] = fast_exp2(y1[qq][0]);
          anchor(y1[qq][1], y2[qq][0], y2[qq][1], p1[qq][0]);
        }
        if constexpr (st == 1) {
          p1[qq][1] = fast_exp2(y1[qq][1]);
          p2[qq][0] = fast_exp2(y2[qq][0]);
#pragma unroll
          for (int i = 0; i < 2; ++i) u[qq][i] = dP[PA][e + i] - D1;
          if constexpr (MASKED) {
#pragma unroll
            for (int i = 0; i < 2; ++i)
              if (idx_of(e + i, 0) > dk) p1[qq][i] = 0.f;
          }
          anchor(p1[qq][0], p1[qq][1], p2[qq][0], u[qq][0], u[qq][1]);
        }
        if constexpr (st == 2) {
          p2[qq][1] = fast_exp2(y2[qq][1]);
          if constexpr (MASKED) {
#pragma unroll
            for (int i = 0; i < 2; ++i)
              if (idx_of(e + i, 0) > dk) p2[qq][i] = 0.f;
          }
          g1w[PA][pr] = pack_bf16x2(p1[qq][0] * u[qq][0], p1[qq][1] * u[qq][1]);
          anchor(p2[qq][0], p2[qq][1], g1w[PA][pr]);
        }
      }
      {   // steps 3..5 of the previous pair (pair 7 of B(j-1) in slots 0..2)
        constexpr int pr = (k / 3 + 7) % 8, st = k % 3, qq = pr & 1, e = 2 * pr;
        constexpr int P = (k < 3) ? PN : PA;
        if constexpr (st == 0) {
          ww[qq][0] = D2 - dP[P][e];
          ww[qq][1] = D2 - dP[P][e + 1];
          anchor(ww[qq][0], ww[qq][1]);
        }
        if constexpr (st == 1) {
          g2w[P][pr] = pack_bf16x2(p2[qq][0] * ww[qq][0], p2[qq][1] * ww[qq][1]);
          anchor(g2w[P][pr]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    };
    static_for<0, Sc::SLOTS>(slot);
  };

  // Prologue (as for dK/dV): tile 0 resident, A(0), P(-1) = 0, C(-1)'s first
  // transposing reads in flight.
  if (nT > 2) vm_wait<8>();
  else if (nT > 1) vm_wait<4>();
  else vm_wait<0>();
  barrier();
  {
    const int b0 = slot_of(0);
    u32x4 r[16];
    static_for<0, 16>([&](auto ic) __attribute__((always_inline)) {
      constexpr int i = decltype(ic)::value, kind = a_kind(i), kb = a_kb(i);
      constexpr int toff = kind == 0 ? Q_K1 : (kind == 1 ? Q_K2 : Q_V);
      r[i] = rd128<toff + REG * (kb >> 1)>(b0 + la.rb[kb & 1]);
    });
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    static_for<0, 16>([&](auto ic) __attribute__((always_inline)) {
      constexpr int i = decltype(ic)::value, kind = a_kind(i), kb = a_kb(i);
      a_product<kind, kb>(S1[0], S2[0], dP[0], as_bf16x8(r[i]), qr1, qr2, gr);
    });
    s_guard3(S1[0], S2[0], dP[0]);   // the first half-step reads them at once
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) g1w[1][i] = g2w[1][i] = 0u;
#pragma unroll
  for (int i = 0; i < 2; ++i) p2[1][i] = 0.f;
#pragma unroll
  for (int e = 0; e < 16; ++e) dP[1][e] = 0.f;
  {
    const int b0 = slot_of(0);
    const int a0 = b0 + la.tb[0], a1 = b0 + la.tb[1];
    static_for<0, Sc::LT>([&](auto ic) __attribute__((always_inline)) {
      constexpr int i = decltype(ic)::value, mp = qc_map(i), b = qc_b(i), ks = qc_ks(i);
      constexpr int off = (mp ? Q_K2 : Q_K1) + REG * b + 1024 * (2 + ks);
      trl[i] = rdtr<off>(a0);
      trh[i] = rdtr<off>(a1);
    });
  }

  // Trips as for dK/dV; the causal band (keys q0 .. q0 + 255) is in the last four tiles.
  auto trip = [&](auto masked, int T) __attribute__((always_inline)) {
    DIFFATTN_DEBUG_BARRIER();   // every wave runs the same trips
    half(masked, Int<0>{}, 2 * T);
    if (T + 1 < nT) {
      q_tile_barrier(T + 2 < nT);
      if (T + 3 < nT) q_dma(rs, ldsu, T + 3, (T + 3) * TB, wv, lane);
    }
    half(masked, Int<1>{}, 2 * T + 1);
  };
  const int nfree = nT > 4 ? nT - 4 : 0;
  for (int T = 0; T < nfree; ++T) trip(Flag<false>{}, T);
  for (int T = nfree; T < nT; ++T) trip(Flag<true>{}, T);
  // The last half-step's score products (of a sub-tile that does not exist) are not
  // read; keep their registers until the products have written them.
  s_guard3(S1[0], S2[0], dP[0]);

  // Drain: C of the last sub-tile (parity 1) and the last steps of its pair 7.
  {
    const int jl = 2 * nT - 1;
    const int bl = slot_of(jl);
    const int a0 = bl + la.tb[0], a1 = bl + la.tb[1];
    {
      constexpr int qq = 1, e = 14;
      ww[qq][0] = D2 - dP[1][e];
      ww[qq][1] = D2 - dP[1][e + 1];
      g2w[1][7] = pack_bf16x2(p2[qq][0] * ww[qq][0], p2[qq][1] * ww[qq][1]);
    }
    static_for<Sc::LT, 8>([&](auto ic) __attribute__((always_inline)) {
      constexpr int i = decltype(ic)::value, mp = qc_map(i), b = qc_b(i), ks = qc_ks(i);
      constexpr int off = (mp ? Q_K2 : Q_K1) + REG * b + 1024 * (2 + ks);
      trl[i] = rdtr<off>(a0);
      trh[i] = rdtr<off>(a1);
    });
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    static_for<0, 8>([&](auto ic) __attribute__((always_inline)) {
      constexpr int i = decltype(ic)::value, mp = qc_map(i), b = qc_b(i), ks = qc_ks(i);
      const bf16x8 a = tr_operand(trl[i], trh[i]);
      if constexpr (mp == 0) aq1[b] = mfma(a, words(g1w[1], ks), aq1[b]);
      else aq2[b] = mfma(a, words(g2w[1], ks), aq2[b]);
    });
  }

  // Stores through LDS, in this wave's region of the ring once every wave is done with it
  // (no tile load is in flight after the last tile's barrier).
  barrier();
  {
    const float s = 0.125f;  // 1 / sqrt(64)
    // Map 2's score gradients were accumulated without their factor lambda (the same for
    // every score): dS2 = lambda P2 (D2 - dP).
    const float s2 = s * lamst->lambda_f;
    const int s1 = lds0 + wv * Q_STAGE, s2b = s1 + stage_bytes<D>();
#pragma unroll
    for (int b = 0; b < 2; ++b) {
#pragma unroll
      for (int jg = 0; jg < 4; ++jg) {
        u32x2 pa = {pack_bf16x2(s * aq1[b][4 * jg], s * aq1[b][4 * jg + 1]),
                    pack_bf16x2(s * aq1[b][4 * jg + 2], s * aq1[b][4 * jg + 3])};
        u32x2 pb = {pack_bf16x2(s2 * aq2[b][4 * jg], s2 * aq2[b][4 * jg + 1]),
                    pack_bf16x2(s2 * aq2[b][4 * jg + 2], s2 * aq2[b][4 * jg + 3])};
        stage_put<D>(s1, m, h, b, jg, pa);
        stage_put<D>(s2b, m, h, b, jg, pb);
      }
    }
    const int r0 = q0 + 32 * wv, valid = N - r0;
    stage_flush<D>(s1, dq1 + (ho + r0) * D, valid, lane);
    stage_flush<D>(s2b, dq2 + (ho + r0) * D, valid, lane);
  }
}

}  // namespace bwd

// Workspace (floats): bf16 G [rows, 128] (64 floats per row), the per-row vector
// (lse1 log2 e, lse2 log2 e, D1, D2) [rows, 4], and one partial sum of D2 per 64 rows.
// Workspace (float32 words): G in bf16 [rows, 2d] | per-row vectors [rows, 4] |
// D2 partials [nparts, padded to 4] | weight-gradient partials [nparts, 2d] | 64 spare;
// nparts = B H ceil(N / 64) (one per bwd_pre_kernel workgroup).
size_t bwd_workspace_floats(int64_t B, int64_t H, int64_t N, int d) {
  (void)d;
  const int64_t rows = B * H * N;
  const int64_t nparts = B * H * ((N + 63) / 64);
  return static_cast<size_t>(rows) * (bwd::DV / 2 + 4) +
         static_cast<size_t>((nparts + 3) / 4 * 4) + static_cast<size_t>(nparts) * bwd::DV + 64;
}

hipError_t launch_bwd_bf16(const BwdArgs& a, hipStream_t s) {
  using namespace bwd;
  static std::atomic<uint64_t> attr_done{0};
  const hipError_t ea = once_per_device(attr_done, [] {
    hipError_t r = hipFuncSetAttribute(reinterpret_cast<const void*>(bwd_dkdv_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, KV_LDS);
    if (r == hipSuccess)
      r = hipFuncSetAttribute(reinterpret_cast<const void*>(bwd_dq_kernel),
                              hipFuncAttributeMaxDynamicSharedMemorySize, Q_LDS);
    return r;
  });
  if (ea != hipSuccess) return ea;
  const int64_t rows = a.B * a.H * a.N;
  const int64_t nchunk = (a.N + 63) / 64;
  const int64_t nparts = a.B * a.H * nchunk;
  bf16_t* gbuf = reinterpret_cast<bf16_t*>(a.ws);
  f32x4* vec = reinterpret_cast<f32x4*>(a.ws + rows * (DV / 2));
  float* part = a.ws + rows * (DV / 2 + 4);
  float* pw = part + (nparts + 3) / 4 * 4;
  if (rows > 0) {
    hipLaunchKernelGGL(bwd_pre_kernel, dim3(static_cast<unsigned>(nparts)), dim3(256), 0, s,
                       a.saved.o1, a.saved.o2, a.saved.rstd, a.saved.lse1, a.saved.lse2,
                       static_cast<const bf16_t*>(a.dout), a.lam, a.rms_weight, a.d_attn, gbuf,
                       vec, part, reinterpret_cast<f32x4*>(pw), a.N, a.H, nchunk,
                       a.dout_bnh ? 1 : 0);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int BH = static_cast<int>(a.B * a.H);
    const int N = static_cast<int>(a.N);
    const int nb = static_cast<int>((a.N + BW - 1) / BW);
    const int BHK = BH / a.G;
    hipLaunchKernelGGL(bwd_dkdv_kernel, dim3(static_cast<unsigned>(BHK * nb)), dim3(NT), KV_LDS,
                       s, static_cast<const bf16_t*>(a.q1), static_cast<const bf16_t*>(a.q2),
                       static_cast<const bf16_t*>(a.k1), static_cast<const bf16_t*>(a.k2),
                       static_cast<const bf16_t*>(a.v), gbuf, vec, a.lam,
                       static_cast<bf16_t*>(a.dk1), static_cast<bf16_t*>(a.dk2),
                       static_cast<bf16_t*>(a.dv), BHK, N, a.G);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int nbq = static_cast<int>((a.N + BWQ - 1) / BWQ);
    hipLaunchKernelGGL(bwd_dq_kernel, dim3(static_cast<unsigned>(BH * nbq)), dim3(NTQ), Q_LDS, s,
                       static_cast<const bf16_t*>(a.q1), static_cast<const bf16_t*>(a.q2),
                       static_cast<const bf16_t*>(a.k1), static_cast<const bf16_t*>(a.k2),
                       static_cast<const bf16_t*>(a.v), gbuf, vec, a.lam,
                       static_cast<bf16_t*>(a.dq1), static_cast<bf16_t*>(a.dq2), BH, N, nbq, a.G);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(lambda_grad_kernel, dim3(1), dim3(1024), 0, s, part, rows > 0 ? nparts : 0,
                     a.lam, a.lq1, a.lk1, a.lq2, a.lk2, a.dlq1, a.dlk1, a.dlq2, a.dlk2, a.d);
  if (a.d_rms_weight && a.H > 0) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // With no rows (B = 0 or N = 0) the sums are empty and the gradient is zero.
    hipLaunchKernelGGL(rms_weight_grad_kernel, dim3(static_cast<unsigned>(a.H), DV / WG_CH),
                       dim3(WG_GROUPS * WG_CH), 0, s,
                       pw, rows > 0 ? a.B : 0, a.H, nchunk, a.d_rms_weight);
  }
  return hipGetLastError();
}

}  // namespace diffattn
