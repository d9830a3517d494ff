// In-place append of one generated token to the K1/K2/V decode caches (bf16, d = 64).
//
// In autoregressive serving the cache grows by one token of K1, K2 and V per generated
// token and is then read whole by the decode step (priorstack.com, "Multi-Head Latent
// Attention: Scaling LLM Serving Throughput via Low-Rank KV Compression", section "The
// Memory Wall: Why the KV Cache Constrains LLM Serving"). This kernel is the write half of
// that step: for sequence b with n = cache_len[b] < L it copies the new rows of every head
// into cache row n and sets cache_len[b] = n + 1, so that a following decode call sees the
// new token as its query position.
//
// One workgroup per sequence: its threads read the length once, copy the H x 512 bytes
// (K1 and K2 rows of 128 B, V rows of 256 B) with 16-byte accesses, and only after a
// workgroup barrier does one thread store the new length, so no copy can see it.
#include "common.h"
#include "launch.h"

namespace diffattn {
namespace app {

constexpr int D = 64;
constexpr int DV = 128;
constexpr int NT = 256;

__global__ void __launch_bounds__(NT) cache_append_kernel(
    const u32x4* __restrict__ k1n, const u32x4* __restrict__ k2n, const u32x4* __restrict__ vn,
    u32x4* __restrict__ k1c, u32x4* __restrict__ k2c, u32x4* __restrict__ vc,
    int32_t* __restrict__ cache_len, int H, int64_t L) {
  __shared__ int32_t len_s;
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  if (tid == 0) len_s = cache_len[b];
  __syncthreads();
  const int64_t n = len_s < 0 ? 0 : len_s;
  if (n >= L) return;   // full cache: nothing written, length unchanged
  // Per head: 8 chunks of 16 B for each K row, 16 for the V row.
  constexpr int KC = D * 2 / 16, VC = DV * 2 / 16, PER = 2 * KC + VC;
  for (int i = tid; i < H * PER; i += NT) {
    const int h = i / PER, c = i % PER;
    const int64_t bh = static_cast<int64_t>(b) * H + h;
    if (c < KC) {
      k1c[(bh * L + n) * KC + c] = k1n[bh * KC + c];
    } else if (c < 2 * KC) {
      k2c[(bh * L + n) * KC + (c - KC)] = k2n[bh * KC + (c - KC)];
    } else {
      vc[(bh * L + n) * VC + (c - 2 * KC)] = vn[bh * VC + (c - 2 * KC)];
    }
  }
  __syncthreads();
  if (tid == 0) cache_len[b] = static_cast<int32_t>(n + 1);
}

}  // namespace app

hipError_t launch_cache_append_bf16(const AppendArgs& a, hipStream_t s) {
  using namespace app;
  hipLaunchKernelGGL(cache_append_kernel, dim3(static_cast<unsigned>(a.B)), dim3(NT), 0, s,
                     static_cast<const u32x4*>(a.k1n), static_cast<const u32x4*>(a.k2n),
                     static_cast<const u32x4*>(a.vn), static_cast<u32x4*>(a.k1c),
                     static_cast<u32x4*>(a.k2c), static_cast<u32x4*>(a.vc), a.cache_len,
                     static_cast<int>(a.H), a.L);
  return hipGetLastError();
}

}  // namespace diffattn
