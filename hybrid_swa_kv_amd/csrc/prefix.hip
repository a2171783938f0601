// Window-safe prefix length of a sliding-window KV pool (integer, exact).
//
// A reused prefix of length l needs the sliding-window KV of its last min(l, W)
// positions; position p is present when its ring slot p mod W still holds p.
// Per sequence the answer is the largest l <= match_len that satisfies this,
// computed in closed form from three reductions over the W slots:
//   * r: the first slot s that does not hold position s (positions 0..r-1 are
//     present, so every l <= min(r, match_len) is safe);
//   * for l >= W the W needed positions are one per slot, so the slots must hold
//     exactly W consecutive positions ending at l - 1: every slot holds a
//     position p >= 0 with p mod W == s, and max - min == W - 1; then
//     l = max + 1 (if <= match_len).
// One workgroup per sequence.
#include <climits>

#include "common.hpp"
#include "kernels.hpp"

namespace hsk {

namespace {

constexpr int WS_THREADS = 256;

__global__ __launch_bounds__(WS_THREADS) void window_safe_kernel(WindowSafeArgs a) {
  __shared__ int red_r[WS_THREADS / 64], red_min[WS_THREADS / 64], red_max[WS_THREADS / 64];
  __shared__ int red_bad[WS_THREADS / 64];
  const int b = blockIdx.x;
  const int W = a.W;
  const int32_t* sp = a.slot_pos + (size_t)b * W;
  int r = W, pmin = INT_MAX, pmax = -1, bad = 0;
  for (int s = threadIdx.x; s < W; s += WS_THREADS) {
    const int p = sp[s];
    if (p != s) r = min(r, s);
    bad |= (p < 0) || (p % W != s);
    pmin = min(pmin, p);
    pmax = max(pmax, p);
  }
  // wave reductions, then across the four waves
  for (int o = 32; o >= 1; o >>= 1) {
    r = min(r, __shfl_xor(r, o));
    pmin = min(pmin, __shfl_xor(pmin, o));
    pmax = max(pmax, __shfl_xor(pmax, o));
    bad |= __shfl_xor(bad, o);
  }
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    red_r[w] = r;
    red_min[w] = pmin;
    red_max[w] = pmax;
    red_bad[w] = bad;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int i = 1; i < WS_THREADS / 64; ++i) {
      r = min(r, red_r[i]);
      pmin = min(pmin, red_min[i]);
      pmax = max(pmax, red_max[i]);
      bad |= red_bad[i];
    }
    const int M = a.match_len[b];
    const bool window = !bad && pmax - pmin == W - 1;
    const int la = (window && pmax < M) ? pmax + 1 : 0;  // pmax + 1 <= M
    const int lb = min(r, M);
    a.safe_len[b] = max(la, max(lb, 0));
  }
}

}  // namespace

hipError_t launch_window_safe(const WindowSafeArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(window_safe_kernel, dim3(a.B), dim3(WS_THREADS), 0, s, a);
  return hipGetLastError();
}

}  // namespace hsk
