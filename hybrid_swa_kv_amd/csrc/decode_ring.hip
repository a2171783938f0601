// One-token decode against a sliding-window ring buffer (bandwidth bound).
//
// One workgroup per (sequence, KV head, group of up to 16 query heads); its 4
// waves take interleaved 32-slot chunks of the ring and run the 16x16x32 MFMA
// decode of decode_mfma.hpp (heads on the MFMA N axis), then merge their
// (max, sum, acc) states through LDS behind a single barrier.  Every load of the
// ring is issued at the start of a chunk, so one HBM round trip covers the
// 128-slot window.  The new token's K/V is written to slot pos mod W and used
// from k_new/v_new (the stale slot is never read); slots whose position would be
// negative (ring not yet full) are neither read nor attended.
#include "common.hpp"
#include "decode_mfma.hpp"
#include "kernels.hpp"

namespace hsk {

namespace {

constexpr int RD_THREADS = 256;

template <int D>
__global__ __launch_bounds__(RD_THREADS) void ring_decode_kernel(RingDecodeArgs a) {
  __shared__ float sm_m[4][16], sm_l[4][16];
  __shared__ float sm_o[4][16][D];

  const int G = a.Hq / a.Hkv;
  const int HG = G < 16 ? G : 16;  // heads served by this workgroup
  const int nhg = G / HG;
  const int hg = blockIdx.x % nhg;
  const int g = (blockIdx.x / nhg) % a.Hkv;
  const int b = blockIdx.x / (nhg * a.Hkv);
  const int t = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int W = a.W;
  const int h0 = g * G + hg * HG;
  // No branch on pos before the ring loads: their addresses do not depend on it,
  // only the masks do, so the pos load and the ring loads travel together.  A
  // negative pos (a violated precondition) attends nothing, writes no slot and
  // yields zeros.
  const int p = a.pos[b];
  const bool ok = p >= 0;
  const int slot = ok ? p % W : 0;
  const size_t kvoff = (size_t)b * a.Hkv + g;
  uint16_t* rk = a.ring_k + kvoff * (size_t)W * D;
  uint16_t* rv = a.ring_v + kvoff * (size_t)W * D;
  const uint16_t* kn = a.k_new + kvoff * D;
  const uint16_t* vn = a.v_new + kvoff * D;
  DecodeWave<D> st;
  st.init(a.q + ((size_t)b * a.Hq + h0) * D, HG);
  const RingRows<D> rows{rk, rv, kn, vn, W, slot, ok ? p : -1};
  for (int c0 = 32 * w; c0 < W; c0 += 128) st.template chunk<false>(rows, c0, a.scale_log2, 1.f);

  st.stash(sm_m, sm_l, sm_o, w, HG);
  __syncthreads();
  // append (after every read of the ring in this workgroup): the first head
  // group's workgroup writes the new token into its slot
  if (ok && hg == 0 && t < D / 8) {
    *(uint4*)(rk + (size_t)slot * D + 8 * t) = *(const uint4*)(kn + 8 * t);
    *(uint4*)(rv + (size_t)slot * D + 8 * t) = *(const uint4*)(vn + 8 * t);
  }
  if (ok && hg == 0 && g == 0 && t == 0 && a.slot_out) a.slot_out[b] = slot;
  for (int e = t; e < HG * D; e += RD_THREADS) {
    const int head = e / D, d = e % D;
    float M, Ls;
    const float O = merge_waves<4, D>(sm_m, sm_l, sm_o, head, d, M, Ls);
    a.out[((size_t)b * a.Hq + h0 + head) * D + d] = f32_to_bf16(ok ? O / Ls : 0.f);
  }
}

}  // namespace

hipError_t launch_ring_decode(const RingDecodeArgs& a, hipStream_t s) {
  const int G = a.Hq / a.Hkv;
  const int nhg = G <= 16 ? 1 : G / 16;
  const int grid = a.B * a.Hkv * nhg;
  if (a.D == 128)
    hipLaunchKernelGGL(ring_decode_kernel<128>, dim3(grid), dim3(RD_THREADS), 0, s, a);
  else
    hipLaunchKernelGGL(ring_decode_kernel<64>, dim3(grid), dim3(RD_THREADS), 0, s, a);
  return hipGetLastError();
}

}  // namespace hsk
