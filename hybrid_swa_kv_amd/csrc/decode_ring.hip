// One-token decode against a sliding-window ring buffer (bandwidth bound).
//
// One workgroup per (sequence, KV head, group of up to 8 query heads).  The ring
// rows are streamed with 16-byte loads, D/8 lanes per row; K and V of a chunk of
// 128 slots are in flight together.  The new token's K/V is written to slot
// pos mod W and used from registers (the stale slot is never read).  Slots whose
// position would be negative (ring not yet full) are excluded from the softmax.
#include "common.hpp"
#include "kernels.hpp"

namespace hsk {

namespace {

constexpr int RD_THREADS = 256;
constexpr int RD_CH = 128;  // ring slots per chunk

template <int D, int HG>
__global__ __launch_bounds__(RD_THREADS) void ring_decode_kernel(RingDecodeArgs a) {
  constexpr int LPR = D / 8;               // lanes per ring row (one uint4 each)
  constexpr int RPP = RD_THREADS / LPR;    // rows per pass
  constexpr int PASSES = RD_CH / RPP;
  constexpr int RG = 64 / LPR;             // row groups per wave
  __shared__ float sc[HG][RD_CH];
  __shared__ float s_m[HG], s_l[HG], s_alpha[HG];
  __shared__ float red[RD_THREADS / 64][HG][D];

  const int G = a.Hq / a.Hkv;
  const int nhg = G / HG;
  const int hg = blockIdx.x % nhg;
  const int g = (blockIdx.x / nhg) % a.Hkv;
  const int b = blockIdx.x / (nhg * a.Hkv);
  const int t = threadIdx.x;
  const int rr = t / LPR, c = t % LPR;
  const int W = a.W;
  const int p = a.pos[b];
  const int h0 = g * G + hg * HG;
  if (p < 0) {  // precondition violated: leave the ring alone, emit zeros
    for (int e = t; e < HG * D; e += RD_THREADS) a.out[((size_t)b * a.Hq + h0 + e / D) * D + e % D] = 0;
    return;
  }
  const int slot = p % W;

  float qv[HG][8];
#pragma unroll
  for (int h = 0; h < HG; ++h) {
    const uint4 u = *(const uint4*)(a.q + ((size_t)b * a.Hq + h0 + h) * D + 8 * c);
    qv[h][0] = bf16lo(u.x); qv[h][1] = bf16hi(u.x); qv[h][2] = bf16lo(u.y); qv[h][3] = bf16hi(u.y);
    qv[h][4] = bf16lo(u.z); qv[h][5] = bf16hi(u.z); qv[h][6] = bf16lo(u.w); qv[h][7] = bf16hi(u.w);
  }
  const size_t kvoff = (size_t)b * a.Hkv + g;
  const uint4 kn = *(const uint4*)(a.k_new + kvoff * D + 8 * c);
  const uint4 vn = *(const uint4*)(a.v_new + kvoff * D + 8 * c);
  uint16_t* rk = a.ring_k + kvoff * (size_t)W * D;
  uint16_t* rv = a.ring_v + kvoff * (size_t)W * D;
  if (hg == 0 && rr == 0) {
    *(uint4*)(rk + (size_t)slot * D + 8 * c) = kn;
    *(uint4*)(rv + (size_t)slot * D + 8 * c) = vn;
  }
  if (hg == 0 && g == 0 && t == 0 && a.slot_out) a.slot_out[b] = slot;
  if (t < HG) { s_m[t] = kNegInf; s_l[t] = 0.f; }

  float acc[HG][8];
#pragma unroll
  for (int h = 0; h < HG; ++h)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[h][j] = 0.f;

  for (int c0 = 0; c0 < W; c0 += RD_CH) {
    uint4 kr[PASSES], vr[PASSES];
    bool ok[PASSES];
#pragma unroll
    for (int i = 0; i < PASSES; ++i) {
      const int s = c0 + i * RPP + rr;
      // slot s holds position p - ((p - s) mod W); usable when that is >= 0
      const int dist = (slot - s + W) % W;
      ok[i] = (s < W) && (dist <= p);
      if (ok[i] && s == slot) {
        kr[i] = kn;
        vr[i] = vn;
      } else if (ok[i]) {
        kr[i] = *(const uint4*)(rk + (size_t)s * D + 8 * c);
        vr[i] = *(const uint4*)(rv + (size_t)s * D + 8 * c);
      } else {
        kr[i] = make_uint4(0, 0, 0, 0);
        vr[i] = make_uint4(0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int i = 0; i < PASSES; ++i) {
      float kf[8] = {bf16lo(kr[i].x), bf16hi(kr[i].x), bf16lo(kr[i].y), bf16hi(kr[i].y),
                     bf16lo(kr[i].z), bf16hi(kr[i].z), bf16lo(kr[i].w), bf16hi(kr[i].w)};
#pragma unroll
      for (int h = 0; h < HG; ++h) {
        float part = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) part = fmaf(qv[h][j], kf[j], part);
        part = (LPR == 16) ? row16_sum(part) : row8_sum(part);
        if (c == 0) sc[h][i * RPP + rr] = ok[i] ? part * a.scale_log2 : kNegInf;
      }
    }
    __syncthreads();
    {
      const int wv = t >> 6, lane = t & 63;
      for (int h = wv; h < HG; h += RD_THREADS / 64) {
        const float x0 = sc[h][lane], x1 = sc[h][lane + 64];
        const float mx = wave_max(fmaxf(x0, x1));
        const float m_old = s_m[h];
        const float m_new = fmaxf(m_old, mx);
        const float base = (m_new == kNegInf) ? 0.f : m_new;
        const float p0 = fast_exp2(x0 - base), p1 = fast_exp2(x1 - base);
        sc[h][lane] = p0;
        sc[h][lane + 64] = p1;
        const float sum = wave_sum(p0 + p1);
        if (lane == 0) {
          const float alpha = fast_exp2(m_old - base);
          s_alpha[h] = alpha;
          s_l[h] = s_l[h] * alpha + sum;
          s_m[h] = m_new;
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int h = 0; h < HG; ++h) {
      const float al = s_alpha[h];
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[h][j] *= al;
    }
#pragma unroll
    for (int i = 0; i < PASSES; ++i) {
      float vf[8] = {bf16lo(vr[i].x), bf16hi(vr[i].x), bf16lo(vr[i].y), bf16hi(vr[i].y),
                     bf16lo(vr[i].z), bf16hi(vr[i].z), bf16lo(vr[i].w), bf16hi(vr[i].w)};
#pragma unroll
      for (int h = 0; h < HG; ++h) {
        const float pp = sc[h][i * RPP + rr];
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[h][j] = fmaf(pp, vf[j], acc[h][j]);
      }
    }
    __syncthreads();
  }

  // reduce over the row groups of each wave, then over the waves
  const int wv = t >> 6;
#pragma unroll
  for (int h = 0; h < HG; ++h)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float x = acc[h][j];
      if (RG >= 8) x += __shfl_xor(x, 8);
      x += __shfl_xor(x, 16);
      x += xor32(x);
      acc[h][j] = x;
    }
  if ((t & 63) < LPR) {
#pragma unroll
    for (int h = 0; h < HG; ++h)
#pragma unroll
      for (int j = 0; j < 8; ++j) red[wv][h][8 * c + j] = acc[h][j];
  }
  __syncthreads();
  for (int e = t; e < HG * D; e += RD_THREADS) {
    const int h = e / D, d = e % D;
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < RD_THREADS / 64; ++w) s += red[w][h][d];
    a.out[((size_t)b * a.Hq + h0 + h) * D + d] = f32_to_bf16(s / s_l[h]);
  }
}

template <int D>
hipError_t launch_d(const RingDecodeArgs& a, hipStream_t s) {
  const int G = a.Hq / a.Hkv;
  const int HG = (G % 8 == 0) ? 8 : (G % 4 == 0) ? 4 : (G % 2 == 0) ? 2 : 1;
  const int grid = a.B * a.Hkv * (G / HG);
  switch (HG) {
    case 8: hipLaunchKernelGGL((ring_decode_kernel<D, 8>), dim3(grid), dim3(RD_THREADS), 0, s, a); break;
    case 4: hipLaunchKernelGGL((ring_decode_kernel<D, 4>), dim3(grid), dim3(RD_THREADS), 0, s, a); break;
    case 2: hipLaunchKernelGGL((ring_decode_kernel<D, 2>), dim3(grid), dim3(RD_THREADS), 0, s, a); break;
    default: hipLaunchKernelGGL((ring_decode_kernel<D, 1>), dim3(grid), dim3(RD_THREADS), 0, s, a); break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_ring_decode(const RingDecodeArgs& a, hipStream_t s) {
  return a.D == 128 ? launch_d<128>(a, s) : launch_d<64>(a, s);
}

}  // namespace hsk
