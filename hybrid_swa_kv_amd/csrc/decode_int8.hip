// Full-attention decode over an INT8 block-quantised region plus a bf16 hot tail.
//
// Split-K: one workgroup (4 waves) per (sequence, KV head, key range); waves take
// interleaved 32-token chunks (one quantisation block each).  Per chunk a wave
// runs v_mfma_f32_16x16x32_bf16 with the 16 query heads of the group on the N
// axis (unused heads are zero columns):
//   S   = K * q^T      A = K rows (16 keys x 32 d),  B = q^T,  lane l <-> head l%16
//   O^T += V^T * P^T   A = V^T (16 d x 32 keys),     B = P^T (in place: a lane's
//                      8 probabilities are exactly its B operand)
// INT8 codes are converted exactly to bf16 in registers; the K scale is folded
// into the scores and the V scale multiplies each chunk's PV partial once.
// The V^T operand needs 8 keys at one d per lane: each lane reads one dword (4 d)
// from 8 rows and the int8->bf16 packing order performs the transpose.
// Partial (max, sum, acc) records of the 4 waves are merged in LDS and written
// to the workspace; a second kernel merges the splits in a fixed order.
#include "common.hpp"
#include "kernels.hpp"

namespace hsk {

namespace {

constexpr int DQ_THREADS = 256;

__device__ __forceinline__ float i8(unsigned w, int byte) {
  return (float)(int)(signed char)(w >> (8 * byte));
}

// 16 int8 codes -> two bf16x8 operands (codes 0..7, 8..15)
__device__ __forceinline__ void cvt16(uint4 c, bf16x8& lo, bf16x8& hi) {
  u32x4 a, b;
  a[0] = pack_bf16x2(i8(c.x, 0), i8(c.x, 1));
  a[1] = pack_bf16x2(i8(c.x, 2), i8(c.x, 3));
  a[2] = pack_bf16x2(i8(c.y, 0), i8(c.y, 1));
  a[3] = pack_bf16x2(i8(c.y, 2), i8(c.y, 3));
  b[0] = pack_bf16x2(i8(c.z, 0), i8(c.z, 1));
  b[1] = pack_bf16x2(i8(c.z, 2), i8(c.z, 3));
  b[2] = pack_bf16x2(i8(c.w, 0), i8(c.w, 1));
  b[3] = pack_bf16x2(i8(c.w, 2), i8(c.w, 3));
  lo = as_bf16x8(a);
  hi = as_bf16x8(b);
}

template <int D>
struct WaveState {
  static constexpr int NH = D / 64;
  f32x4 o[NH][4];
  float m, l;
};

// One 32-token chunk starting at row c0 of the region; rows >= rend are masked.
// key of P^T slot j (of lane group gq): 16 (j/4) + 4 gq + j%4
template <int D, bool INT8>
__device__ __forceinline__ void chunk(WaveState<D>& st, const bf16x8 (&qb)[D / 64][2],
                                      const void* kbase, const void* vbase, int c0, int rend,
                                      float sk, float sv, int lane) {
  constexpr int NK = D / 64;
  const int hl = lane & 15, gq = lane >> 4;
  f32x4 s[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
#pragma unroll
    for (int r = 0; r < 4; ++r) s[t][r] = 0.f;
    const int row = c0 + 16 * t + hl;
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
      bf16x8 a0, a1;
      if (INT8) {
        const uint4 raw = *(const uint4*)((const int8_t*)kbase + (size_t)row * D + 64 * kk + 16 * gq);
        cvt16(raw, a0, a1);
      } else {
        uint4 r0 = make_uint4(0, 0, 0, 0), r1 = r0;
        if (row < rend) {
          const uint16_t* p = (const uint16_t*)kbase + (size_t)row * D + 64 * kk + 16 * gq;
          r0 = *(const uint4*)p;
          r1 = *(const uint4*)(p + 8);
        }
        a0 = as_bf16x8(r0);
        a1 = as_bf16x8(r1);
      }
      s[t] = mfma16(a0, qb[kk][0], s[t]);
      s[t] = mfma16(a1, qb[kk][1], s[t]);
    }
  }
  // V^T operands, loaded before the softmax so the loads overlap it
  bf16x8 va[NK][4];
#pragma unroll
  for (int hv = 0; hv < NK; ++hv) {
    if (INT8) {
      unsigned rw[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int row = c0 + 16 * (j >> 2) + 4 * gq + (j & 3);
        rw[j] = *(const unsigned*)((const int8_t*)vbase + (size_t)row * D + 64 * hv + 4 * hl);
      }
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        u32x4 t;
#pragma unroll
        for (int q = 0; q < 4; ++q) t[q] = pack_bf16x2(i8(rw[2 * q], jj), i8(rw[2 * q + 1], jj));
        va[hv][jj] = as_bf16x8(t);
      }
    } else {
      uint2 rw[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int row = c0 + 16 * (j >> 2) + 4 * gq + (j & 3);
        rw[j] = make_uint2(0, 0);
        if (row < rend) rw[j] = *(const uint2*)((const uint16_t*)vbase + (size_t)row * D + 64 * hv + 4 * hl);
      }
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        u32x4 t;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const unsigned x0 = (jj < 2) ? rw[2 * q].x : rw[2 * q].y;
          const unsigned x1 = (jj < 2) ? rw[2 * q + 1].x : rw[2 * q + 1].y;
          // low or high bf16 of each dword -> one packed pair
          t[q] = (jj & 1) ? __builtin_amdgcn_perm(x1, x0, 0x07060302u)
                          : __builtin_amdgcn_perm(x1, x0, 0x05040100u);
        }
        va[hv][jj] = as_bf16x8(t);
      }
    }
  }
  float x[8];
  float mx = kNegInf;
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float v = s[t][r] * sk;
      if (!INT8 && c0 + 16 * t + 4 * gq + r >= rend) v = kNegInf;
      x[4 * t + r] = v;
      mx = fmaxf(mx, v);
    }
  mx = fmaxf(mx, __shfl_xor(mx, 16));
  mx = fmaxf(mx, xor32(mx));
  const float m_new = fmaxf(st.m, mx);
  const float base = (m_new == kNegInf) ? 0.f : m_new;
  const float alpha = fast_exp2(st.m - base);
  // P is rounded to bf16 for the MFMA; the normaliser sums the same rounded
  // values, so a row dominated by one key returns that key's value exactly.
  float ps = 0.f;
  u32x4 pw;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float p0 = fast_exp2(x[2 * q] - base), p1 = fast_exp2(x[2 * q + 1] - base);
    pw[q] = pack_bf16x2(p0, p1);
    ps += bf16lo(pw[q]) + bf16hi(pw[q]);
  }
  st.l = st.l * alpha + ps;
  st.m = m_new;
  const bf16x8 pb = as_bf16x8(pw);
  // the chunk's V scale (1 for bf16 rows) multiplies its fresh partial product once
#pragma unroll
  for (int hv = 0; hv < NK; ++hv)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      f32x4 part = {0.f, 0.f, 0.f, 0.f};
      part = mfma16(va[hv][jj], pb, part);
#pragma unroll
      for (int r = 0; r < 4; ++r) st.o[hv][jj][r] = fmaf(st.o[hv][jj][r], alpha, sv * part[r]);
    }
}

template <int D>
__global__ __launch_bounds__(DQ_THREADS) void int8_decode_kernel(Int8DecodeArgs a) {
  constexpr int NK = D / 64;
  __shared__ float sm_m[4][16], sm_l[4][16];
  __shared__ float sm_o[4][16][D];

  const int nsplit = a.ns8 + a.nsh;
  const int split = blockIdx.x % nsplit;
  const int unit = blockIdx.x / nsplit;  // b * Hkv + g
  const int g = unit % a.Hkv, b = unit / a.Hkv;
  const int G = a.Hq / a.Hkv;
  const int lane = __lane_id(), w = threadIdx.x >> 6;
  const int hl = lane & 15, gq = lane >> 4;

  bf16x8 qb[NK][2];
#pragma unroll
  for (int kk = 0; kk < NK; ++kk)
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      uint4 t = make_uint4(0, 0, 0, 0);
      if (hl < G) t = *(const uint4*)(a.q + ((size_t)b * a.Hq + g * G + hl) * D + 64 * kk + 16 * gq + 8 * e);
      qb[kk][e] = as_bf16x8(t);
    }

  WaveState<D> st;
#pragma unroll
  for (int hv = 0; hv < NK; ++hv)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj)
#pragma unroll
      for (int r = 0; r < 4; ++r) st.o[hv][jj][r] = 0.f;
  st.m = kNegInf;
  st.l = 0.f;

  if (split < a.ns8) {
    const int tok0 = split * a.split8;
    const int tok1 = min(a.T8, tok0 + a.split8);
    const int8_t* kc = a.kc + (size_t)unit * a.T8 * D;
    const int8_t* vc = a.vc + (size_t)unit * a.T8 * D;
    const float* ks = a.ks + (size_t)unit * (a.T8 / 32);
    const float* vs = a.vs + (size_t)unit * (a.T8 / 32);
    for (int c0 = tok0 + 32 * w; c0 < tok1; c0 += 128) {
      const float sk = ks[c0 >> 5] * a.scale_log2;
      const float sv = vs[c0 >> 5];
      chunk<D, true>(st, qb, kc, vc, c0, tok1, sk, sv, lane);
    }
  } else {
    const int tok0 = (split - a.ns8) * a.splith;
    const int tok1 = min(a.Th, tok0 + a.splith);
    const uint16_t* kh = a.kh + (size_t)unit * a.Th * D;
    const uint16_t* vh = a.vh + (size_t)unit * a.Th * D;
    for (int c0 = tok0 + 32 * w; c0 < tok1; c0 += 128)
      chunk<D, false>(st, qb, kh, vh, c0, tok1, a.scale_log2, 1.f, lane);
  }

  // merge the four waves of this workgroup
  float lsum = st.l;
  lsum += __shfl_xor(lsum, 16);
  lsum += xor32(lsum);
  if (hl < G) {
#pragma unroll
    for (int hv = 0; hv < NK; ++hv)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
#pragma unroll
        for (int r = 0; r < 4; ++r) sm_o[w][hl][64 * hv + 16 * gq + 4 * r + jj] = st.o[hv][jj][r];
    if (gq == 0) {
      sm_m[w][hl] = st.m;
      sm_l[w][hl] = lsum;
    }
  }
  __syncthreads();
  float* rec0 = a.ws + ((size_t)unit * nsplit + split) * G * (D + 2);
  for (int e = threadIdx.x; e < G * D; e += DQ_THREADS) {
    const int head = e / D, d = e % D;
    float M = kNegInf;
#pragma unroll
    for (int i = 0; i < 4; ++i) M = fmaxf(M, sm_m[i][head]);
    float O = 0.f, Ls = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float f = (sm_m[i][head] == kNegInf) ? 0.f : fast_exp2(sm_m[i][head] - M);
      O += f * sm_o[i][head][d];
      Ls += f * sm_l[i][head];
    }
    float* rec = rec0 + (size_t)head * (D + 2);
    rec[d] = O;
    if (d == 0) {
      rec[D] = M;
      rec[D + 1] = Ls;
    }
  }
}

// merge split records in split order: out = sum 2^(m_i - M) acc_i / sum 2^(m_i - M) l_i
template <int D>
__global__ __launch_bounds__(D) void int8_combine_kernel(Int8DecodeArgs a) {
  const int bh = blockIdx.x;
  const int b = bh / a.Hq, h = bh % a.Hq;
  const int G = a.Hq / a.Hkv;
  const int unit = b * a.Hkv + h / G, head = h % G;
  const int nsplit = a.ns8 + a.nsh;
  const int d = threadIdx.x;
  const float* base = a.ws + (size_t)unit * nsplit * G * (D + 2) + (size_t)head * (D + 2);
  const size_t stride = (size_t)G * (D + 2);
  float M = kNegInf;
  for (int i = 0; i < nsplit; ++i) M = fmaxf(M, base[i * stride + D]);
  float O = 0.f, Ls = 0.f;
  for (int i = 0; i < nsplit; ++i) {
    const float* rec = base + i * stride;
    const float mi = rec[D];
    const float f = (mi == kNegInf) ? 0.f : fast_exp2(mi - M);
    O += f * rec[d];
    Ls += f * rec[D + 1];
  }
  a.out[((size_t)b * a.Hq + h) * D + d] = f32_to_bf16(O / Ls);
}

}  // namespace

void int8_decode_plan(int B, int Hkv, int T8, int Th, int* split8, int* splith, int* ns8, int* nsh) {
  const long units = (long)B * Hkv;
  const long T = (long)T8 + Th;
  long want = (4096 + units - 1) / units;
  if (want < 1) want = 1;
  long split = (T + want - 1) / want;
  split = (split + 127) / 128 * 128;
  if (split < 128) split = 128;
  *split8 = (int)split;
  *splith = (int)split;
  *ns8 = T8 > 0 ? (int)((T8 + split - 1) / split) : 0;
  *nsh = (int)((Th + split - 1) / split);
}

hipError_t launch_int8_decode(const Int8DecodeArgs& a, hipStream_t s) {
  const int grid = a.B * a.Hkv * (a.ns8 + a.nsh);
  if (a.D == 128) {
    hipLaunchKernelGGL(int8_decode_kernel<128>, dim3(grid), dim3(DQ_THREADS), 0, s, a);
    hipLaunchKernelGGL(int8_combine_kernel<128>, dim3(a.B * a.Hq), dim3(128), 0, s, a);
  } else {
    hipLaunchKernelGGL(int8_decode_kernel<64>, dim3(grid), dim3(DQ_THREADS), 0, s, a);
    hipLaunchKernelGGL(int8_combine_kernel<64>, dim3(a.B * a.Hq), dim3(64), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace hsk
