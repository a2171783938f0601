// Full-attention decode over an INT8 block-quantised region plus a bf16 hot tail.
//
// Split-K: one workgroup (4 waves) per (sequence, KV head, key range); waves take
// interleaved 32-token chunks (one quantisation block each).  The key ranges
// carry equal bytes (an INT8 token's 256 code bytes count once, a bf16 hot
// token's 512 bytes twice); the last range of a sequence runs on from the INT8
// tokens into the hot ones, so the grid is a whole number of rounds of equal
// workgroups.  Per chunk a wave
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
#include "decode_mfma.hpp"
#include "kernels.hpp"

namespace hsk {

namespace {

constexpr int DQ_THREADS = 256;
constexpr int DQ_TARGET_WGS = 2048;  // workgroups of the dense INT8 decode in all

template <int D>
__global__ __launch_bounds__(DQ_THREADS, 3) void int8_decode_kernel(Int8DecodeArgs a) {
  __shared__ float sm_m[4][16], sm_l[4][16];
  __shared__ __attribute__((aligned(16))) float sm_o[4][16][stash_row<D>()];

  const int nsplit = a.nsplit;
  const int unit = blockIdx.x / nsplit;  // b * Hkv + g
  const int split = blockIdx.x % nsplit;
  const int g = unit % a.Hkv, b = unit / a.Hkv;
  // this split's weight range -> INT8 tokens [t0, t1) and hot tokens [h0, h1)
  const int wt = a.T8 + 2 * a.Th;
  const int w0 = split * a.wsplit, w1 = min(wt, w0 + a.wsplit);
  const int t0 = min(w0, a.T8), t1 = min(w1, a.T8);
  const int h0 = max(w0 - a.T8, 0) / 2, h1 = max(w1 - a.T8, 0) / 2;
  const int G = a.Hq / a.Hkv;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  DecodeWave<D> st;
  st.init(a.q + ((size_t)b * a.Hq + g * G) * D, G);

  if (t0 < t1) {
    const int tok0 = t0, tok1 = t1;
    const int8_t* kc = a.kc + (size_t)unit * a.T8 * D;
    const int8_t* vc = a.vc + (size_t)unit * a.T8 * D;
    const int nbytes = a.T8 * D;  // < 2^31: checked at the boundary
    const Int8Rows<D> rows{kc, vc, __builtin_amdgcn_make_buffer_rsrc((void*)kc, (short)0, nbytes, 0x00020000),
                           __builtin_amdgcn_make_buffer_rsrc((void*)vc, (short)0, nbytes, 0x00020000)};
    const float* ks = a.ks + (size_t)unit * (a.T8 / 32);
    const float* vs = a.vs + (size_t)unit * (a.T8 / 32);
    // two chunks in flight per wave: the loads of chunk i+1 are issued before
    // chunk i's math (unrolled by two, so the register images alternate instead
    // of being copied).  Two images keep the kernel within 168 VGPRs, three
    // waves per SIMD; a third image in flight measured slower, since it halves
    // the waves that hide the chunk math's latency.
    using Raw = typename DecodeWave<D>::template Raw<true>;
    auto step = [&](int c, Raw& cur, Raw& ahead) {
      if (c + 128 < tok1) st.template load<true>(rows, c + 128, ahead);
      st.template compute<true>(rows, c, cur, ks[c >> 5] * a.scale_log2, vs[c >> 5]);
    };
    int c0 = tok0 + 32 * w;
    if (c0 < tok1) {
      Raw r0, r1;
      st.template load<true>(rows, c0, r0);
      for (;; c0 += 256) {
        step(c0, r0, r1);
        if (c0 + 128 >= tok1) break;
        step(c0 + 128, r1, r0);
        if (c0 + 256 >= tok1) break;
      }
    }
  }
  if (h0 < h1) {
    const int tok0 = h0, tok1 = h1;
    const Bf16Rows<D> rows{a.kh + (size_t)unit * a.Th * D, a.vh + (size_t)unit * a.Th * D, tok1};
    for (int c0 = tok0 + 32 * w; c0 < tok1; c0 += 128) st.template chunk<false>(rows, c0, a.scale_log2, 1.f);
  }

  // merge the four waves of this workgroup into one split record
  st.stash(sm_m, sm_l, sm_o, w, G);
  __syncthreads();
  float* rec0 = a.ws + ((size_t)unit * nsplit + split) * G * (D + 2);
  for (int e = threadIdx.x; e < G * D; e += DQ_THREADS) {
    const int head = e / D, d = e % D;
    float M, Ls;
    const float O = merge_waves<4, D>(sm_m, sm_l, sm_o, head, d, M, Ls);
    float* rec = rec0 + (size_t)head * (D + 2);
    rec[d] = O;
    if (d == 0) {
      rec[D] = M;
      rec[D + 1] = Ls;
    }
  }
}

// Block-sparse variant: the INT8 splits walk the union of blocks kept by the
// group's heads (written by the selection) instead of a token range; each chunk
// is one kept block, and heads that did not keep it have its scores masked.  A
// wave's list entries are read once into lanes and broadcast per step.  Hot
// splits and split records are as above.
template <int D>
__global__ __launch_bounds__(DQ_THREADS, 3) void int8_sparse_decode_kernel(SparseDecodeArgs a) {
  __shared__ float sm_m[4][16], sm_l[4][16];
  __shared__ __attribute__((aligned(16))) float sm_o[4][16][stash_row<D>()];

  const int nsplit = a.nss + a.nsh;
  const int nhot = a.B * a.Hkv * a.nsh;
  const int i = blockIdx.x;
  const int unit = i < nhot ? i / a.nsh : (i - nhot) / a.nss;
  const int split = i < nhot ? a.nss + i % a.nsh : (i - nhot) % a.nss;
  const int g = unit % a.Hkv, b = unit / a.Hkv;
  const int G = a.Hq / a.Hkv;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = __lane_id();

  DecodeWave<D> st;
  st.init(a.q + ((size_t)b * a.Hq + g * G) * D, G);

  if (split < a.nss) {
    const int cnt = a.ucount[unit];
    const int e0 = split * a.epsplit, e1 = min(cnt, e0 + a.epsplit);
    const int nmine = e1 > e0 + w ? (e1 - e0 - w + 3) / 4 : 0;  // entries e0 + w + 4 k
    int myblk = 0;
    unsigned mymask = 0u;
    if (lane < nmine) {
      myblk = a.ulist[(size_t)unit * a.lmax + e0 + w + 4 * lane];
      mymask = a.umask[(size_t)unit * a.lmax + e0 + w + 4 * lane];
    }
    const int8_t* kc = a.kc + (size_t)unit * a.T8 * D;
    const int8_t* vc = a.vc + (size_t)unit * a.T8 * D;
    const int nbytes = a.T8 * D;
    const Int8Rows<D> rows{kc, vc, __builtin_amdgcn_make_buffer_rsrc((void*)kc, (short)0, nbytes, 0x00020000),
                           __builtin_amdgcn_make_buffer_rsrc((void*)vc, (short)0, nbytes, 0x00020000)};
    const float* ks = a.ks + (size_t)unit * a.nblk;
    const float* vs = a.vs + (size_t)unit * a.nblk;
    using Raw = typename DecodeWave<D>::template Raw<true>;
    auto blk = [&](int k) { return __builtin_amdgcn_readlane(myblk, k); };
    auto step = [&](int k, Raw& cur, Raw& ahead) {
      if (k + 1 < nmine) st.template load<true>(rows, 32 * blk(k + 1), ahead);
      const int j = blk(k);
      st.template compute<true>(rows, 32 * j, cur, ks[j] * a.scale_log2, vs[j],
                                (unsigned)__builtin_amdgcn_readlane((int)mymask, k));
    };
    if (nmine > 0) {  // two blocks in flight at three waves per SIMD, as in the dense decode
      Raw r0, r1;
      st.template load<true>(rows, 32 * blk(0), r0);
      for (int k = 0;; k += 2) {
        step(k, r0, r1);
        if (k + 1 >= nmine) break;
        step(k + 1, r1, r0);
        if (k + 2 >= nmine) break;
      }
    }
  } else {
    const int tok0 = (split - a.nss) * a.hsplit;
    const int tok1 = min(a.Th, tok0 + a.hsplit);
    const Bf16Rows<D> rows{a.kh + (size_t)unit * a.Th * D, a.vh + (size_t)unit * a.Th * D, tok1};
    for (int c0 = tok0 + 32 * w; c0 < tok1; c0 += 128) st.template chunk<false>(rows, c0, a.scale_log2, 1.f);
  }

  st.stash(sm_m, sm_l, sm_o, w, G);
  __syncthreads();
  float* rec0 = a.ws + ((size_t)unit * nsplit + split) * G * (D + 2);
  for (int e = threadIdx.x; e < G * D; e += DQ_THREADS) {
    const int head = e / D, d = e % D;
    float M, Ls;
    const float O = merge_waves<4, D>(sm_m, sm_l, sm_o, head, d, M, Ls);
    float* rec = rec0 + (size_t)head * (D + 2);
    rec[d] = O;
    if (d == 0) {
      rec[D] = M;
      rec[D + 1] = Ls;
    }
  }
}

// merge split records in split order: out = sum 2^(m_i - M) acc_i / sum 2^(m_i - M) l_i
// One workgroup per (sequence, query head); split weights go through LDS so the
// per-d loop issues independent loads.
template <int D>
__global__ __launch_bounds__(D) void int8_combine_kernel(Int8DecodeArgs a) {
  constexpr int CH = 256;  // splits weighed per pass
  __shared__ float sf[CH];
  __shared__ float red[D / 64];
  __shared__ float s_M;
  const int bh = blockIdx.x;
  const int b = bh / a.Hq, h = bh % a.Hq;
  const int G = a.Hq / a.Hkv;
  const int unit = b * a.Hkv + h / G, head = h % G;
  const int nsplit = a.nsplit;
  const int t = threadIdx.x;
  const float* base = a.ws + (size_t)unit * nsplit * G * (D + 2) + (size_t)head * (D + 2);
  const size_t stride = (size_t)G * (D + 2);
  float mx = kNegInf;
  for (int i = t; i < nsplit; i += D) mx = fmaxf(mx, base[i * stride + D]);
  mx = wave_max(mx);
  if ((t & 63) == 0) red[t >> 6] = mx;
  __syncthreads();
  if (t == 0) {
    float M = kNegInf;
    for (int i = 0; i < D / 64; ++i) M = fmaxf(M, red[i]);
    s_M = M;
  }
  __syncthreads();
  const float M = s_M;
  float O = 0.f, Lpart = 0.f;
  for (int c0 = 0; c0 < nsplit; c0 += CH) {
    const int n = min(CH, nsplit - c0);
    for (int i = t; i < n; i += D) {
      const float* rec = base + (size_t)(c0 + i) * stride;
      const float mi = rec[D];
      const float f = (mi == kNegInf) ? 0.f : fast_exp2(mi - M);
      sf[i] = f;
      Lpart += f * rec[D + 1];
    }
    __syncthreads();
#pragma unroll 8
    for (int i = 0; i < n; ++i) O += sf[i] * base[(size_t)(c0 + i) * stride + t];
    __syncthreads();
  }
  Lpart = wave_sum(Lpart);
  if ((t & 63) == 0) red[t >> 6] = Lpart;
  __syncthreads();
  float L = 0.f;
#pragma unroll
  for (int i = 0; i < D / 64; ++i) L += red[i];
  a.out[((size_t)b * a.Hq + h) * D + t] = f32_to_bf16(O / L);
}

}  // namespace

void int8_decode_plan(int B, int Hkv, int T8, int Th, int* nsplit, int* wsplit) {
  // about DQ_TARGET_WGS workgroups in all, each range a multiple of 128 weights
  // (128 INT8 tokens: one chunk per wave; 64 hot tokens)
  const long units = (long)B * Hkv;
  const long wt = (long)T8 + 2l * Th;
  long want = (DQ_TARGET_WGS + units - 1) / units;
  if (want < 1) want = 1;
  long ws = (wt + want - 1) / want;
  ws = (ws + 127) / 128 * 128;
  *wsplit = (int)ws;
  *nsplit = (int)((wt + ws - 1) / ws);
}

hipError_t launch_int8_decode(const Int8DecodeArgs& a, hipStream_t s) {
  const int grid = a.B * a.Hkv * a.nsplit;
  if (a.D == 128) {
    hipLaunchKernelGGL(int8_decode_kernel<128>, dim3(grid), dim3(DQ_THREADS), 0, s, a);
    hipLaunchKernelGGL(int8_combine_kernel<128>, dim3(a.B * a.Hq), dim3(128), 0, s, a);
  } else {
    hipLaunchKernelGGL(int8_decode_kernel<64>, dim3(grid), dim3(DQ_THREADS), 0, s, a);
    hipLaunchKernelGGL(int8_combine_kernel<64>, dim3(a.B * a.Hq), dim3(64), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_sparse_decode(const SparseDecodeArgs& a, hipStream_t s) {
  const int grid = a.B * a.Hkv * (a.nss + a.nsh);
  Int8DecodeArgs c{};  // the combine reads only these fields
  c.out = a.out; c.ws = a.ws;
  c.B = a.B; c.Hq = a.Hq; c.Hkv = a.Hkv; c.D = a.D;
  c.nsplit = a.nss + a.nsh;
  if (a.D == 128) {
    hipLaunchKernelGGL(int8_sparse_decode_kernel<128>, dim3(grid), dim3(DQ_THREADS), 0, s, a);
    hipLaunchKernelGGL(int8_combine_kernel<128>, dim3(a.B * a.Hq), dim3(128), 0, s, c);
  } else {
    hipLaunchKernelGGL(int8_sparse_decode_kernel<64>, dim3(grid), dim3(DQ_THREADS), 0, s, a);
    hipLaunchKernelGGL(int8_combine_kernel<64>, dim3(a.B * a.Hq), dim3(64), 0, s, c);
  }
  return hipGetLastError();
}

}  // namespace hsk
