// Top-k block-sparse causal attention: block sums, fp64 block scores and top-k
// selection, then attention over the union of the selected key blocks and the
// local window.
//
//  1. bs_sums:   per 64-token block, fp64 sums of Q (all query heads) and of K.
//                bf16 values have 8-bit significands, so these sums are exact in
//                fp64 for the value ranges met here and do not depend on order.
//                Q sums are stored [Hq][nb][D], K sums d-major [Hkv][D][nb] so the
//                candidate-parallel dot products read 64 consecutive blocks.
//  2. bs_select: one workgroup per (KV head, query block, up to 4 query heads).
//                Each lane scores one key block at a time with a sequential fp64
//                FMA chain over d; the scores sit in LDS.  One wave per query head
//                then finds the top-k threshold by a 64-step bitwise search over
//                order-preserving 64-bit keys, takes ties in ascending block order
//                and writes the chosen blocks ascending (-1 padded).
//  3. bs_attend: one workgroup (2 waves, 64 query rows = one query block) per
//                (query head, query block); key tiles are the selected blocks
//                before the window followed by the window's blocks; selected
//                tiles need no mask, window tiles use the sliding-window mask.
//                A single LDS tile buffer (next tile staged in registers) keeps
//                four workgroups resident per CU.
#include "common.hpp"
#include "flash_tile.hpp"
#include "kernels.hpp"

namespace hsk {

namespace {

constexpr int BS_BLOCK = 64;
constexpr int SUM_THREADS = 256;
constexpr int SEL_THREADS = 256;
constexpr int SEL_MAXNB = 4096;     // key blocks supported (L <= 262144 at block 64)
constexpr int AT_THREADS = 128;

// grid: nb (Q sums) + nb (K sums)
__global__ __launch_bounds__(SUM_THREADS) void bs_sums_kernel(BlockSparseArgs a) {
  const bool isq = (int)blockIdx.x < a.nb;
  const int blk = isq ? blockIdx.x : blockIdx.x - a.nb;
  const int H = isq ? a.Hq : a.Hkv;
  const uint16_t* src = (isq ? a.q : a.k) + (size_t)blk * BS_BLOCK * H * a.D;
  const int nvec = H * a.D / 8;
  const size_t rstride = (size_t)H * a.D;
  for (int vi = threadIdx.x; vi < nvec; vi += SUM_THREADS) {
    double acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = 0.0;
    for (int r = 0; r < BS_BLOCK; ++r) {
      const uint4 u = *(const uint4*)(src + r * rstride + (size_t)vi * 8);
      acc[0] += (double)bf16lo(u.x); acc[1] += (double)bf16hi(u.x);
      acc[2] += (double)bf16lo(u.y); acc[3] += (double)bf16hi(u.y);
      acc[4] += (double)bf16lo(u.z); acc[5] += (double)bf16hi(u.z);
      acc[6] += (double)bf16lo(u.w); acc[7] += (double)bf16hi(u.w);
    }
    const int e = vi * 8;
    const int h = e / a.D, d = e % a.D;
    if (isq) {
      double* dst = a.qsum + ((size_t)h * a.nb + blk) * a.D + d;
#pragma unroll
      for (int j = 0; j < 8; ++j) dst[j] = acc[j];
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) a.ksum[((size_t)h * a.D + d + j) * a.nb + blk] = acc[j];
    }
  }
}

__device__ __forceinline__ unsigned long long order_key(double x) {
  const unsigned long long u = (unsigned long long)__double_as_longlong(x + 0.0);  // -0 -> +0
  return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}

// grid: Hkv * nb * (G / hpw); MAXG * 64 >= nb (key groups held per lane)
template <int HPW, int MAXG>
__global__ __launch_bounds__(SEL_THREADS) void bs_select_kernel(BlockSparseArgs a) {
  __shared__ double qs[256][HPW];               // query block means, [d][head]
  extern __shared__ double sc_dyn[];            // scores, [head][nb]
  const int G = a.Hq / a.Hkv;
  const int ngrp = G / HPW;
  const int grp = blockIdx.x % ngrp;
  const int qb = (blockIdx.x / ngrp) % a.nb;
  const int g = blockIdx.x / (ngrp * a.nb);
  const int h0 = g * G + grp * HPW;
  const int D = a.D;
  const int lane = __lane_id(), w = threadIdx.x >> 6;
  const double inv = 1.0 / BS_BLOCK;

  for (int e = threadIdx.x; e < HPW * D; e += SEL_THREADS) {
    const int hh = e / D, d = e % D;
    qs[d][hh] = a.qsum[((size_t)(h0 + hh) * a.nb + qb) * D + d] * inv;
  }
  __syncthreads();
  const int n = qb;  // candidates: blocks 0 .. qb-1
  const double* kcol = a.ksum + (size_t)g * D * a.nb;
  for (int base = 64 * w; base < n; base += SEL_THREADS) {
    const int kb = base + lane;
    double acc[HPW];
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) acc[hh] = 0.0;
    if (kb < n) {
      for (int d = 0; d < D; ++d) {
        const double kv = kcol[(size_t)d * a.nb + kb] * inv;
#pragma unroll
        for (int hh = 0; hh < HPW; ++hh) acc[hh] = fma(qs[d][hh], kv, acc[hh]);
      }
#pragma unroll
      for (int hh = 0; hh < HPW; ++hh) sc_dyn[(size_t)hh * a.nb + kb] = acc[hh];
    }
  }
  __syncthreads();
  if (w >= HPW) return;
  const int h = h0 + w;
  int32_t* out = a.sel + ((size_t)h * a.nb + qb) * a.topk;
  const int topk = a.topk;
  if (n <= topk) {
    for (int i = lane; i < topk; i += 64) out[i] = (i < n) ? i : -1;
    return;
  }
  // top-k threshold: the largest T with #{key >= T} >= topk, found bit by bit.
  // Each lane keeps its keys (blocks lane, lane+64, ...) in registers; a wave
  // ballot + popcount counts them, so no step needs a cross-lane reduction.
  const int ngr = (n + 63) >> 6;
  unsigned long long keys[MAXG];
#pragma unroll
  for (int i = 0; i < MAXG; ++i) {
    const int kb = i * 64 + lane;
    keys[i] = (i < ngr && kb < n) ? order_key(sc_dyn[(size_t)w * a.nb + kb]) : 0ull;
  }
  // absent slots hold key 0, which sorts below every real key
  unsigned long long T = 0;
  for (int bit = 63; bit >= 0; --bit) {
    const unsigned long long cand = T | (1ull << bit);
    int cnt = 0;
#pragma unroll
    for (int i = 0; i < MAXG; ++i)
      if (i < ngr) cnt += __popcll(__ballot(keys[i] >= cand));
    if (cnt >= topk) T = cand;
  }
  int gt = 0;
#pragma unroll
  for (int i = 0; i < MAXG; ++i)
    if (i < ngr) gt += __popcll(__ballot(keys[i] > T));
  const int need = topk - gt;
  const unsigned long long lt_mask = (1ull << lane) - 1ull;
  int eq_before = 0, written = 0;
#pragma unroll
  for (int i = 0; i < MAXG; ++i) {
    if (i >= ngr) continue;
    const int kb = i * 64 + lane;
    const bool valid = kb < n;
    const bool is_gt = valid && keys[i] > T;
    const bool is_eq = valid && keys[i] == T;
    const unsigned long long eqb = __ballot(is_eq);
    const int rank = eq_before + __popcll(eqb & lt_mask);
    const bool take = is_gt || (is_eq && rank < need);
    const unsigned long long tb = __ballot(take);
    if (take) out[written + __popcll(tb & lt_mask)] = kb;
    written += __popcll(tb);
    eq_before += __popcll(eqb);
  }
  for (int i = written + lane; i < topk; i += 64) out[i] = -1;
}

// grid: Hq * nb
template <int D>
__global__ __launch_bounds__(AT_THREADS) void bs_attend_kernel(BlockSparseArgs a) {
  using C = FtCfg<D>;
  __shared__ __attribute__((aligned(16))) char smem[2 * 2 * C::TILE];
  __shared__ int list[256];                  // selected blocks before the window
  __shared__ unsigned selbits[SEL_MAXNB / 32];
  __shared__ int s_npre;

  // KV-head-major order across the whole chip: the workgroups in flight share
  // one KV head, whose K/V (67 MB at 131072 x 128) stays in the 256 MB MALL;
  // the selected blocks are scattered, so reuse comes from the MALL, not L2.
  const int total = a.Hq * a.nb;
  const int nlin = blockIdx.x;
  if (nlin >= total) return;
  const int G = a.Hq / a.Hkv;
  const int hh = nlin % G;
  const int t1 = nlin / G;
  const int qb = a.nb - 1 - (t1 % a.nb);
  const int g = t1 / a.nb;
  const int h = g * G + hh;
  const int W = a.window;
  const int L = a.L;
  const int q0 = qb * BS_BLOCK;
  const int kfirst = max(0, q0 - W + 1);
  const int kw0 = kfirst / BS_BLOCK;

  for (int i = threadIdx.x; i < (a.nb + 31) / 32; i += AT_THREADS) selbits[i] = 0u;
  if (threadIdx.x == 0) s_npre = 0;
  __syncthreads();
  const int32_t* srow = a.sel + ((size_t)h * a.nb + qb) * a.topk;
  for (int i = threadIdx.x; i < a.topk; i += AT_THREADS) {
    const int s = srow[i];
    if (s >= 0 && s < a.nb) {
      atomicOr(&selbits[s >> 5], 1u << (s & 31));
      if (s < kw0) {
        list[i] = s;  // selected blocks are ascending, so those before the window are a prefix
        atomicAdd(&s_npre, 1);
      }
    }
  }
  __syncthreads();
  const int npre = s_npre;
  const int ntiles = npre + (qb - kw0 + 1);  // then the window's blocks kw0 .. qb

  const int lane = __lane_id();
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform (scalar)
  const int r0 = q0 + 32 * w;
  const int row = r0 + (lane & 31);
  FlashWave<D> fw;
  fw.init(a.q + ((size_t)row * a.Hq + h) * D);

  TileDma<D, AT_THREADS> dma;
  dma.init(a.k + (size_t)g * D, a.v + (size_t)g * D, (unsigned)(a.Hkv * D * 2), L, w);
  auto tile_of = [&](int it) { return it < npre ? list[it] : kw0 + (it - npre); };
  dma.issue(tile_of(0), smem);
  for (int it = 0; it < ntiles; ++it) {
    wait_vmem();
    __syncthreads();
    const int kt = tile_of(it);
    if (it + 1 < ntiles) dma.issue(tile_of(it + 1), smem + ((it + 1) & 1) * 2 * C::TILE);
    const char* ks = smem + (it & 1) * 2 * C::TILE;
    const bool full = (selbits[kt >> 5] >> (kt & 31)) & 1u;
    fw.tile(ks, ks + C::TILE, kt * FT_BN, r0, row, W, full, a.scale_log2);
  }
  fw.store(a.out + ((size_t)row * a.Hq + h) * D);
}

}  // namespace

hipError_t launch_blocksparse(const BlockSparseArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(bs_sums_kernel, dim3(2 * a.nb), dim3(SUM_THREADS), 0, s, a);
  const int G = a.Hq / a.Hkv;
  const int hpw = (G % 4 == 0) ? 4 : (G % 2 == 0) ? 2 : 1;
  const int sgrid = a.topk > 0 ? a.Hkv * a.nb * (G / hpw) : 0;
  const size_t dyn = (size_t)hpw * a.nb * sizeof(double);
  const bool big = a.nb > 2048;
  if (sgrid == 0) {
    // no long-range blocks: the attention below is the sliding window alone
  } else if (hpw == 4) {
    if (big) hipLaunchKernelGGL((bs_select_kernel<4, 64>), dim3(sgrid), dim3(SEL_THREADS), dyn, s, a);
    else hipLaunchKernelGGL((bs_select_kernel<4, 32>), dim3(sgrid), dim3(SEL_THREADS), dyn, s, a);
  } else if (hpw == 2) {
    if (big) hipLaunchKernelGGL((bs_select_kernel<2, 64>), dim3(sgrid), dim3(SEL_THREADS), dyn, s, a);
    else hipLaunchKernelGGL((bs_select_kernel<2, 32>), dim3(sgrid), dim3(SEL_THREADS), dyn, s, a);
  } else {
    if (big) hipLaunchKernelGGL((bs_select_kernel<1, 64>), dim3(sgrid), dim3(SEL_THREADS), dyn, s, a);
    else hipLaunchKernelGGL((bs_select_kernel<1, 32>), dim3(sgrid), dim3(SEL_THREADS), dyn, s, a);
  }
  const int total = a.Hq * a.nb;
  const int grid = (total + 7) / 8 * 8;
  if (a.D == 128)
    hipLaunchKernelGGL(bs_attend_kernel<128>, dim3(grid), dim3(AT_THREADS), 0, s, a);
  else
    hipLaunchKernelGGL(bs_attend_kernel<64>, dim3(grid), dim3(AT_THREADS), 0, s, a);
  return hipGetLastError();
}

}  // namespace hsk
