// Block-sparse decode over the hot + INT8 pool: the K block means stored with
// the INT8 blocks, and the per-query-head top-k selection of blocks.
//
//  int8_block_means_kernel: mean of each 32-token block's dequantised K,
//      fl32(fl32(sum of codes) * scale) / 32 -- the code sum is an exact integer,
//      so one rounding; the division by 32 is exact.  Stored d-major.
//  int8_sparse_scores_kernel: q . mean per (query head, block) in fp64, one
//      sequential FMA chain over d, into the workspace.
//  int8_sparse_select_kernel: one workgroup per (sequence, KV head); its four
//      waves take the group's query heads in turn, load a head's scores as order
//      keys into registers and run the shared top-k threshold search; every kept
//      block sets its head's bit in an LDS word per block, and the four waves
//      then write the union of the group's kept blocks in ascending order with
//      those bits, each a quarter of the blocks.
#include "common.hpp"
#include "kernels.hpp"
#include "topk.hpp"

namespace hsk {

namespace {

constexpr int BLK = 32;

// one thread per (unit, block, d)
__global__ __launch_bounds__(256) void int8_block_means_kernel(BlockMeansArgs a) {
  const int nblk = a.T8 / BLK;
  const long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
  const long total = (long)a.units * nblk * a.D;
  if (idx >= total) return;
  const int d = (int)(idx % a.D);
  const long t = idx / a.D;
  const int blk = (int)(t % nblk);
  const int unit = (int)(t / nblk);
  const int8_t* c = a.codes + ((size_t)unit * a.T8 + (size_t)blk * BLK) * a.D + d;
  int sum = 0;
#pragma unroll 8
  for (int r = 0; r < BLK; ++r) sum += c[(size_t)r * a.D];
  const float prod = (float)sum * a.scales[(size_t)unit * nblk + blk];  // one rounding
  a.means[((size_t)unit * a.D + d) * nblk + blk] = prod * (1.0f / BLK);  // exact
}

// grid: B * Hkv * ceil(nblk / 256); lane t of the workgroup scores block
// 256 tile + t for every head of the group.  The block's means are read once,
// 16 d at a time with the next 16 in flight, and NH chains of fp64 FMAs (one per
// head, d ascending; heads past G have zero q rows) consume them.
template <int D, int NH>
__global__ __launch_bounds__(256) void int8_sparse_scores_kernel(SparseDecodeArgs a) {
  constexpr int DC = 16;  // means per chunk
  __shared__ float4 q4[NH * D / 4];  // the group's q as fp32 (exact for bf16), [head][d / 4]
  const int G = a.Hq / a.Hkv;
  const int ntile = (a.nblk + 255) / 256;
  const int unit = blockIdx.x / ntile, tile = blockIdx.x % ntile;
  const int b = unit / a.Hkv, g = unit % a.Hkv;
  float* qf = (float*)q4;
  for (int i = threadIdx.x; i < NH * D; i += blockDim.x) {
    const int hh = i / D, d = i % D;
    qf[i] = hh < G ? bf16_to_f32(a.q[((size_t)b * a.Hq + g * G + hh) * D + d]) : 0.f;
  }
  const int j = tile * 256 + threadIdx.x;
  const float* mcol = a.means + (size_t)unit * D * a.nblk + min(j, a.nblk - 1);  // in range
  const size_t st = a.nblk;
  auto load = [&](int c, float (&m)[DC]) {
#pragma unroll
    for (int k = 0; k < DC; ++k) m[k] = mcol[(size_t)(c * DC + k) * st];
  };
  double sc[NH];
#pragma unroll
  for (int hh = 0; hh < NH; ++hh) sc[hh] = 0.0;
  auto use = [&](int c, const float (&m)[DC]) {
#pragma unroll
    for (int k4 = 0; k4 < DC / 4; ++k4)
#pragma unroll
      for (int hh = 0; hh < NH; ++hh) {
        const float4 qv = q4[hh * (D / 4) + c * (DC / 4) + k4];
        sc[hh] = fma((double)qv.x, (double)m[4 * k4 + 0], sc[hh]);
        sc[hh] = fma((double)qv.y, (double)m[4 * k4 + 1], sc[hh]);
        sc[hh] = fma((double)qv.z, (double)m[4 * k4 + 2], sc[hh]);
        sc[hh] = fma((double)qv.w, (double)m[4 * k4 + 3], sc[hh]);
      }
  };
  float m0[DC], m1[DC];
  load(0, m0);
  __syncthreads();
  for (int c = 0; c < D / DC; c += 2) {
    load(c + 1, m1);  // D / DC is even
    use(c, m0);
    if (c + 2 < D / DC) load(c + 2, m0);
    use(c + 1, m1);
  }
  if (j >= a.nblk) return;
#pragma unroll
  for (int hh = 0; hh < NH; ++hh)
    if (hh < G) a.scores[((size_t)b * a.Hq + g * G + hh) * a.nblk + j] = sc[hh];
}

// grid: B * Hkv; 4 waves, wave w serving heads w, w+4, ... of the group (G <= 16);
// dynamic LDS: nblk words of head bits
template <int MAXG>
__global__ __launch_bounds__(256) void int8_sparse_select_kernel(SparseDecodeArgs a) {
  extern __shared__ unsigned hb[];  // [nblk] head bits
  __shared__ unsigned long long gather[4][64];
  __shared__ int wcount[4];
  constexpr int CF = 16;  // pre-filtered candidate groups (the slowest row sets this kernel's time)
  __shared__ unsigned long long fck[4][64 * CF];
  __shared__ int fci[4][64 * CF];
  const int G = a.Hq / a.Hkv;
  const int unit = blockIdx.x;
  const int b = unit / a.Hkv, g = unit % a.Hkv;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = __lane_id();
  const int nblk = a.nblk;
  for (int i = threadIdx.x; i < nblk; i += blockDim.x) hb[i] = 0u;
  __syncthreads();
  const int topk = a.topk;
  for (int hh = w; hh < G; hh += 4) {
    const size_t row = (size_t)b * a.Hq + g * G + hh;
    int32_t* out = a.sel + row * topk;
    if (nblk <= topk) {  // every block is kept
      for (int i = lane; i < topk; i += 64) out[i] = i < nblk ? i : -1;
      for (int j = lane; j < nblk; j += 64) atomicOr(&hb[j], 1u << hh);
      continue;
    }
    const double* sr = a.scores + row * nblk;
    // every load unconditional from an in-range address, then the selects (a
    // load under a per-lane condition is waited for where it is issued)
    double v[MAXG];
#pragma unroll
    for (int i = 0; i < MAXG; ++i) v[i] = sr[min(i * 64 + lane, nblk - 1)];
    unsigned long long keys[MAXG];
#pragma unroll
    for (int i = 0; i < MAXG; ++i) keys[i] = i * 64 + lane < nblk ? order_key(v[i]) : 0ull;  // absent: 0
    const int written = topk_select_row_filtered<CF, MAXG>(keys, nblk, topk, gather[w], fck[w], fci[w],
                                                       [&](int slot, int j) {
      out[slot] = j;
      atomicOr(&hb[j], 1u << hh);
    });
    for (int i = written + lane; i < topk; i += 64) out[i] = -1;
  }
  __syncthreads();
  // union of the group's kept blocks, ascending, with their head bits: the four
  // waves take consecutive quarters of the 64-block groups, count their kept
  // blocks, and write them after the counts of the waves before
  constexpr int MAXQ = (MAXG + 3) / 4;  // groups per wave (MAXG groups hold nblk)
  const int per = (((nblk + 63) >> 6) + 3) >> 2;
  unsigned mm[MAXQ];
  int mine = 0;
#pragma unroll
  for (int q = 0; q < MAXQ; ++q) {
    const int j = (w * per + q) * 64 + lane;
    mm[q] = (q < per && j < nblk) ? hb[j] : 0u;
    mine += __popcll(__ballot(mm[q] != 0u));
  }
  if (lane == 0) wcount[w] = mine;
  __syncthreads();
  int cnt = 0;
  for (int i = 0; i < w; ++i) cnt += wcount[i];
  int32_t* ul = a.ulist + (size_t)unit * a.lmax;
  uint32_t* um = a.umask + (size_t)unit * a.lmax;
  const unsigned long long lt = (1ull << lane) - 1ull;
#pragma unroll
  for (int q = 0; q < MAXQ; ++q) {
    const unsigned long long bal = __ballot(mm[q] != 0u);
    const int pos = cnt + __popcll(bal & lt);
    if (mm[q] != 0u && pos < a.lmax) {
      ul[pos] = (w * per + q) * 64 + lane;
      um[pos] = mm[q];
    }
    cnt += __popcll(bal);
  }
  if (w == 3 && lane == 0) a.ucount[unit] = min(cnt, a.lmax);  // the last wave ends at the total
}

}  // namespace

hipError_t launch_block_means(const BlockMeansArgs& a, hipStream_t s) {
  const long total = (long)a.units * (a.T8 / BLK) * a.D;
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(int8_block_means_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_sparse_select(const SparseDecodeArgs& a, hipStream_t s) {
  if (a.nblk > a.topk) {
    const dim3 grid(a.B * a.Hkv * ((a.nblk + 255) / 256));
    const int G = a.Hq / a.Hkv;  // <= 16, checked at the boundary
    if (a.D == 128) {
      if (G <= 4) hipLaunchKernelGGL((int8_sparse_scores_kernel<128, 4>), grid, dim3(256), 0, s, a);
      else if (G <= 8) hipLaunchKernelGGL((int8_sparse_scores_kernel<128, 8>), grid, dim3(256), 0, s, a);
      else hipLaunchKernelGGL((int8_sparse_scores_kernel<128, 16>), grid, dim3(256), 0, s, a);
    } else {
      if (G <= 4) hipLaunchKernelGGL((int8_sparse_scores_kernel<64, 4>), grid, dim3(256), 0, s, a);
      else if (G <= 8) hipLaunchKernelGGL((int8_sparse_scores_kernel<64, 8>), grid, dim3(256), 0, s, a);
      else hipLaunchKernelGGL((int8_sparse_scores_kernel<64, 16>), grid, dim3(256), 0, s, a);
    }
  }
  // key groups of 64 candidates per lane: the smallest of 8, 16, 32, 64 that holds nblk (<= 4096)
  const size_t dyn = (size_t)a.nblk * sizeof(unsigned);
  const dim3 grid(a.B * a.Hkv);
  if (a.nblk > 2048)
    hipLaunchKernelGGL((int8_sparse_select_kernel<64>), grid, dim3(256), dyn, s, a);
  else if (a.nblk > 1024)
    hipLaunchKernelGGL((int8_sparse_select_kernel<32>), grid, dim3(256), dyn, s, a);
  else if (a.nblk > 512)
    hipLaunchKernelGGL((int8_sparse_select_kernel<16>), grid, dim3(256), dyn, s, a);
  else
    hipLaunchKernelGGL((int8_sparse_select_kernel<8>), grid, dim3(256), dyn, s, a);
  return hipGetLastError();
}

}  // namespace hsk
