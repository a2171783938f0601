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
//      block sets its head's bit in an LDS word per block, and wave 0 then writes
//      the union of the group's kept blocks in ascending order with those bits.
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

// grid: B * Hkv * ceil(nblk / 64); 4 waves: lane l of wave w scores block
// 64 tile + l for heads w, w+4, ... of the group (fp64, one FMA chain over d)
__global__ __launch_bounds__(256) void int8_sparse_scores_kernel(SparseDecodeArgs a) {
  __shared__ double qd[16 * 128];  // the group's q as fp64, [G][D]
  const int G = a.Hq / a.Hkv;
  const int ntile = (a.nblk + 63) / 64;
  const int unit = blockIdx.x / ntile, tile = blockIdx.x % ntile;
  const int b = unit / a.Hkv, g = unit % a.Hkv;
  const int w = threadIdx.x >> 6, lane = __lane_id();
  for (int i = threadIdx.x; i < G * a.D; i += blockDim.x) {
    const int hh = i / a.D, d = i % a.D;
    qd[i] = (double)bf16_to_f32(a.q[((size_t)b * a.Hq + g * G + hh) * a.D + d]);
  }
  __syncthreads();
  const int j = tile * 64 + lane;
  if (j >= a.nblk) return;
  const float* mcol = a.means + (size_t)unit * a.D * a.nblk + j;
  for (int hh = w; hh < G; hh += 4) {
    const double* qh = qd + hh * a.D;
    double sc = 0.0;
    for (int d = 0; d < a.D; ++d) sc = fma(qh[d], (double)mcol[(size_t)d * a.nblk], sc);
    a.scores[((size_t)b * a.Hq + g * G + hh) * a.nblk + j] = sc;
  }
}

// grid: B * Hkv; 4 waves, wave w serving heads w, w+4, ... of the group (G <= 16);
// dynamic LDS: nblk words of head bits
template <int MAXG>
__global__ __launch_bounds__(256) void int8_sparse_select_kernel(SparseDecodeArgs a) {
  extern __shared__ unsigned hb[];  // [nblk] head bits
  __shared__ unsigned long long gather[4][64];
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
    const int ngr = (nblk + 63) >> 6;
    unsigned long long keys[MAXG];
#pragma unroll
    for (int i = 0; i < MAXG; ++i) {
      const int j = i * 64 + lane;
      keys[i] = (i < ngr && j < nblk) ? order_key(sr[j]) : 0ull;  // absent: below every key
    }
    const int written = topk_select_row<MAXG>(keys, ngr, nblk, topk, gather[w], [&](int slot, int j) {
      out[slot] = j;
      atomicOr(&hb[j], 1u << hh);
    });
    for (int i = written + lane; i < topk; i += 64) out[i] = -1;
  }
  __syncthreads();
  if (w != 0) return;
  // union of the group's kept blocks, ascending, with their head bits
  int32_t* ul = a.ulist + (size_t)unit * a.lmax;
  uint32_t* um = a.umask + (size_t)unit * a.lmax;
  const unsigned long long lt = (1ull << lane) - 1ull;
  int cnt = 0;
  for (int base = 0; base < nblk; base += 64) {
    const int j = base + lane;
    const unsigned m = j < nblk ? hb[j] : 0u;
    const unsigned long long bal = __ballot(m != 0u);
    const int pos = cnt + __popcll(bal & lt);
    if (m != 0u && pos < a.lmax) {
      ul[pos] = j;
      um[pos] = m;
    }
    cnt += __popcll(bal);
  }
  if (lane == 0) a.ucount[unit] = min(cnt, a.lmax);
}

}  // namespace

hipError_t launch_block_means(const BlockMeansArgs& a, hipStream_t s) {
  const long total = (long)a.units * (a.T8 / BLK) * a.D;
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(int8_block_means_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_sparse_select(const SparseDecodeArgs& a, hipStream_t s) {
  const int ntile = (a.nblk + 63) / 64;
  if (a.nblk > a.topk)
    hipLaunchKernelGGL(int8_sparse_scores_kernel, dim3(a.B * a.Hkv * ntile), dim3(256), 0, s, a);
  const size_t dyn = (size_t)a.nblk * sizeof(unsigned);
  if (a.nblk > 2048)
    hipLaunchKernelGGL((int8_sparse_select_kernel<64>), dim3(a.B * a.Hkv), dim3(256), dyn, s, a);
  else
    hipLaunchKernelGGL((int8_sparse_select_kernel<32>), dim3(a.B * a.Hkv), dim3(256), dyn, s, a);
  return hipGetLastError();
}

}  // namespace hsk
