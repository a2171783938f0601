// Top-k block-sparse causal attention: block sums, fp64 block scores and top-k
// selection, then attention over the union of the selected key blocks and the
// local window.
//
//  1. bs_sums:   per 64-token block, fp64 sums of Q (all query heads) and of K.
//                bf16 values have 8-bit significands, so these sums are exact in
//                fp64 for the value ranges met here and do not depend on order.
//                Both are stored block-major, [H][nbp][D]: one thread's 8
//                consecutive d of a block are 64 contiguous bytes.  Q and K are
//                read once, non-temporally (280 -> 242 us at L = 131072).
//  2. bs_scores: per query head, the lower triangle of sumQ * sumK^T (fp64) as a
//                64 x 64-tiled GEMM with 4 x 4 register tiles: each K sum read from
//                LDS serves 64 query blocks.  score = sumQ . sumK / 4096 orders
//                exactly like the mean-vector product (a power-of-two scale), and
//                each entry is one sequential FMA chain over d.  Rows go to the
//                workspace as a packed triangle (row qb holds key blocks 0..qb-1).
//  3. bs_select: one wave per (query head, query block) row.  The top-k threshold
//                is the largest 64-bit order key T with #{key >= T} >= topk,
//                found bit by bit: the top 16 bits over all candidates, then the
//                remaining 48 over the few candidates that share that prefix
//                (gathered into one key per lane; the full search is kept for
//                rows with more than 64 such candidates).  Ties take ascending
//                block order; the chosen blocks are written ascending, -1 padded.
//  4. bs_attend: one workgroup (2 waves, 64 query rows = one query block) per
//                (query head, query block); key tiles are the selected blocks
//                before the window followed by the window's blocks; selected
//                tiles need no mask, window tiles use the sliding-window mask.
#include "common.hpp"
#include "flash_tile.hpp"
#include "kernels.hpp"
#include "topk.hpp"

namespace hsk {

namespace {

constexpr int BS_BLOCK = 64;
constexpr int SUM_THREADS = 256;
constexpr int SEL_MAXNB = 4096;     // key blocks supported (L <= 262144 at block 64)
constexpr int AT_THREADS = 128;
constexpr int BS_FILTER = 8;      // pre-filtered candidate groups of the block selection

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
      const uint4 u = __builtin_bit_cast(uint4, __builtin_nontemporal_load((const u32x4*)(src + r * rstride + (size_t)vi * 8)));
      acc[0] += (double)bf16lo(u.x); acc[1] += (double)bf16hi(u.x);
      acc[2] += (double)bf16lo(u.y); acc[3] += (double)bf16hi(u.y);
      acc[4] += (double)bf16lo(u.z); acc[5] += (double)bf16hi(u.z);
      acc[6] += (double)bf16lo(u.w); acc[7] += (double)bf16hi(u.w);
    }
    const int e = vi * 8;
    const int h = e / a.D, d = e % a.D;
    double* dst = (isq ? a.qsum : a.ksum) + ((size_t)h * a.nbp + blk) * a.D + d;  // block-major
#pragma unroll
    for (int j = 0; j < 8; j += 2) *(double2*)(dst + j) = make_double2(acc[j], acc[j + 1]);
  }
}


// row qb of head h in the packed score triangle (key blocks 0 .. qb-1)
__device__ __forceinline__ size_t tri_row(const BlockSparseArgs& a, int h, int qb) {
  return (size_t)h * ((size_t)a.nb * (a.nb - 1) / 2) + (size_t)qb * (qb - 1) / 2;
}

constexpr int SC_TILE = 64;     // query blocks x key blocks per workgroup
constexpr int SC_SLAB = 32;     // d values staged per pass

// grid: Hq * T(T+1)/2 lower-triangle tiles, T = nbp / 64.  Sums are read with
// row stride nbp, so a tile never leaves its arrays; entries past nb are never
// stored.
__global__ __launch_bounds__(256) void bs_scores_kernel(BlockSparseArgs a) {
  // d-major slabs; rows padded by two doubles (rows stay 16-byte aligned) to
  // spread the transposing writes over the banks
  __shared__ __attribute__((aligned(16))) double sq[SC_SLAB][SC_TILE + 2];
  __shared__ __attribute__((aligned(16))) double sk[SC_SLAB][SC_TILE + 2];
  const int T = a.nbp / SC_TILE;
  const int ntri = T * (T + 1) / 2;
  const int h = blockIdx.x / ntri;
  const int r = blockIdx.x % ntri;
  int ti = 0;  // tile row: r = ti (ti + 1) / 2 + tj, tj <= ti
  while ((ti + 1) * (ti + 2) / 2 <= r) ++ti;
  const int tj = r - ti * (ti + 1) / 2;
  const int g = h / (a.Hq / a.Hkv);
  const int t = threadIdx.x, tx = t & 15, ty = t >> 4;
  const double* qsrc = a.qsum + ((size_t)h * a.nbp + ti * SC_TILE) * a.D;  // block-major sums
  const double* ksrc = a.ksum + ((size_t)g * a.nbp + tj * SC_TILE) * a.D;
  double acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.0;
  for (int d0 = 0; d0 < a.D; d0 += SC_SLAB) {
    // stage 64 blocks x 32 d of each operand (a block's 32 d are 256 contiguous
    // bytes): 4 x 16 bytes per thread per operand, transposed into the d-major slabs
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int u = i * 256 + t;  // 16-byte unit: block u / 16, d pair u % 16
      const int c = u >> 4, dd = (u & 15) * 2;
      const double2 qv = *(const double2*)(qsrc + (size_t)c * a.D + d0 + dd);
      const double2 kv = *(const double2*)(ksrc + (size_t)c * a.D + d0 + dd);
      sq[dd][c] = qv.x;
      sq[dd + 1][c] = qv.y;
      sk[dd][c] = kv.x;
      sk[dd + 1][c] = kv.y;
    }
    __syncthreads();
#pragma unroll 8
    for (int dd = 0; dd < SC_SLAB; ++dd) {
      const double2 q01 = *(const double2*)&sq[dd][4 * ty], q23 = *(const double2*)&sq[dd][4 * ty + 2];
      const double2 k01 = *(const double2*)&sk[dd][4 * tx], k23 = *(const double2*)&sk[dd][4 * tx + 2];
      const double qv[4] = {q01.x, q01.y, q23.x, q23.y}, kv[4] = {k01.x, k01.y, k23.x, k23.y};
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fma(qv[i], kv[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int qb = ti * SC_TILE + 4 * ty + i;
    if (qb >= a.nb) continue;
    double* row = a.scores + tri_row(a, h, qb);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int kb = tj * SC_TILE + 4 * tx + j;
      if (kb < qb) row[kb] = acc[i][j];
    }
  }
}

// grid: Hq * nb / 4, four rows (waves) per workgroup; MAXG * 64 >= nb
// one row's selection with MAXG key groups (64 candidates each per lane)
template <int MAXG>
__device__ __forceinline__ void bs_select_row(const double* row, int n, int topk, int32_t* out,
                                              unsigned long long* gather, unsigned long long* fck, int* fci) {
  const int lane = __lane_id();
  // every load unconditional from an in-range address, then the selects: a load
  // under a per-lane condition is waited for where it is issued, one at a time
  double v[MAXG];
#pragma unroll
  for (int i = 0; i < MAXG; ++i) v[i] = row[min(i * 64 + lane, n - 1)];
  unsigned long long keys[MAXG];
#pragma unroll
  for (int i = 0; i < MAXG; ++i) keys[i] = i * 64 + lane < n ? order_key(v[i]) : 0ull;  // 0: below every key
  const int written =
      topk_select_row_filtered<BS_FILTER, MAXG>(keys, n, topk, gather, fck, fci,
                                                [&](int slot, int kb) { out[slot] = kb; });
  for (int i = written + lane; i < topk; i += 64) out[i] = -1;
}

// grid: ceil(Hq * nb / 4); wave w of block x selects row 4x + w, its key groups
// sized to the row (8, 16, 32 or 64 groups of 64 candidates, at most MAXG: the
// largest size sets the kernel's registers)
template <int MAXG>
__global__ __launch_bounds__(256) void bs_select_kernel(BlockSparseArgs a) {
  __shared__ unsigned long long gather[4][64];
  __shared__ unsigned long long fck[4][64 * BS_FILTER];  // pre-filtered candidates
  __shared__ int fci[4][64 * BS_FILTER];
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = __lane_id();
  const int rowid = blockIdx.x * 4 + w;  // h * nb + qb
  if (rowid >= a.Hq * a.nb) return;
  const int h = rowid / a.nb, qb = rowid % a.nb;
  int32_t* out = a.sel + (size_t)rowid * a.topk;
  const int topk = a.topk;
  const int n = qb;  // candidates: blocks 0 .. qb-1
  if (n <= topk) {
    for (int i = lane; i < topk; i += 64) out[i] = (i < n) ? i : -1;
    return;
  }
  const double* row = a.scores + tri_row(a, h, qb);
  if (n <= 512) bs_select_row<8>(row, n, topk, out, gather[w], fck[w], fci[w]);
  else if (n <= 1024) bs_select_row<16>(row, n, topk, out, gather[w], fck[w], fci[w]);
  else if (MAXG <= 32 || n <= 2048)
    bs_select_row<MAXG <= 32 ? MAXG : 32>(row, n, topk, out, gather[w], fck[w], fci[w]);
  else bs_select_row<64>(row, n, topk, out, gather[w], fck[w], fci[w]);
}

// The attend kernel double-buffers its tiles: one tile in flight while the other
// is computed.  Two stages (64 KB of LDS at D = 128) leave room for two
// workgroups per CU; three or four stages keep more tiles in flight but fit one
// workgroup per CU and measured about 1.7x slower; a single stage with four
// workgroups per CU measured 7 % slower.
//
// Stage S, one __shared__ object each: slices of a single array would make the
// compiler wait for every outstanding tile DMA before each LDS read, since it
// could not tell the stages apart.
template <int D, int S>
__device__ __forceinline__ char* bs_stage() {
  __shared__ __attribute__((aligned(16))) char buf[2 * FtCfg<D>::TILE];
  return buf;
}

// grid: Hq * nb
template <int D>
__global__ __launch_bounds__(AT_THREADS) void bs_attend_kernel(BlockSparseArgs a) {
  using C = FtCfg<D>;
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
  // the tile index is uniform; saying so keeps the DMA offset scalar (an LDS value
  // would otherwise count as per-lane and the DMA would loop over lanes)
  auto tile_of = [&](int it) { return __builtin_amdgcn_readfirstlane(it < npre ? list[it] : kw0 + (it - npre)); };
  char* const s0 = bs_stage<D, 0>();
  char* const s1 = bs_stage<D, 1>();
  dma.issue(tile_of(0), s0);  // ntiles >= 1: the window holds the query block itself
  // one tile step: tile it is in cur, tile it+1 goes to nxt
  auto step = [&](int it, char* cur, char* nxt) {
    wait_vmem();    // this wave's part of tile it has landed
    lds_barrier();  // ... everyone's has, and tile it-1's stage is free
    const int kt = tile_of(it);
    if (it + 1 < ntiles) dma.issue(tile_of(it + 1), nxt);
    const bool full = (selbits[kt >> 5] >> (kt & 31)) & 1u;
    fw.tile(cur, cur + C::TILE, kt * FT_BN, r0, row, W, full, a.scale_log2);
  };
  // unrolled by two so that every stage address is a compile-time constant
  int it = 0;
  for (; it + 1 < ntiles; it += 2) {
    step(it, s0, s1);
    step(it + 1, s1, s0);
  }
  if (it < ntiles) step(it, s0, s1);
  fw.store(a.out + ((size_t)row * a.Hq + h) * D);
}

}  // namespace

hipError_t launch_blocksparse(const BlockSparseArgs& a, hipStream_t s) {
  if (a.topk > 0) {
    // block sums, the score triangle and the per-row selection
    hipLaunchKernelGGL(bs_sums_kernel, dim3(2 * a.nb), dim3(SUM_THREADS), 0, s, a);
    const int T = a.nbp / SC_TILE;
    hipLaunchKernelGGL(bs_scores_kernel, dim3(a.Hq * T * (T + 1) / 2), dim3(256), 0, s, a);
    const int sgrid = (a.Hq * a.nb + 3) / 4;
    if (a.nb > 2048)
      hipLaunchKernelGGL((bs_select_kernel<64>), dim3(sgrid), dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((bs_select_kernel<32>), dim3(sgrid), dim3(256), 0, s, a);
  }
  // with topk == 0 the attention below is the sliding window alone
  const int total = a.Hq * a.nb;
  const int grid = (total + 7) / 8 * 8;
  if (a.D == 128)
    hipLaunchKernelGGL(bs_attend_kernel<128>, dim3(grid), dim3(AT_THREADS), 0, s, a);
  else
    hipLaunchKernelGGL(bs_attend_kernel<64>, dim3(grid), dim3(AT_THREADS), 0, s, a);
  return hipGetLastError();
}

}  // namespace hsk
