// Causal sliding-window / full GQA prefill for gfx950.
//
// bf16 path: one workgroup = 4 waves = 128 query rows of one head; the key axis
// is walked in 64-key tiles that LDS DMA (buffer_load ... lds) stages into a
// double buffer one tile ahead.  Each wave owns 32
// query rows and computes S^T = K * Q^T with v_mfma_f32_32x32x16_bf16, so every
// lane holds 32 of its row's 64 scores and the other 32 sit in lane ^ 32: the
// online softmax needs one permlane32 swap per tile.  P stays in registers and
// feeds O^T += V^T * P^T directly; V^T comes out of LDS with ds_read_b64_tr_b16.
// Tiles wholly outside a wave's window are skipped; only edge tiles are masked.
//
// fp32 path: one wave per (row, head), online softmax over 64-key blocks in fp32,
// for small cases.
#include "common.hpp"
#include "flash_tile.hpp"
#include "kernels.hpp"

namespace hsk {

namespace {

constexpr int PF_BM = 128;
constexpr int PF_THREADS = 256;

// CHUNK: the rows are positions pos0 .. pos0+L-1 of a longer sequence; key
// tiles before pos0 are fetched from the ring (slot tile (position mod W) / 64),
// later ones from the chunk's own K/V.  pos0 and W are multiples of 64, so no
// tile straddles the two sources.
// smem0 / smem1 are the two tile stages.  They must be distinct __shared__
// objects: carved out of one array, the compiler cannot tell the next tile's DMA
// from the current tile's reads and waits for that DMA before every V read.
template <int D, bool CHUNK>
__device__ __forceinline__ void prefill_body(const PrefillArgs& a, char* smem0, char* smem1) {
  using C = FtCfg<D>;

  // XCD-aware order: consecutive logical units share (b, kv head, query block)
  // and land on the same XCD (workgroups are dealt round-robin over 8 XCDs).
  const int per = gridDim.x >> 3;
  const int n = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
  if (n >= a.total) return;
  const int G = a.Hq / a.Hkv;
  const int hh = n % G;
  const int t1 = n / G;
  const int qi = t1 % a.nqb;
  const int t2 = t1 / a.nqb;
  const int g = t2 % a.Hkv;
  const int b = t2 / a.Hkv;
  const int qblk = a.nqb - 1 - qi;  // longest rows first
  const int h = g * G + hh;
  const int L = a.L;
  const int W = a.window;           // >= 1; full causal is passed as a window > L
  const int q0 = qblk * PF_BM;
  const int lane = __lane_id();
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform (scalar)
  const int base = CHUNK ? a.pos0 : 0;  // position of row 0
  const int r0 = base + q0 + 32 * w;    // position of this wave's first row
  const int row = r0 + (lane & 31);     // this lane's query position
  const int rrow = row - base;          // ... as a row of q / out

  const int k_lo = max(0, base + q0 - W + 1);
  const int k_hi = base + min(L, q0 + PF_BM) - 1;
  const int kt0 = k_lo / FT_BN;
  const int ntiles = k_hi / FT_BN - kt0 + 1;

  FlashWave<D> fw;
  fw.init(rrow < L ? a.q + ((size_t)(b * (size_t)L + rrow) * a.Hq + h) * D : nullptr);

  const uint16_t* kbase = a.k + ((size_t)b * L * a.Hkv + g) * D;
  const uint16_t* vbase = a.v + ((size_t)b * L * a.Hkv + g) * D;
  TileDma<D, PF_THREADS> dma;
  dma.init(kbase, vbase, (unsigned)(a.Hkv * D * 2), L, w);
  TileDma<D, PF_THREADS> dring;  // chunk mode: the ring of (b, g), rows of D values
  if (CHUNK) {
    const size_t roff = ((size_t)b * a.Hkv + g) * W * D;
    dring.init(a.ring_k + roff, a.ring_v + roff, (unsigned)(D * 2), W, w);
  }
  auto issue = [&](int kt, char* buf) {
    if (CHUNK) {
      const bool ring = kt * FT_BN < base;
      TileDma<D, PF_THREADS>::pick(ring, dring, dma).issue(ring ? (kt * FT_BN % W) / FT_BN : kt - base / FT_BN, buf);
    } else {
      dma.issue(kt, buf);
    }
  };
  issue(kt0, smem0);

  // unrolled by two so each buffer's LDS offsets are compile-time constants
  auto step = [&](int it, char* cur, char* nxt) {
    wait_vmem();      // this wave's part of tile it has landed
    __syncthreads();  // ... everyone's has, and tile it-1's buffer is free
    const int kt = kt0 + it;
    if (it + 1 < ntiles) issue(kt + 1, nxt);
    fw.tile(cur, cur + C::TILE, kt * FT_BN, r0, row, W, false, a.scale_log2);
  };
  int it = 0;
  for (; it + 1 < ntiles; it += 2) {
    step(it, smem0, smem1);
    step(it + 1, smem1, smem0);
  }
  if (it < ntiles) step(it, smem0, smem1);
  fw.store(rrow < L ? a.o + ((size_t)(b * (size_t)L + rrow) * a.Hq + h) * D : nullptr);
}

template <int D>
__global__ __launch_bounds__(PF_THREADS, 2) void prefill_bf16_kernel(PrefillArgs a) {
  __shared__ __attribute__((aligned(16))) char smem0[2 * FtCfg<D>::TILE];
  __shared__ __attribute__((aligned(16))) char smem1[2 * FtCfg<D>::TILE];
  prefill_body<D, false>(a, smem0, smem1);
}

template <int D>
__global__ __launch_bounds__(PF_THREADS, 2) void prefill_chunk_kernel(PrefillArgs a) {
  __shared__ __attribute__((aligned(16))) char smem0[2 * FtCfg<D>::TILE];
  __shared__ __attribute__((aligned(16))) char smem1[2 * FtCfg<D>::TILE];
  prefill_body<D, true>(a, smem0, smem1);
}

// fp32: one wave per (b, row, head), exact fp32 arithmetic with expf.  The
// visible keys are taken 64 at a time: lane j scores key j0 + j (a sequential
// fp32 dot product over d), the wave forms the block's maximum and sum and
// rescales the running state, then each lane accumulates P V for its own
// output dimensions d = lane + 64 i with the block's probabilities read from LDS.
template <int D>
__global__ __launch_bounds__(64) void prefill_f32_kernel(PrefillArgs a) {
  constexpr int ND = D / 64;  // output dimensions per lane
  __shared__ float sq[D];
  __shared__ float sp[64];
  const long idx = blockIdx.x;  // (b * L + row) * Hq + h
  const int h = (int)(idx % a.Hq);
  const long t = idx / a.Hq;
  const int row = (int)(t % a.L);
  const int b = (int)(t / a.L);
  const int g = h / (a.Hq / a.Hkv);
  const int lane = threadIdx.x;
  const float* qf = (const float*)a.q + ((size_t)(b * (size_t)a.L + row) * a.Hq + h) * D;
  const float* kf = (const float*)a.k + ((size_t)b * a.L * a.Hkv + g) * D;
  const float* vf = (const float*)a.v + ((size_t)b * a.L * a.Hkv + g) * D;
  const size_t rs = (size_t)a.Hkv * D;
#pragma unroll
  for (int i = 0; i < ND; ++i) sq[lane + 64 * i] = qf[lane + 64 * i];
  __syncthreads();
  const int lo = max(0, row - a.window + 1);
  float m = kNegInf, l = 0.f, acc[ND];
#pragma unroll
  for (int i = 0; i < ND; ++i) acc[i] = 0.f;
  for (int j0 = lo; j0 <= row; j0 += 64) {
    const int j = j0 + lane;
    float s = kNegInf;
    if (j <= row) {
      const float4* kr = (const float4*)(kf + (size_t)j * rs);
      float dot = 0.f;
#pragma unroll
      for (int d4 = 0; d4 < D / 4; ++d4) {
        const float4 kv = kr[d4];
        dot = fmaf(sq[4 * d4], kv.x, dot);
        dot = fmaf(sq[4 * d4 + 1], kv.y, dot);
        dot = fmaf(sq[4 * d4 + 2], kv.z, dot);
        dot = fmaf(sq[4 * d4 + 3], kv.w, dot);
      }
      s = dot * a.scale;
    }
    const float m_new = fmaxf(m, wave_max(s));
    const float alpha = (m == kNegInf) ? 0.f : expf(m - m_new);
    const float p = (j <= row) ? expf(s - m_new) : 0.f;
    l = fmaf(l, alpha, wave_sum(p));
    sp[lane] = p;
    __syncthreads();
    const int n = min(64, row - j0 + 1);
#pragma unroll
    for (int i = 0; i < ND; ++i) acc[i] *= alpha;
    for (int jj = 0; jj < n; ++jj) {
      const float pj = sp[jj];
      const float* vr = vf + (size_t)(j0 + jj) * rs + lane;
#pragma unroll
      for (int i = 0; i < ND; ++i) acc[i] = fmaf(pj, vr[64 * i], acc[i]);
    }
    m = m_new;
    __syncthreads();  // sp is rewritten by the next block
  }
  float* orow = (float*)a.o + ((size_t)(b * (size_t)a.L + row) * a.Hq + h) * D;
#pragma unroll
  for (int i = 0; i < ND; ++i) orow[lane + 64 * i] = acc[i] / l;
}

// ring copy: positions max(0, L-W) .. L-1 -> slot p mod W of [B, Hkv, W, D]
__global__ void prefill_ring_kernel(RingCopyArgs a) {
  const long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;   // one 16-byte chunk
  const int cpr = a.row_bytes / 16;
  const int n = min(a.L, a.W);
  const long total = (long)a.B * a.Hkv * n * cpr;
  if (idx >= total) return;
  const int c = (int)(idx % cpr);
  long t = idx / cpr;
  const int i = (int)(t % n);
  t /= n;
  const int g = (int)(t % a.Hkv);
  const int b = (int)(t / a.Hkv);
  const int p = a.L - n + i;
  const int slot = (a.pos0 + p) % a.W;
  const size_t src = (((size_t)b * a.L + p) * a.Hkv + g) * a.row_bytes + (size_t)c * 16;
  const size_t dst = (((size_t)b * a.Hkv + g) * a.W + slot) * a.row_bytes + (size_t)c * 16;
  *(uint4*)((char*)a.ring_k + dst) = *(const uint4*)((const char*)a.k + src);
  *(uint4*)((char*)a.ring_v + dst) = *(const uint4*)((const char*)a.v + src);
}

}  // namespace

hipError_t launch_prefill_bf16(const PrefillArgs& in, hipStream_t stream) {
  PrefillArgs a = in;
  a.nqb = (a.L + PF_BM - 1) / PF_BM;
  a.total = a.B * a.Hq * a.nqb;
  const int grid = (a.total + 7) / 8 * 8;
  const bool chunk = a.ring_k != nullptr;
  if (a.D == 128) {
    if (chunk) hipLaunchKernelGGL(prefill_chunk_kernel<128>, dim3(grid), dim3(PF_THREADS), 0, stream, a);
    else hipLaunchKernelGGL(prefill_bf16_kernel<128>, dim3(grid), dim3(PF_THREADS), 0, stream, a);
  } else {
    if (chunk) hipLaunchKernelGGL(prefill_chunk_kernel<64>, dim3(grid), dim3(PF_THREADS), 0, stream, a);
    else hipLaunchKernelGGL(prefill_bf16_kernel<64>, dim3(grid), dim3(PF_THREADS), 0, stream, a);
  }
  return hipGetLastError();
}

hipError_t launch_prefill_f32(const PrefillArgs& a, hipStream_t stream) {
  const long total = (long)a.B * a.L * a.Hq;  // one wave each; < 2^31 (checked at the boundary)
  if (a.D == 128)
    hipLaunchKernelGGL(prefill_f32_kernel<128>, dim3((unsigned)total), dim3(64), 0, stream, a);
  else
    hipLaunchKernelGGL(prefill_f32_kernel<64>, dim3((unsigned)total), dim3(64), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_prefill_ring(const RingCopyArgs& a, hipStream_t stream) {
  const long total = (long)a.B * a.Hkv * (long)(a.L < a.W ? a.L : a.W) * (a.row_bytes / 16);
  if (total == 0) return hipSuccess;
  const int grid = (int)((total + 255) / 256);
  hipLaunchKernelGGL(prefill_ring_kernel, dim3(grid), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace hsk
