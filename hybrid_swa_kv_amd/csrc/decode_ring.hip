// One-token decode against a sliding-window ring buffer (bandwidth bound).
//
// One workgroup per (sequence, KV head, group of up to 16 query heads); its 8
// waves take interleaved 16-slot chunks of the ring and run the 16x16x32 MFMA
// decode of decode_mfma.hpp (heads on the MFMA N axis), then merge their
// (max, sum, acc) states through LDS behind a single barrier.  Every load of a
// chunk is issued before anything waits on one (q and the new token's rows are
// fetched once per workgroup into LDS, ahead of the ring loads),
// so one HBM round trip covers a 128-slot window; longer windows keep the next
// chunk in flight while the current one is computed.  Small chunks keep each
// wave's serial work short: the decode of one chunk is the kernel's tail once
// its data has arrived.  The new token's K/V is written to slot pos mod W and
// used from k_new/v_new (whatever is read from that slot is discarded); slots
// whose position would be negative (ring not yet full) are not attended.
#include "common.hpp"
#include "decode_mfma.hpp"
#include "kernels.hpp"

namespace hsk {

namespace {

constexpr int RD_WAVES = 8;
constexpr int RD_THREADS = 64 * RD_WAVES;
constexpr int RD_CHUNK = 16;                     // slots per wave per step
constexpr int RD_STRIDE = RD_CHUNK * RD_WAVES;   // slots per workgroup step
constexpr int RD_NT = RD_CHUNK / 16;             // 16-key MFMA blocks per chunk

// One LDS object, the small per-wave (max, sum) arrays first, so the merge
// addresses them with immediate offsets.
template <int D>
struct RingShared {
  float m[RD_WAVES][16], l[RD_WAVES][16];
  float o[RD_WAVES][16][stash_row<D>()];
  uint16_t in[(16 + 2) * D];
};

// Grid (Hkv * nhg, B): blockIdx.y is the sequence, blockIdx.x the KV head and
// head group; with at most 16 heads per KV head (ONE_HG, nhg = 1) nothing is
// divided before the ring loads are issued (G comes from the host).
template <int D, bool ONE_HG>
__global__ __launch_bounds__(RD_THREADS) void ring_decode_kernel(RingDecodeArgs a) {
  __shared__ __attribute__((aligned(16))) RingShared<D> sh;
  uint16_t* const sm_in = sh.in;

  const int G = a.G;
  const int HG = ONE_HG ? G : 16;  // heads served by this workgroup
  const int nhg = ONE_HG ? 1 : G / 16;
  const int hg = ONE_HG ? 0 : (int)blockIdx.x % nhg;
  const int g = ONE_HG ? (int)blockIdx.x : (int)blockIdx.x / nhg;
  const int b = blockIdx.y;
  const int t = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int W = a.W;
  const int h0 = g * G + hg * HG;
  // No branch on pos before the ring loads: their addresses do not depend on it,
  // only the masks do, so the pos load and the ring loads travel together.  A
  // negative pos (a violated precondition) attends nothing, writes no slot and
  // yields zeros.
  const size_t kvoff = (size_t)b * a.Hkv + g;
  uint16_t* rk = a.ring_k + kvoff * (size_t)W * D;
  uint16_t* rv = a.ring_v + kvoff * (size_t)W * D;
  const uint16_t* kn = a.k_new + kvoff * D;
  const uint16_t* vn = a.v_new + kvoff * D;
  // q of the served heads and the new token's K and V rows are staged once per
  // workgroup in LDS (sm_in: HG*D q values, then D of k_new, then D of v_new):
  // each thread fetches up to RD_PIECES 16-byte pieces, issued before its ring
  // loads so the wait for them does not wait for the ring data.
  const int nq = HG * D / 8, nin = nq + D / 4;
  constexpr int RD_PIECES = ((16 + 2) * D / 8 + RD_THREADS - 1) / RD_THREADS;
  uint4 piece[RD_PIECES];
#pragma unroll
  for (int i = 0; i < RD_PIECES; ++i) {
    const int pi = min(t + i * RD_THREADS, nin - 1);
    const uint16_t* src = pi < nq ? a.q + ((size_t)b * a.Hq + h0) * D + 8 * pi
                          : pi < nq + D / 8 ? kn + 8 * (pi - nq) : vn + 8 * (pi - nq - D / 8);
    piece[i] = *(const uint4*)src;
  }
  __builtin_amdgcn_sched_barrier(0);
  DecodeWave<D, true> st;
  RingRows<D> rows{rk, rv, sm_in + HG * D, sm_in + HG * D + D, W, 0, -1};
  // software pipelined over the wave's chunks: chunk c+1 is in flight while c is computed
  using Raw = typename DecodeWave<D, true>::template Raw<false>;
  Raw cur, nxt;
  const int first = RD_CHUNK * w;
  st.template load<false, RD_NT>(rows, first, cur);
  __builtin_amdgcn_sched_barrier(0);  // keep the pos load and its use behind the chunk loads
  const int p = a.pos[b];
  const bool ok = p >= 0;
  const int slot = (int)((unsigned)max(p, 0) % (unsigned)W);  // branch-free
  rows.slot = slot;
  rows.p = ok ? p : -1;
#pragma unroll
  for (int i = 0; i < RD_PIECES; ++i)
    if (t + i * RD_THREADS < nin) *(uint4*)(sm_in + 8 * (t + i * RD_THREADS)) = piece[i];
  __syncthreads();
  // append: the first head group's workgroup writes the new token into its slot
  // now, so the stores complete while the ring loads are in flight.  This and
  // the output are written non-temporally (no L2 allocation): nothing in the
  // launch reads them again, and the launch measured 1.2 % shorter so.  Any read of
  // that slot (here or in another head group's workgroup) is replaced by the new
  // token's rows from LDS, so it does not matter whether it sees old or new bytes.
  if (ok && hg == 0 && t < D / 8) {
    typedef __attribute__((ext_vector_type(4))) unsigned u4;
    __builtin_nontemporal_store(*(const u4*)(sm_in + HG * D + 8 * t), (u4*)(rk + (size_t)slot * D + 8 * t));
    __builtin_nontemporal_store(*(const u4*)(sm_in + HG * D + D + 8 * t), (u4*)(rv + (size_t)slot * D + 8 * t));
  }
  if (ok && hg == 0 && g == 0 && t == 0 && a.slot_out) a.slot_out[b] = slot;
  st.init(sm_in, HG);
  typename DecodeWave<D, true>::AltRow alt;
  st.load_alt(rows, alt);
  int c0 = first;
  for (; c0 + RD_STRIDE < W; c0 += 2 * RD_STRIDE) {
    st.template load<false, RD_NT>(rows, c0 + RD_STRIDE, nxt);
    st.template compute<false, RD_NT>(rows, c0, cur, a.scale_log2, 1.f, alt, ~0u, c0 == first);
    if (c0 + 2 * RD_STRIDE < W) st.template load<false, RD_NT>(rows, c0 + 2 * RD_STRIDE, cur);
    st.template compute<false, RD_NT>(rows, c0 + RD_STRIDE, nxt, a.scale_log2, 1.f, alt);
  }
  if (c0 < W) st.template compute<false, RD_NT>(rows, c0, cur, a.scale_log2, 1.f, alt, ~0u, c0 == first);

  st.stash(sh.m, sh.l, sh.o, w, HG);
  __syncthreads();
  // One stashed tile (four columns) per thread, so the waves' factors are formed
  // once for four outputs; its outputs are d = base + 4 r.  Thread order runs
  // over jj fastest, so four lanes' stores of one r cover 8 contiguous bytes.
  for (int e = t; e < HG * D / 4; e += RD_THREADS) {
    const int head = e / (D / 4), q = e % (D / 4);
    const int hv = q >> 4, gq = (q >> 2) & 3, jj = q & 3;
    float M, Ls;
    const f32x4 O = merge_waves4<RD_WAVES, D>(sh.m, sh.l, sh.o, head, 64 * hv + 16 * jj + 4 * gq, M, Ls);
    const float rl = __builtin_amdgcn_rcpf(Ls);
    uint16_t* dst = a.out + ((size_t)b * a.Hq + h0 + head) * D + 64 * hv + 16 * gq + jj;
#pragma unroll
    for (int r = 0; r < 4; ++r) __builtin_nontemporal_store(f32_to_bf16(ok ? O[r] * rl : 0.f), dst + 4 * r);
  }
}

}  // namespace

hipError_t launch_ring_decode(const RingDecodeArgs& a, hipStream_t s) {
  const int nhg = a.G <= 16 ? 1 : a.G / 16;
  const dim3 grid(a.Hkv * nhg, a.B);
  if (a.D == 128) {
    if (nhg == 1) hipLaunchKernelGGL((ring_decode_kernel<128, true>), grid, dim3(RD_THREADS), 0, s, a);
    else hipLaunchKernelGGL((ring_decode_kernel<128, false>), grid, dim3(RD_THREADS), 0, s, a);
  } else {
    if (nhg == 1) hipLaunchKernelGGL((ring_decode_kernel<64, true>), grid, dim3(RD_THREADS), 0, s, a);
    else hipLaunchKernelGGL((ring_decode_kernel<64, false>), grid, dim3(RD_THREADS), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace hsk
