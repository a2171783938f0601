// The attention tile pipeline shared by the sliding-window / full prefill and the
// block-sparse union attention (gfx950, bf16 in, fp32 accumulate).
//
// A wave owns 32 query rows of one head.  For each 64-key tile staged in LDS it
//   1. computes S^T = K * Q^T with v_mfma_f32_32x32x16_bf16 (A = K rows from LDS,
//      B = the wave's Q fragment held in registers for the whole loop), so lane l
//      holds 32 scores of query row l%32 and lane l^32 the other 32;
//   2. masks edge tiles, runs the online softmax in the log2 domain (row max via
//      one permlane32 swap, v_exp_f32 on fma(s, scale*log2e, -m)); the offset m
//      and the accumulator are only rescaled when a row maximum grows by > 2^8,
//      and the row sum is taken with v_dot2_f32_bf16 on the packed bf16 P;
//   3. accumulates O^T += V^T * P^T: P^T is the softmax output in place (its key
//      order is matched by the V^T operand), V^T comes from LDS through two
//      ds_read_b64_tr_b16 per MFMA.
// K/V tiles are stored in LDS with a 16-byte-chunk XOR swizzle.
#pragma once

#include "common.hpp"

namespace hsk {

constexpr int FT_BN = 64;  // keys per tile
constexpr int FT_KPF = 4;  // K fragments read ahead

template <int D>
struct FtCfg {
  static constexpr int NCH = D / 8;          // 16-byte chunks per K/V row
  static constexpr int TILE = FT_BN * D * 2;  // bytes of one K (or V) tile
  static constexpr int DC = D / 16;          // k-steps of S^T
  static constexpr int DB = D / 32;          // 32-row d blocks of O^T
};

// Chunk swizzle.  D = 128 (16 chunks of 16 B per row): 16 consecutive rows read at
// one logical chunk land on 16 different chunks (the K operand reads), and the 4
// consecutive rows of one transpose read keep an aligned group of 4 chunks on 4
// disjoint groups (the V^T reads).  D = 64 (8 chunks): the same idea on 3 bits.
template <int NCH>
__device__ __forceinline__ int ft_swz(int row) {
  if (NCH == 16) return ((row & 3) << 2) | ((row >> 2) & 3);
  return ((row & 1) << 2) | ((row >> 1) & 3);
}

template <int NCH>
__device__ __forceinline__ int ft_off(int row, int chunk) {
  return row * NCH * 16 + ((chunk ^ ft_swz<NCH>(row)) << 4);
}

typedef __attribute__((address_space(3))) void lds_void;

// Wait until this wave's vector-memory operations (here: LDS DMA loads) are done.
__device__ __forceinline__ void wait_vmem() {
  // s_waitcnt vmcnt(0); expcnt and lgkmcnt left at their maximum (no wait)
  __builtin_amdgcn_s_waitcnt(0x0F70);
}

// Workgroup barrier for the tile loops.  This wave's LDS reads complete first
// (lgkmcnt 0); there is no memory fence, so the tile DMAs still in flight stay
// in flight (the caller has already waited for the ones it needs).  The memory
// clobber keeps the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Global -> LDS staging by buffer_load_dwordx4 ... lds (no registers involved).
// One instruction moves 1 KB: lane i's 16 bytes land at LDS base + 16 i, so each
// lane fetches the global chunk that the XOR swizzle places there.  Reads past
// num_records return zero, which pads the last partial tile.  Offsets are 32-bit
// byte offsets from a per-(sequence, head) base.
template <int D, int NT>
struct TileDma {
  using C = FtCfg<D>;
  static constexpr int RPI = 1024 / (D * 2);                 // rows per 1 KB instruction
  static constexpr int PER_WAVE = FT_BN / RPI / (NT / 64);   // instructions per wave per tensor
  __amdgpu_buffer_rsrc_t rk, rv;
  unsigned voff[PER_WAVE];
  unsigned tile_bytes;  // bytes between consecutive 64-row tiles
  int wave_lds;         // this wave's first 1 KB block in a tile

  // kbase/vbase: row 0 of this head; row stride in bytes; nrows valid rows
  __device__ __forceinline__ void init(const uint16_t* kbase, const uint16_t* vbase, unsigned row_bytes,
                                       int nrows, int wave) {
    const unsigned nrec = (unsigned)(nrows - 1) * row_bytes + D * 2;
    rk = __builtin_amdgcn_make_buffer_rsrc((void*)kbase, (short)0, (int)nrec, 0x00020000);
    rv = __builtin_amdgcn_make_buffer_rsrc((void*)vbase, (short)0, (int)nrec, 0x00020000);
    tile_bytes = FT_BN * row_bytes;
    wave_lds = wave * PER_WAVE * 1024;
    const int lane = __lane_id();
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) {
      const int blk = wave * PER_WAVE + i;
      const int row = blk * RPI + lane / C::NCH;
      const int chunk = (lane % C::NCH) ^ ft_swz<C::NCH>(row);
      voff[i] = (unsigned)row * row_bytes + chunk * 16;
    }
  }
  // one of two staging descriptors, chosen by value (a wave-uniform choice); a
  // choice by reference would send both descriptors through scratch memory
  __device__ __forceinline__ static TileDma pick(bool first, const TileDma& x, const TileDma& y) {
    TileDma r;
    r.rk = first ? x.rk : y.rk;
    r.rv = first ? x.rv : y.rv;
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) r.voff[i] = first ? x.voff[i] : y.voff[i];
    r.tile_bytes = first ? x.tile_bytes : y.tile_bytes;
    r.wave_lds = x.wave_lds;
    return r;
  }
  // start loading tile kt into the LDS buffer kv_lds (K then V, TILE bytes each)
  __device__ __forceinline__ void issue(int kt, char* kv_lds) const {
    const unsigned so = (unsigned)kt * tile_bytes;
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void*)(kv_lds + wave_lds + i * 1024), 16, voff[i], so, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void*)(kv_lds + C::TILE + wave_lds + i * 1024), 16, voff[i],
                                               so, 0, 0);
    }
  }
};

template <int D>
struct FlashWave {
  using C = FtCfg<D>;
  bf16x8 qf[C::DC];
  f32x16 o[C::DB];
  float m, l;
  // Per-lane LDS byte offsets of the K reads (k-step c, key sub-block 0) and the
  // V^T reads (d block, low/high 8 keys, key group 0).  The swizzle of a lane's
  // row does not change between key sub-blocks or key groups, so every other
  // read is one of these plus a constant.
  int ko[C::DC];
  int vo[C::DB][2];

  // qrow: this lane's query row (D values) or nullptr for rows past the end
  __device__ __forceinline__ void init(const uint16_t* qrow) {
    const int lane = __lane_id();
#pragma unroll
    for (int c = 0; c < C::DC; ++c) {
      uint4 t = make_uint4(0, 0, 0, 0);
      if (qrow) t = *(const uint4*)(qrow + 16 * c + 8 * (lane >> 5));
      qf[c] = as_bf16x8(t);
    }
#pragma unroll
    for (int d = 0; d < C::DB; ++d)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[d][r] = 0.f;
    m = kNegInf;
    l = 0.f;
#pragma unroll
    for (int c = 0; c < C::DC; ++c) ko[c] = ft_off<C::NCH>(lane & 31, 2 * c + (lane >> 5));
    const int gq = lane >> 4, sl = lane & 15;
    const int kr = 4 * (gq >> 1) + (sl >> 2);
#pragma unroll
    for (int d = 0; d < C::DB; ++d) {
      const int col = 32 * d + 16 * (gq & 1) + 4 * (sl & 3);
      vo[d][0] = ft_off<C::NCH>(kr, col >> 3) + ((col & 7) << 1);
      vo[d][1] = ft_off<C::NCH>(kr + 8, col >> 3) + ((col & 7) << 1);
    }
  }

  // Visibility of the 64-key tile at k0 for rows r0 .. r0+31 (0 <= row - key < W,
  // or every key when `full`): 0 none, 1 partly (edge tile, needs the mask), 2 all.
  __device__ __forceinline__ static int visible(int k0, int r0, int W, bool full) {
    if (full) return 2;
    if ((k0 > r0 + 31) || (k0 + FT_BN - 1 < r0 - W + 1)) return 0;
    return ((k0 + FT_BN - 1 <= r0) && (r0 + 31 - k0 < W)) ? 2 : 1;
  }

  // S^T for the tile whose K rows are at ks: lane l gets the scores of query row
  // l%32 with keys 32 sub + 8 (r/4) + 4 (l/32) + r%4 in s[sub][r].
  __device__ __forceinline__ void qk(const char* ks, f32x16 (&s)[2]) const {
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[sub][r] = 0.f;
    // the two key blocks are independent accumulation chains: alternate them.
    // K fragments are read FT_KPF steps ahead of their MFMA (a rolling window of
    // registers), so LDS latency hides behind the MFMAs in between; the
    // scheduling barriers keep the compiler from regrouping the reads next to
    // their MFMAs (its own order waited for a read before nearly every MFMA).
    constexpr int NS = 2 * C::DC;
    bf16x8 kb[FT_KPF];
    auto kread = [&](int i) {  // step i: key block i % 2, k-step i / 2
      return *(const bf16x8*)(ks + 32 * (i & 1) * C::NCH * 16 + ko[i >> 1]);
    };
#pragma unroll
    for (int i = 0; i < FT_KPF; ++i) kb[i] = kread(i);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const bf16x8 ka = kb[i % FT_KPF];
      if (i + FT_KPF < NS) kb[i % FT_KPF] = kread(i + FT_KPF);
      s[i & 1] = mfma32(ka, qf[i >> 1], s[i & 1]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // Online softmax of one tile's scores (masked when `mask`; k0: first key of the
  // tile, row: this lane's query row): updates m, l (and rescales o) and packs the
  // probabilities as bf16 pairs in the key order the P^T operand of pv() expects.
  __device__ __forceinline__ void softmax(f32x16 (&s)[2], bool mask, int k0, int row, int W,
                                          float scale_log2, u32x4 (&pw)[4]) {
    const int lane = __lane_id();
    if (__builtin_expect(mask, 0)) {  // edge tile (wave-uniform branch)
      // key of register r: k0 + 32 sub + 8 (r/4) + 4 (lane/32) + r%4
      const int d0 = row - k0 - 4 * (lane >> 5);
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int dd = d0 - 32 * sub - 8 * (r >> 2) - (r & 3);
          if ((unsigned)dd >= (unsigned)W) s[sub][r] = kNegInf;
        }
    }
    float mx = kNegInf;
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[sub][r]);
    mx = fmaxf(mx, xor32(mx));
    // Lazy rescale: the exponent offset m only moves when a row's maximum grows
    // by more than 8 (a factor 256), so most tiles skip the accumulator rescale.
    // Exact after the final division: numerator and denominator share m.
    const float mts = mx * scale_log2;
    if (__any(mts > m + 8.f)) {
      const float m_new = fmaxf(m, mts);
      const float alpha = (m == kNegInf) ? 0.f : fast_exp2(m - m_new);
      l *= alpha;
#pragma unroll
      for (int d = 0; d < C::DB; ++d)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[d][r] *= alpha;
      m = m_new;
    }
    const float negm = (m == kNegInf) ? 0.f : -m;
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
    for (int kap = 0; kap < 4; ++kap) {
      const int sub = kap >> 1, half = kap & 1;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float p0 = fast_exp2(fmaf(s[sub][8 * half + 2 * j], scale_log2, negm));
        const float p1 = fast_exp2(fmaf(s[sub][8 * half + 2 * j + 1], scale_log2, negm));
        bf16x2 pp;
        pp[0] = (__bf16)p0;
        pp[1] = (__bf16)p1;
        pw[kap][j] = __builtin_bit_cast(unsigned, pp);
        // the normaliser sums the same bf16-rounded probabilities the MFMA uses
        // (the pair is kept as its own value: bit-casting a u32x4 element here
        // made hipcc reuse element 0 for every j)
        l = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, l, false);
      }
    }
  }

  // O^T += V^T * P^T for the tile whose V rows are at vs.
  __device__ __forceinline__ void pv(const char* vs, const u32x4 (&pw)[4]) {
#pragma unroll
    for (int kap = 0; kap < 4; ++kap) {
      const bf16x8 pb = as_bf16x8(pw[kap]);
      // k-slot j of lane group gq/2 <-> key 16 kap + 4 (gq/2) + j (j < 4) or + 8 + (j - 4);
      // lane (gq, sl) reads V row 16 kap + 4 (gq/2) + sl/4 (+ 8), columns
      // 32 d + 16 (gq&1) + 4 (sl&3) .. + 3
      const char* vk = vs + 16 * kap * C::NCH * 16;
#pragma unroll
      for (int d = 0; d < C::DB; ++d) {
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vk + vo[d][0]));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vk + vo[d][1]));
        typedef __attribute__((ext_vector_type(8))) short s16x8;
        const s16x8 va = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        o[d] = mfma32(__builtin_bit_cast(bf16x8, va), pb, o[d]);
      }
    }
  }

  // One 64-key tile at key position k0 held in LDS (K at ks, V at vs).
  // r0: first query row of the wave; row: this lane's row; visibility is
  // 0 <= row - key < W unless `full` (every key of the tile visible to every row).
  __device__ __forceinline__ void tile(const char* ks, const char* vs, int k0, int r0, int row,
                                       int W, bool full, float scale_log2) {
    const int v = visible(k0, r0, W, full);
    if (v == 0) return;
    f32x16 s[2];
    u32x4 pw[4];
    qk(ks, s);
    softmax(s, v == 1, k0, row, W, scale_log2, pw);
    pv(vs, pw);
  }

  // normalise and store this lane's row (orow = nullptr: row not stored)
  __device__ __forceinline__ void store(uint16_t* orow) {
    const int lane = __lane_id();
    const float lt = l + xor32(l);
    const float inv = 1.f / lt;
    if (!orow) return;
#pragma unroll
    for (int d = 0; d < C::DB; ++d)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d0 = 32 * d + 8 * r4 + 4 * (lane >> 5);
        uint2 st;
        st.x = pack_bf16x2(o[d][4 * r4 + 0] * inv, o[d][4 * r4 + 1] * inv);
        st.y = pack_bf16x2(o[d][4 * r4 + 2] * inv, o[d][4 * r4 + 3] * inv);
        *(uint2*)(orow + d0) = st;
      }
  }
};

}  // namespace hsk
