// One-token decode on v_mfma_f32_16x16x32_bf16, shared by the ring decode and
// the INT8 + bf16 decode.
//
// A wave processes 32-key (or 16-key) chunks with the (up to 16) query heads of
// one KV head on the MFMA N axis; lane l serves head l%16 (lanes past the group
// duplicate its last head) and lane group g = l/16:
//   S   = K * q^T      A = K rows (16 keys x 32 d), B = q^T
//                      -> lane l holds the scores of keys 16t + 4g + r (t<2, r<4)
//   O^T += V^T * P^T   A = V^T (16 d x 32 keys), B = P^T: a lane's 8 probabilities
//                      are exactly its B operand, in the key order of its scores;
//                      the V^T operand takes, for its lane's d, the same 8 keys:
//                      each lane reads 4 adjacent d from 8 rows and the packing
//                      order performs the transpose.
// Output: lane l holds O[head l%16][64 hv + 16 g + 4 r + jj] for the tile (hv, jj).
// INT8 rows are converted exactly to bf16 in registers (|code| <= 127); the K
// scale multiplies the chunk's scores, the V scale the chunk's PV partial.
#pragma once

#include "common.hpp"

namespace hsk {

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

// Branch-free selects on loaded data: a conditional overwrite of a register
// that a load is filling makes the compiler wait for that load right away, so
// masking is done with bit operations on the loaded value instead.
__device__ __forceinline__ unsigned lane_mask(bool c) { return c ? 0xffffffffu : 0u; }
__device__ __forceinline__ uint2 and2(uint2 a, unsigned m) { return make_uint2(a.x & m, a.y & m); }
__device__ __forceinline__ uint4 sel4(uint4 a, uint4 b, unsigned m) {  // m ? a : b
  return make_uint4((a.x & m) | (b.x & ~m), (a.y & m) | (b.y & ~m), (a.z & m) | (b.z & ~m), (a.w & m) | (b.w & ~m));
}
__device__ __forceinline__ uint2 sel2(uint2 a, uint2 b, unsigned m) {
  return make_uint2((a.x & m) | (b.x & ~m), (a.y & m) | (b.y & ~m));
}

// BLOCKED selects which 8 d values lane group g contributes to QK MFMA (kk, e):
//   false: d = 64 kk + 16 g + 8 e + j (a 16-byte load of 16 INT8 codes feeds e = 0, 1)
//   true:  d = 64 kk + 32 e + 8 g + j (bf16 rows: each load instruction then reads
//          64 contiguous bytes of a row instead of 16 bytes every 32)
// Any consistent assignment of d to the contraction slots gives the same scores.
// Row length of a stashed wave state in LDS: D floats padded to a multiple of
// 16 bytes plus 16, so each head's row starts 16-byte aligned (128-bit stores)
// and the rows of neighbouring heads start in different banks.
template <int D>
constexpr int stash_row() { return D + 4; }

template <int D, bool BLOCKED = false>
struct DecodeWave {
  static constexpr int NK = D / 64;
  __device__ __forceinline__ static int qk_col(int kk, int e, int gq) {
    return BLOCKED ? 64 * kk + 32 * e + 8 * gq : 64 * kk + 16 * gq + 8 * e;
  }
  bf16x8 qb[NK][2];  // q^T operands
  f32x4 o[NK][4];    // O^T tiles (hv, jj)
  float m, l;

  // q: the group's first query head; G heads of D values each, stride D.
  // Lanes past G re-read head G-1: every head is its own MFMA column, so those
  // duplicate columns never mix with the real ones and are simply not stored.
  // (No use of the loaded values here: the ring/cache loads that follow are
  // issued before anything waits for q.)
  __device__ __forceinline__ void init(const uint16_t* q, int G) {
    const int lane = __lane_id();
    const int hl = lane & 15, gq = lane >> 4;
    const uint16_t* qh = q + (size_t)min(hl, G - 1) * D;
#pragma unroll
    for (int kk = 0; kk < NK; ++kk)
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        qb[kk][e] = as_bf16x8(*(const uint4*)(qh + qk_col(kk, e, gq)));
      }
#pragma unroll
    for (int hv = 0; hv < NK; ++hv)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
#pragma unroll
        for (int r = 0; r < 4; ++r) o[hv][jj][r] = 0.f;
    m = kNegInf;
    l = 0.f;
  }

  // Raw register image of one 32-row chunk (K operand rows, V^T source dwords).
  template <bool INT8>
  struct Raw {
    static constexpr int KV = INT8 ? 1 : 2;  // 16-byte loads per (t, kk)
    uint4 k[2][NK][KV];
    unsigned v8[NK][8];
    uint2 v16[NK][8];
  };

  // The replacing row of a ring (bf16 K operand chunks and V^T source dwords),
  // loaded once per workgroup instead of once per chunk.
  struct AltRow {
    uint4 k[NK][2];
    uint2 v[NK];
  };
  template <class Rows>
  __device__ __forceinline__ void load_alt(const Rows& rows, AltRow& alt) const {
    const int lane = __lane_id();
    const int hl = lane & 15, gq = lane >> 4;
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
#pragma unroll
      for (int e = 0; e < 2; ++e)
        alt.k[kk][e] = *(const uint4*)((const uint16_t*)rows.kalt + qk_col(kk, e, gq));
      alt.v[kk] = *(const uint2*)((const uint16_t*)rows.valt + 64 * kk + 4 * hl);
    }
  }

  // One chunk of 16 NT rows c0 .. c0+16 NT-1 of `rows` (NT = 1 or 2 blocks of 16
  // keys; see the row sources below).  sk multiplies the raw scores (scale *
  // log2 e, times the K scale for INT8), sv multiplies the chunk's PV partial
  // (the V scale; INT8 only: bf16 rows accumulate PV in place, sv is ignored).
  template <bool INT8, int NT = 2, class Rows>
  __device__ __forceinline__ void chunk(const Rows& rows, int c0, float sk, float sv) {
    Raw<INT8> raw;
    load<INT8, NT>(rows, c0, raw);
    compute<INT8, NT>(rows, c0, raw, sk, sv);
  }

  // Every load is issued unconditionally from an in-range address; absent rows
  // are zeroed (V) or masked (scores) later with selects, so all of a chunk's
  // loads can be in flight at once (and the next chunk's during this one).
  template <bool INT8, int NT = 2, class Rows>
  __device__ __forceinline__ void load(const Rows& rows, int c0, Raw<INT8>& raw) const {
    static_assert(!(INT8 && BLOCKED), "INT8 rows use the interleaved operand layout");
    const int lane = __lane_id();
    const int hl = lane & 15, gq = lane >> 4;
    constexpr int KV = Raw<INT8>::KV;
    if constexpr (INT8 && Rows::kBuffer) {
      // buffer loads: one per-lane offset each for K and V, the chunk start as the
      // scalar offset and the row / column steps as immediates (no 64-bit address
      // arithmetic per load)
      const int soff = c0 * D;
      const int kl = hl * D + 16 * gq;
      const int vl = 4 * gq * D + 4 * hl;
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int kk = 0; kk < NK; ++kk)
          raw.k[t][kk][0] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                          rows.rk, kl + 16 * t * D + 64 * kk, soff, 0));
#pragma unroll
      for (int hv = 0; hv < NK; ++hv)
#pragma unroll
        for (int j = 0; j < 4 * NT; ++j)
          raw.v8[hv][j] = __builtin_amdgcn_raw_buffer_load_b32(
              rows.rv, vl + (16 * (j >> 2) + (j & 3)) * D + 64 * hv, soff, 0);
      return;
    }
    // Rows::kStream: the rows are read once per call and are too large to stay
    // cached, so they are loaded non-temporally (measured faster for long bf16
    // contexts, slower for the latency-bound 128-slot ring)
    auto ld4 = [](const char* p) {
      if constexpr (Rows::kStream) return __builtin_bit_cast(uint4, __builtin_nontemporal_load((const u32x4*)p));
      else return *(const uint4*)p;
    };
    auto ld2 = [](const char* p) {
      if constexpr (Rows::kStream) return __builtin_bit_cast(uint2, __builtin_nontemporal_load((const u32x2*)p));
      else return *(const uint2*)p;
    };
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const char* kp = (const char*)rows.kaddr(c0 + 16 * t + hl);
#pragma unroll
      for (int kk = 0; kk < NK; ++kk)
#pragma unroll
        for (int e = 0; e < KV; ++e) raw.k[t][kk][e] = ld4(kp + (INT8 ? 64 * kk + 16 * gq : 2 * qk_col(kk, e, gq)));
    }
#pragma unroll
    for (int hv = 0; hv < NK; ++hv)
#pragma unroll
      for (int j = 0; j < 4 * NT; ++j) {
        const char* vp = (const char*)rows.vaddr(c0 + 16 * (j >> 2) + 4 * gq + (j & 3));
        if (INT8) raw.v8[hv][j] = *(const unsigned*)(vp + 64 * hv + 4 * hl);
        else raw.v16[hv][j] = ld2(vp + 2 * (64 * hv + 4 * hl));
      }
  }

  // head_bits: bit hl set when head hl takes part in this chunk (a block-sparse
  // decode keeps different blocks per head); the other heads' scores are masked.
  template <bool INT8, int NT = 2, class Rows>
  __device__ __forceinline__ void compute(const Rows& rows, int c0, Raw<INT8>& raw, float sk, float sv,
                                          unsigned head_bits = ~0u) {
    AltRow none;
    compute<INT8, NT>(rows, c0, raw, sk, sv, none, head_bits);
  }

  // alt: the replacing row (used when Rows::kHasAlt and it falls in this chunk)
  template <bool INT8, int NT = 2, class Rows>
  // first: this is the wave's first chunk (o and l are still zero, m is -inf), so
  // the offset is simply the chunk's maximum and nothing needs rescaling
  __device__ __forceinline__ void compute(const Rows& rows, int c0, Raw<INT8>& raw, float sk, float sv,
                                          const AltRow& alt, unsigned head_bits = ~0u, bool first = false) {
    const int lane = __lane_id();
    const int hl = lane & 15, gq = lane >> 4;
    constexpr int KV = Raw<INT8>::KV;
    auto& kraw = raw.k;
    auto& vraw8 = raw.v8;
    auto& vraw16 = raw.v16;
    // Both conditions are wave-uniform: chunks without the replaced row, and
    // chunks whose rows are all present, skip the per-register selects.
    if (Rows::kHasAlt && !INT8 && rows.alt_in(c0, 16 * NT)) {
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const unsigned am = lane_mask(rows.is_alt(c0 + 16 * t + hl));
#pragma unroll
        for (int kk = 0; kk < NK; ++kk)
#pragma unroll
          for (int e = 0; e < KV; ++e) kraw[t][kk][e] = sel4(alt.k[kk][e], kraw[t][kk][e], am);
      }
#pragma unroll
      for (int j = 0; j < 4 * NT; ++j) {
        const unsigned am = lane_mask(rows.is_alt(c0 + 16 * (j >> 2) + 4 * gq + (j & 3)));
#pragma unroll
        for (int hv = 0; hv < NK; ++hv) vraw16[hv][j] = sel2(alt.v[hv], vraw16[hv][j], am);
      }
    }
    const bool partial = !Rows::kAllValid && !rows.all_valid(c0, 16 * NT);
    if (partial) {  // absent rows contribute nothing (their bytes may be anything)
#pragma unroll
      for (int j = 0; j < 4 * NT; ++j) {
        const unsigned ok = lane_mask(rows.valid(c0 + 16 * (j >> 2) + 4 * gq + (j & 3)));
#pragma unroll
        for (int hv = 0; hv < NK; ++hv) {
          if (INT8) vraw8[hv][j] &= ok;
          else vraw16[hv][j] = and2(vraw16[hv][j], ok);
        }
      }
    }
    f32x4 s[2];
    if (NT == 1) {  // one key block: split its contraction into two chains
      f32x4 s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int r = 0; r < 4; ++r) s[0][r] = 0.f;
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) {
        bf16x8 a0, a1;
        if (INT8) {
          cvt16(kraw[0][kk][0], a0, a1);
        } else {
          a0 = as_bf16x8(kraw[0][kk][0]);
          a1 = as_bf16x8(kraw[0][kk][KV - 1]);
        }
        s[0] = mfma16(a0, qb[kk][0], s[0]);
        s1 = mfma16(a1, qb[kk][1], s1);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) s[0][r] += s1[r];
    } else {
#pragma unroll
      for (int t = 0; t < NT; ++t) {
#pragma unroll
        for (int r = 0; r < 4; ++r) s[t][r] = 0.f;
#pragma unroll
        for (int kk = 0; kk < NK; ++kk) {
          bf16x8 a0, a1;
          if (INT8) {
            cvt16(kraw[t][kk][0], a0, a1);
          } else {
            a0 = as_bf16x8(kraw[t][kk][0]);
            a1 = as_bf16x8(kraw[t][kk][KV - 1]);
          }
          s[t] = mfma16(a0, qb[kk][0], s[t]);
          s[t] = mfma16(a1, qb[kk][1], s[t]);
        }
      }
    }
    u32x4 va[NK][4];
#pragma unroll
    for (int hv = 0; hv < NK; ++hv) {
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        u32x4& t = va[hv][jj];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (2 * q >= 4 * NT) {  // key slots past the chunk: zero
            t[q] = 0u;
          } else if (INT8) {
            t[q] = pack_bf16x2(i8(vraw8[hv][2 * q], jj), i8(vraw8[hv][2 * q + 1], jj));
          } else {
            const unsigned x0 = (jj < 2) ? vraw16[hv][2 * q].x : vraw16[hv][2 * q].y;
            const unsigned x1 = (jj < 2) ? vraw16[hv][2 * q + 1].x : vraw16[hv][2 * q + 1].y;
            // low or high bf16 of each dword -> one packed pair
            t[q] = (jj & 1) ? __builtin_amdgcn_perm(x1, x0, 0x07060302u)
                            : __builtin_amdgcn_perm(x1, x0, 0x05040100u);
          }
        }
      }
    }
    float x[8];
    float mx = kNegInf;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float v = kNegInf;
        if (t < NT) {
          v = s[t][r] * sk;
          if (partial && !rows.valid(c0 + 16 * t + 4 * gq + r)) v = kNegInf;
          if (!((head_bits >> hl) & 1u)) v = kNegInf;
        }
        x[4 * t + r] = v;
        mx = fmaxf(mx, v);
      }
    mx = fmaxf(mx, xor16(mx));
    mx = fmaxf(mx, xor32(mx));
    // Lazy offset: m only moves when a head's maximum grows by more than 8 (a
    // factor 256 in the log2 domain), so most chunks skip the accumulator rescale;
    // numerator and denominator always share m.
    if (first) {
      m = mx;
    } else if (__any(mx > m + 8.f)) {
      const float m_new = fmaxf(m, mx);
      const float alpha = (m == kNegInf) ? 0.f : fast_exp2(m - m_new);
      l *= alpha;
#pragma unroll
      for (int hv = 0; hv < NK; ++hv)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
#pragma unroll
          for (int r = 0; r < 4; ++r) o[hv][jj][r] *= alpha;
      m = m_new;
    }
    const float base = (m == kNegInf) ? 0.f : m;
    // P is rounded to bf16 for the MFMA; the normaliser sums the same rounded
    // values, so a row dominated by one key returns that key's value exactly.
    float ps = 0.f;
    u32x4 pw;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (2 * q >= 4 * NT) {
        pw[q] = 0u;
        continue;
      }
      const float p0 = fast_exp2(x[2 * q] - base), p1 = fast_exp2(x[2 * q + 1] - base);
      pw[q] = pack_bf16x2(p0, p1);
      ps += bf16lo(pw[q]) + bf16hi(pw[q]);
    }
    l += ps;
    if constexpr (INT8) {  // the chunk's partial, scaled by its V scale
      const bf16x8 pb = as_bf16x8(pw);
#pragma unroll
      for (int hv = 0; hv < NK; ++hv)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          f32x4 part = {0.f, 0.f, 0.f, 0.f};
          part = mfma16(as_bf16x8(va[hv][jj]), pb, part);
#pragma unroll
          for (int r = 0; r < 4; ++r) o[hv][jj][r] = fmaf(sv, part[r], o[hv][jj][r]);
        }
    } else if constexpr (NT == 1) {
      // one key block: its 16 keys are exactly the 16-deep form's contraction
      // (lane group g holds keys 4g..4g+3 in both operands), so the zero half
      // of the 32-deep operands is not formed; bf16 rows accumulate in place
      const u32x2 pb = {pw[0], pw[1]};
#pragma unroll
      for (int hv = 0; hv < NK; ++hv)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const u32x2 v2 = {va[hv][jj][0], va[hv][jj][1]};
          o[hv][jj] = mfma16k16(v2, pb, o[hv][jj]);
        }
    } else {
      const bf16x8 pb = as_bf16x8(pw);
#pragma unroll
      for (int hv = 0; hv < NK; ++hv)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) o[hv][jj] = mfma16(as_bf16x8(va[hv][jj]), pb, o[hv][jj]);
    }
  }

  // Write this wave's state for the heads it serves (lane%16 < G) to LDS:
  // sm_m/sm_l [waves][16], sm_o [waves][16][stash_row<D>()].  A head's row holds
  // its D accumulators in tile order: tile (hv, jj) of lane group g is one
  // 128-bit write at column 64 hv + 16 jj + 4 g (its four registers r are
  // d = 64 hv + 16 g + 4 r + jj); stash_col maps d to its column.
  __device__ __forceinline__ static int stash_col(int d) {
    return (d & ~63) + 16 * (d & 3) + 4 * ((d >> 4) & 3) + ((d >> 2) & 3);
  }
  __device__ __forceinline__ void stash(float (*sm_m)[16], float (*sm_l)[16], float (*sm_o)[16][stash_row<D>()],
                                        int w, int G) {
    const int lane = __lane_id();
    const int hl = lane & 15, gq = lane >> 4;
    float lsum = l;
    lsum += xor16(lsum);
    lsum += xor32(lsum);
    if (hl < G) {
#pragma unroll
      for (int hv = 0; hv < NK; ++hv)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
          *(f32x4*)&sm_o[w][hl][64 * hv + 16 * jj + 4 * gq] = o[hv][jj];
      if (gq == 0) {
        sm_m[w][hl] = m;
        sm_l[w][hl] = lsum;
      }
    }
  }
};

// Merge NW stashed wave states for (head, d): returns acc, sets M and Lsum.
template <int NW, int D>
__device__ __forceinline__ float merge_waves(const float (*sm_m)[16], const float (*sm_l)[16],
                                             const float (*sm_o)[16][stash_row<D>()], int head, int d,
                                             float& M, float& Ls) {
  const int col = DecodeWave<D>::stash_col(d);
  M = kNegInf;
#pragma unroll
  for (int i = 0; i < NW; ++i) M = fmaxf(M, sm_m[i][head]);
  float O = 0.f;
  Ls = 0.f;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const float f = (sm_m[i][head] == kNegInf) ? 0.f : fast_exp2(sm_m[i][head] - M);
    O += f * sm_o[i][head][col];
    Ls += f * sm_l[i][head];
  }
  return O;
}

// Merge NW stashed wave states for the four columns col .. col+3 (col a
// multiple of 4) of a head's row: returns the four accumulators, sets M and
// Lsum (the wave factors are formed once for the four).  Every LDS read is
// issued before the arithmetic, so the merge waits for LDS once.
template <int NW, int D>
__device__ __forceinline__ f32x4 merge_waves4(const float (*sm_m)[16], const float (*sm_l)[16],
                                              const float (*sm_o)[16][stash_row<D>()], int head, int col,
                                              float& M, float& Ls) {
  float mv[NW], lv[NW];
  float4 ov[NW];
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    mv[i] = sm_m[i][head];
    lv[i] = sm_l[i][head];
    ov[i] = *(const float4*)&sm_o[i][head][col];
  }
  __builtin_amdgcn_sched_barrier(0);
  M = kNegInf;
#pragma unroll
  for (int i = 0; i < NW; ++i) M = fmaxf(M, mv[i]);
  f32x4 O = {0.f, 0.f, 0.f, 0.f};
  Ls = 0.f;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const float f = (mv[i] == kNegInf) ? 0.f : fast_exp2(mv[i] - M);
    O[0] += f * ov[i].x;
    O[1] += f * ov[i].y;
    O[2] += f * ov[i].z;
    O[3] += f * ov[i].w;
    Ls += f * lv[i];
  }
  return O;
}

// ------------------------------------------------------------ row sources ----
// kaddr/vaddr return an in-range row address for any row of a chunk; valid()
// says whether the row takes part; is_alt() marks the row whose data comes from
// kalt/valt instead (a ring slot being overwritten by the new token).

// Contiguous INT8 rows (always in range: callers pass whole 32-row blocks).
template <int D>
struct Int8Rows {
  static constexpr bool kAllValid = true;
  static constexpr bool kHasAlt = false;
  static constexpr bool kBuffer = true;  // loaded through rk / rv
  static constexpr bool kStream = false;
  const int8_t* k;
  const int8_t* v;
  __amdgpu_buffer_rsrc_t rk, rv;       // the same rows as buffer resources
  const void* kalt = nullptr;
  const void* valt = nullptr;
  __device__ __forceinline__ const void* kaddr(int row) const { return k + (size_t)row * D; }
  __device__ __forceinline__ const void* vaddr(int row) const { return v + (size_t)row * D; }
  __device__ __forceinline__ bool valid(int) const { return true; }
  __device__ __forceinline__ bool all_valid(int, int) const { return true; }
  __device__ __forceinline__ bool is_alt(int) const { return false; }
  __device__ __forceinline__ bool alt_in(int, int) const { return false; }
};

// Contiguous bf16 rows; rows >= end are absent.
template <int D>
struct Bf16Rows {
  static constexpr bool kAllValid = false;
  static constexpr bool kHasAlt = false;
  static constexpr bool kBuffer = false;
  static constexpr bool kStream = true;
  const uint16_t* k;
  const uint16_t* v;
  int end;
  const void* kalt = nullptr;
  const void* valt = nullptr;
  __device__ __forceinline__ const void* kaddr(int row) const { return k + (size_t)min(row, end - 1) * D; }
  __device__ __forceinline__ const void* vaddr(int row) const { return v + (size_t)min(row, end - 1) * D; }
  __device__ __forceinline__ bool valid(int row) const { return row < end; }
  __device__ __forceinline__ bool all_valid(int r0, int n) const { return r0 + n <= end; }
  __device__ __forceinline__ bool is_alt(int) const { return false; }
  __device__ __forceinline__ bool alt_in(int, int) const { return false; }
};

// A W-slot ring after appending position p at slot p mod W.  Slot s holds
// position p - ((p - s) mod W); it is attended when that position is >= 0.  The
// new token's K/V comes from kalt/valt (its ring slot is being overwritten).
template <int D>
struct RingRows {
  static constexpr bool kAllValid = false;
  static constexpr bool kHasAlt = true;
  static constexpr bool kBuffer = false;
  static constexpr bool kStream = false;
  const uint16_t* k;
  const uint16_t* v;
  const void* kalt;
  const void* valt;
  int W, slot, p;
  __device__ __forceinline__ const void* kaddr(int s) const { return k + (size_t)min(s, W - 1) * D; }
  __device__ __forceinline__ const void* vaddr(int s) const { return v + (size_t)min(s, W - 1) * D; }
  __device__ __forceinline__ bool valid(int s) const {
    // (slot - s) mod W for 0 <= s < W, without a division or a branch
    const int d = slot - s;
    return (s < W) & ((d < 0 ? d + W : d) <= p);
  }
  // every slot holds a position >= 0 once p >= W - 1
  __device__ __forceinline__ bool all_valid(int s0, int n) const { return p >= W - 1 && s0 + n <= W; }
  __device__ __forceinline__ bool is_alt(int s) const { return s == slot; }
  __device__ __forceinline__ bool alt_in(int s0, int n) const { return slot >= s0 && slot < s0 + n; }
};

}  // namespace hsk
