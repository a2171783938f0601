// Top-k selection of one row of candidates by a wave (order-preserving 64-bit
// keys in registers, bit-by-bit threshold search with ballots).
#pragma once

#include <type_traits>

#include "common.hpp"

namespace hsk {

// 64-bit key whose unsigned order is the order of the double (-0 taken as +0)
__device__ __forceinline__ unsigned long long order_key(double x) {
  const unsigned long long u = (unsigned long long)__double_as_longlong(x + 0.0);  // -0 -> +0
  return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}

// Candidates 0 .. n-1 of one row, lane l holding candidate 64 i + l in keys[i]
// (n <= 64 MAXG; absent candidates hold key 0, below every real key, and every
// threshold tried is above 0, so they never count).  Keeps the topk largest keys,
// ties to the lower index: the threshold T is the largest key with
// #{key >= T} >= topk, searched over the top 16 bits first and then over the
// candidates sharing that 16-bit prefix (gathered one per lane through `gather`,
// 64 words of LDS owned by this wave; the full search remains for rows with more
// than 64 of them).  Calls emit(slot, index) for every kept candidate, slot being
// its rank in ascending index order; returns how many were kept.  Needs n > topk.
// Every loop runs over all MAXG groups with no per-group condition: a runtime
// group count made each group a branch of its own.
//
// topk_core is the search with the candidate's index given by index_of(i) for the
// lane's candidate of group i (positions i*64 + lane must be in ascending index
// order); topk_select_row uses the position itself.
template <int MAXG, class IndexOf, class Emit>
__device__ __forceinline__ int topk_core(const unsigned long long (&keys)[MAXG], int n, int topk,
                                         unsigned long long* gather, IndexOf index_of, Emit emit) {
  const int lane = __lane_id();
  auto count_ge = [&](unsigned long long c) {
    int cnt = 0;
#pragma unroll
    for (int i = 0; i < MAXG; ++i) cnt += __popcll(__ballot(keys[i] >= c));
    return cnt;
  };
  // 1. the top 16 bits over every candidate
  unsigned long long T = 0;
  for (int bit = 63; bit >= 48; --bit) {
    const unsigned long long cand = T | (1ull << bit);
    if (count_ge(cand) >= topk) T = cand;
  }
  // 2. the low 48 bits: only keys with T's 16-bit prefix can still change a count
  const unsigned long long pre = T >> 48;
  const int above = pre == 0xffffull ? 0 : count_ge((pre + 1) << 48);
  const unsigned long long lt_mask = (1ull << lane) - 1ull;
  int neq = 0;
#pragma unroll
  for (int i = 0; i < MAXG; ++i) {
    const bool eq = (keys[i] >> 48) == pre && keys[i] != 0ull;
    const unsigned long long m = __ballot(eq);
    const int pos = neq + __popcll(m & lt_mask);
    if (eq && pos < 64) gather[pos] = keys[i];
    neq += __popcll(m);
  }
  if (neq <= 64) {
    __builtin_amdgcn_wave_barrier();
    const unsigned long long ek = lane < neq ? gather[lane] : 0ull;
    for (int bit = 47; bit >= 0; --bit) {
      const unsigned long long cand = T | (1ull << bit);
      if (above + (int)__popcll(__ballot(ek >= cand)) >= topk) T = cand;
    }
  } else {  // many candidates share the prefix (ties): search over all of them
    for (int bit = 47; bit >= 0; --bit) {
      const unsigned long long cand = T | (1ull << bit);
      if (count_ge(cand) >= topk) T = cand;
    }
  }
  int gt = 0;
#pragma unroll
  for (int i = 0; i < MAXG; ++i) gt += __popcll(__ballot(keys[i] > T));
  const int need = topk - gt;
  int eq_before = 0, written = 0;
#pragma unroll
  for (int i = 0; i < MAXG; ++i) {
    const bool valid = i * 64 + lane < n;
    const bool is_gt = valid && keys[i] > T;
    const bool is_eq = valid && keys[i] == T;
    const unsigned long long eqb = __ballot(is_eq);
    const int rank = eq_before + __popcll(eqb & lt_mask);
    const bool take = is_gt || (is_eq && rank < need);
    const unsigned long long tb = __ballot(take);
    const int slot = written + __popcll(tb & lt_mask);
    if (take && slot < topk) emit(slot, index_of(i));
    written += __popcll(tb);
    eq_before += __popcll(eqb);
  }
  return written;
}

template <int MAXG, class Emit>
__device__ __forceinline__ int topk_select_row(const unsigned long long (&keys)[MAXG], int n, int topk,
                                               unsigned long long* gather, Emit emit) {
  const int lane = __lane_id();
  return topk_core<MAXG>(keys, n, topk, gather, [&](int i) { return i * 64 + lane; }, emit);
}


// The same selection with a pre-filter, for rows of at least 64 candidates and
// topk <= 64: every lane holds a real candidate and its largest key is >= T0, the
// smallest of the 64 lane maxima, so at least 64 keys are >= T0 and every kept key
// (the topk-th largest and above, ties included) is >= T0.  When at most
// 64 CF keys are >= T0 they are gathered in index order through ck / ci (LDS of
// this wave, 64 CF entries each) and searched
// instead of all MAXG groups; otherwise the full search runs.  CF (8 or 16)
// groups of candidates at most: the search runs over CF/2 groups when they fit,
// else over CF (a wider search costs registers, so callers with many rows per
// CU take CF = 8).
template <int CF, int MAXG, class Emit>
__device__ __forceinline__ int topk_select_row_filtered(const unsigned long long (&keys)[MAXG], int n, int topk,
                                                        unsigned long long* gather, unsigned long long* ck,
                                                        int* ci, Emit emit) {
  static_assert(CF == 8 || CF == 16, "8 or 16 candidate groups");
  const int lane = __lane_id();
  if (MAXG <= CF / 2 || n < 64 || topk > 64) return topk_select_row<MAXG>(keys, n, topk, gather, emit);
  unsigned long long lm = 0;
#pragma unroll
  for (int i = 0; i < MAXG; ++i) lm = keys[i] > lm ? keys[i] : lm;
  // wave minimum of the lane maxima (64-bit, as two 32-bit halves)
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const unsigned lo = __shfl_xor((unsigned)lm, off), hi = __shfl_xor((unsigned)(lm >> 32), off);
    const unsigned long long o = ((unsigned long long)hi << 32) | lo;
    lm = o < lm ? o : lm;
  }
  const unsigned long long t0 = lm;
  int cnt = 0;
#pragma unroll
  for (int i = 0; i < MAXG; ++i) cnt += __popcll(__ballot(keys[i] >= t0));
  // the narrower search only pays while it has fewer groups than the full one
  if (cnt > 64 * (CF / 2) && (MAXG <= CF || cnt > 64 * CF)) return topk_select_row<MAXG>(keys, n, topk, gather, emit);
  const unsigned long long lt_mask = (1ull << lane) - 1ull;
  int base = 0;
#pragma unroll
  for (int i = 0; i < MAXG; ++i) {
    const bool c = keys[i] >= t0;
    const unsigned long long m = __ballot(c);
    if (c) {
      const int pos = base + __popcll(m & lt_mask);
      ck[pos] = keys[i];
      ci[pos] = i * 64 + lane;
    }
    base += __popcll(m);
  }
  __builtin_amdgcn_wave_barrier();
  auto search = [&](auto groups) {
    constexpr int NG = decltype(groups)::value;
    unsigned long long fk[NG];
    int fi[NG];
#pragma unroll
    for (int j = 0; j < NG; ++j) {
      const bool in = j * 64 + lane < cnt;
      fk[j] = in ? ck[j * 64 + lane] : 0ull;
      fi[j] = in ? ci[j * 64 + lane] : 0;
    }
    __builtin_amdgcn_wave_barrier();  // ck / ci are free again once read
    return topk_core<NG>(fk, cnt, topk, gather, [&](int j) { return fi[j]; }, emit);
  };
  if (cnt <= 64 * (CF / 2)) return search(std::integral_constant<int, CF / 2>());
  return search(std::integral_constant<int, (MAXG > CF ? CF : CF / 2)>());  // MAXG > CF here
}

}  // namespace hsk
