// Top-k selection of one row of candidates by a wave (order-preserving 64-bit
// keys in registers, bit-by-bit threshold search with ballots).
#pragma once

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
template <int MAXG, class Emit>
__device__ __forceinline__ int topk_select_row(const unsigned long long (&keys)[MAXG], int n, int topk,
                                               unsigned long long* gather, Emit emit) {
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
    const int kb = i * 64 + lane;
    const bool valid = kb < n;
    const bool is_gt = valid && keys[i] > T;
    const bool is_eq = valid && keys[i] == T;
    const unsigned long long eqb = __ballot(is_eq);
    const int rank = eq_before + __popcll(eqb & lt_mask);
    const bool take = is_gt || (is_eq && rank < need);
    const unsigned long long tb = __ballot(take);
    const int slot = written + __popcll(tb & lt_mask);
    if (take && slot < topk) emit(slot, kb);
    written += __popcll(tb);
    eq_before += __popcll(eqb);
  }
  return written;
}

}  // namespace hsk
