// C ABI: host-side argument validation and kernel dispatch.
// Nothing here allocates device memory or keeps state between calls.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>

#include "hybrid_swa_kv.h"
#include "kernels.hpp"

namespace {

constexpr int kAbiVersion = 5;  // 2: swa_window_safe_len, 3: swa_prefill_chunk, 4: sparse INT8 decode,
                                 // 5: attn_decode_int8kv_noalloc

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }
inline bool head_dim_ok(int D) { return D == 64 || D == 128; }
inline float log2e_times(float scale) { return (float)((double)scale * 1.4426950408889634); }

inline int finish(hipError_t e) { return e == hipSuccess ? HSK_OK : HSK_ERR_HIP; }

int check_heads(int Hq, int Hkv, int D) {
  if (Hq <= 0 || Hkv <= 0 || D <= 0) return HSK_ERR_SHAPE;
  if (Hq % Hkv != 0) return HSK_ERR_SHAPE;
  if (!head_dim_ok(D)) return HSK_ERR_UNSUPPORTED;
  return HSK_OK;
}

size_t int8_ws_bytes(int B, int Hq, int Hkv, int D, int T8, int Th) {
  int nsplit, wsplit;
  hsk::int8_decode_plan(B, Hkv, T8, Th, &nsplit, &wsplit);
  return (size_t)B * Hkv * (size_t)nsplit * (size_t)(Hq / Hkv) * (size_t)(D + 2) * sizeof(float);
}

// block sums [Hq + Hkv][nbp][D] and the score triangle [Hq][nb (nb - 1) / 2], fp64
size_t bs_ws_bytes(int L, int Hq, int Hkv, int D, int block) {
  const size_t nb = (size_t)L / block;
  const size_t nbp = (nb + 63) / 64 * 64;
  return (((size_t)Hq + Hkv) * nbp * D + (size_t)Hq * (nb * (nb - 1) / 2)) * sizeof(double);
}

// Block-sparse INT8 decode plan and workspace: fp64 scores [B, Hq, nblk], the
// per-unit union list and head bits [units, lmax], counts [units], then the
// split records [units, nss + nsh, G, D + 2] fp32 (segments 256-byte aligned).
struct SparsePlan {
  int nblk, lmax, epsplit, nss, hsplit, nsh;
  size_t off_scores, off_list, off_mask, off_count, off_rec, bytes;
};

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

SparsePlan sparse_plan(int B, int Hq, int Hkv, int D, int T8, int Th, int topk) {
  SparsePlan p{};
  const int G = Hq / Hkv;
  const size_t units = (size_t)B * Hkv;
  p.nblk = T8 / 32;
  p.lmax = topk > 0 ? std::min(p.nblk, G * topk) : 0;
  // kept blocks per INT8 split: 64 measured 3 % faster than 32 at batch 16 and
  // 1984 blocks (fewer records to merge); 128 and 256 were slower (fewer
  // workgroups than the GPU holds).  At most 256: a wave reads its entries
  // (every fourth) one per lane.
  p.epsplit = 64;
  p.nss = (p.lmax + p.epsplit - 1) / p.epsplit;
  p.hsplit = 512;
  p.nsh = (Th + p.hsplit - 1) / p.hsplit;
  p.off_scores = 0;
  p.off_list = align256(p.off_scores + (size_t)B * Hq * p.nblk * sizeof(double));
  p.off_mask = align256(p.off_list + units * p.lmax * sizeof(int32_t));
  p.off_count = align256(p.off_mask + units * p.lmax * sizeof(uint32_t));
  p.off_rec = align256(p.off_count + units * sizeof(int32_t));
  p.bytes = p.off_rec + units * (size_t)(p.nss + p.nsh) * G * (D + 2) * sizeof(float);
  return p;
}

}  // namespace

namespace hsk {

int int8_decode_validate(const void* q, const int8_t* k_codes, const float* k_scales, const int8_t* v_codes,
                         const float* v_scales, const void* k_hot, const void* v_hot, const void* out, int B,
                         int Hq, int Hkv, int D, int T8, int Th, float scale) {
  if (!q || !k_hot || !v_hot || !out) return HSK_ERR_NULL;
  if (T8 > 0 && (!k_codes || !k_scales || !v_codes || !v_scales)) return HSK_ERR_NULL;
  if (B <= 0 || T8 < 0 || T8 % 32 != 0 || Th <= 0) return HSK_ERR_SHAPE;
  if (int rc = check_heads(Hq, Hkv, D)) return rc;
  if (Hq / Hkv > 16) return HSK_ERR_UNSUPPORTED;
  if ((long long)T8 * D >= (1ll << 31)) return HSK_ERR_UNSUPPORTED;  // 32-bit code offsets per head
  if ((long long)T8 + 2ll * Th >= (1ll << 31)) return HSK_ERR_UNSUPPORTED;  // 32-bit split weights
  if (!std::isfinite(scale)) return HSK_ERR_SHAPE;
  if (!aligned16(q) || !aligned16(k_hot) || !aligned16(v_hot) || !aligned16(out)) return HSK_ERR_ALIGN;
  if (T8 > 0 && (!aligned16(k_codes) || !aligned16(v_codes) || !aligned4(k_scales) || !aligned4(v_scales)))
    return HSK_ERR_ALIGN;
  return HSK_OK;
}

}  // namespace hsk

extern "C" {

const char* hsk_strerror(int status) {
  switch (status) {
    case HSK_OK: return "ok";
    case HSK_ERR_NULL: return "a required pointer is NULL";
    case HSK_ERR_SHAPE: return "invalid or inconsistent sizes";
    case HSK_ERR_UNSUPPORTED: return "unsupported configuration (head_dim, group size, dtype or block)";
    case HSK_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case HSK_ERR_WORKSPACE: return "workspace missing or too small";
    case HSK_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

int hsk_abi_version(void) { return kAbiVersion; }

int swa_prefill(const void* q, const void* k, const void* v, void* out, int B, int L, int Hq, int Hkv,
                int D, int window, float scale, int dtype, void* ring_k, void* ring_v, int ring_w,
                void* stream) {
  if (!q || !k || !v || !out) return HSK_ERR_NULL;
  if ((ring_k == nullptr) != (ring_v == nullptr)) return HSK_ERR_NULL;
  if (B <= 0 || L <= 0) return HSK_ERR_SHAPE;
  if (int rc = check_heads(Hq, Hkv, D)) return rc;
  if (dtype != HSK_F32 && dtype != HSK_BF16) return HSK_ERR_UNSUPPORTED;
  if (!std::isfinite(scale) || scale <= 0.f) return HSK_ERR_SHAPE;
  if ((long long)L > (1ll << 30) || (long long)B * L * Hq > (1ll << 31) - 1) return HSK_ERR_SHAPE;
  // K/V tiles are fetched with 32-bit byte offsets from each sequence's start
  if (dtype == HSK_BF16 && (long long)L * Hkv * D * 2 >= (1ll << 32)) return HSK_ERR_UNSUPPORTED;
  // the fp32 path runs a 64-lane wave per (sequence, row, head): 64 B L Hq work-items < 2^32
  if (dtype == HSK_F32 && (long long)B * L * Hq > (1ll << 26)) return HSK_ERR_UNSUPPORTED;
  if (ring_k && ring_w <= 0) return HSK_ERR_SHAPE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return HSK_ERR_ALIGN;
  if (ring_k && (!aligned16(ring_k) || !aligned16(ring_v))) return HSK_ERR_ALIGN;
  hipStream_t s = (hipStream_t)stream;
  hsk::PrefillArgs a{};
  a.q = (const uint16_t*)q;
  a.k = (const uint16_t*)k;
  a.v = (const uint16_t*)v;
  a.o = (uint16_t*)out;
  a.B = B; a.L = L; a.Hq = Hq; a.Hkv = Hkv; a.D = D;
  a.window = (window <= 0 || window >= L) ? L + 256 : window;
  a.scale = scale;
  a.scale_log2 = log2e_times(scale);
  hipError_t e = dtype == HSK_BF16 ? hsk::launch_prefill_bf16(a, s) : hsk::launch_prefill_f32(a, s);
  if (e != hipSuccess) return HSK_ERR_HIP;
  if (ring_k) {
    hsk::RingCopyArgs r{};
    r.k = k; r.v = v; r.ring_k = ring_k; r.ring_v = ring_v;
    r.B = B; r.L = L; r.Hkv = Hkv; r.W = ring_w;
    r.row_bytes = D * (dtype == HSK_BF16 ? 2 : 4);
    e = hsk::launch_prefill_ring(r, s);
  }
  return finish(e);
}

int swa_prefill_chunk(const void* q, const void* k, const void* v, void* out, void* ring_k, void* ring_v, int B,
                      int C, int Hq, int Hkv, int D, int W, int pos0, float scale, void* stream) {
  if (!q || !k || !v || !out || !ring_k || !ring_v) return HSK_ERR_NULL;
  if (B <= 0 || C <= 0 || pos0 < 0) return HSK_ERR_SHAPE;
  if (int rc = check_heads(Hq, Hkv, D)) return rc;
  if (W < 64 || W > 65536 || W % 64 != 0 || pos0 % 64 != 0) return HSK_ERR_UNSUPPORTED;
  if (!std::isfinite(scale) || scale <= 0.f) return HSK_ERR_SHAPE;
  if ((long long)C > (1ll << 30) || (long long)B * C * Hq > (1ll << 31) - 1) return HSK_ERR_SHAPE;
  if ((long long)pos0 + C > (1ll << 30)) return HSK_ERR_SHAPE;
  if ((long long)C * Hkv * D * 2 >= (1ll << 32)) return HSK_ERR_UNSUPPORTED;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(ring_k) ||
      !aligned16(ring_v))
    return HSK_ERR_ALIGN;
  hipStream_t s = (hipStream_t)stream;
  hsk::PrefillArgs a{};
  a.q = (const uint16_t*)q;
  a.k = (const uint16_t*)k;
  a.v = (const uint16_t*)v;
  a.o = (uint16_t*)out;
  a.B = B; a.L = C; a.Hq = Hq; a.Hkv = Hkv; a.D = D;
  a.window = W;
  a.scale = scale;
  a.scale_log2 = log2e_times(scale);
  a.ring_k = (const uint16_t*)ring_k;
  a.ring_v = (const uint16_t*)ring_v;
  a.pos0 = pos0;
  hipError_t e = hsk::launch_prefill_bf16(a, s);
  if (e != hipSuccess) return HSK_ERR_HIP;
  // then (stream order: after every read of the old ring) the ring keeps the last W positions
  hsk::RingCopyArgs r{};
  r.k = k; r.v = v; r.ring_k = ring_k; r.ring_v = ring_v;
  r.B = B; r.L = C; r.Hkv = Hkv; r.W = W; r.row_bytes = D * 2; r.pos0 = pos0;
  return finish(hsk::launch_prefill_ring(r, s));
}

int swa_decode_ring(const void* q, const void* k_new, const void* v_new, void* ring_k, void* ring_v,
                    const int32_t* pos, void* out, int32_t* slot_out, int B, int Hq, int Hkv, int D,
                    int W, float scale, void* stream) {
  if (!q || !k_new || !v_new || !ring_k || !ring_v || !pos || !out) return HSK_ERR_NULL;
  if (B <= 0 || W <= 0 || W > 65536) return HSK_ERR_SHAPE;
  if (B > 65535) return HSK_ERR_UNSUPPORTED;  // the sequence index is the grid's y dimension
  if (int rc = check_heads(Hq, Hkv, D)) return rc;
  if (Hq / Hkv > 16 && (Hq / Hkv) % 16 != 0) return HSK_ERR_UNSUPPORTED;
  if (!std::isfinite(scale)) return HSK_ERR_SHAPE;
  if (!aligned16(q) || !aligned16(k_new) || !aligned16(v_new) || !aligned16(ring_k) ||
      !aligned16(ring_v) || !aligned16(out) || !aligned4(pos) || (slot_out && !aligned4(slot_out)))
    return HSK_ERR_ALIGN;
  hsk::RingDecodeArgs a{};
  a.q = (const uint16_t*)q;
  a.k_new = (const uint16_t*)k_new;
  a.v_new = (const uint16_t*)v_new;
  a.ring_k = (uint16_t*)ring_k;
  a.ring_v = (uint16_t*)ring_v;
  a.pos = pos;
  a.out = (uint16_t*)out;
  a.slot_out = slot_out;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.D = D; a.W = W;
  a.G = Hq / Hkv;
  a.scale_log2 = log2e_times(scale);
  return finish(hsk::launch_ring_decode(a, (hipStream_t)stream));
}

int kv_quant_int8_b32(const void* x, int8_t* codes, float* scales, int B, int Hkv, int T, int D,
                      void* stream) {
  if (!x || !codes || !scales) return HSK_ERR_NULL;
  if (B <= 0 || Hkv <= 0 || T < 0 || T % 32 != 0) return HSK_ERR_SHAPE;
  if (!head_dim_ok(D)) return HSK_ERR_UNSUPPORTED;
  if ((long long)B * Hkv * (T / 32) >= (1ll << 31)) return HSK_ERR_UNSUPPORTED;  // blocks index the grid
  if (!aligned16(x) || !aligned16(codes) || !aligned4(scales)) return HSK_ERR_ALIGN;
  if (T == 0) return HSK_OK;
  hsk::QuantArgs a{};
  a.x = (const uint16_t*)x;
  a.codes = codes;
  a.scales = scales;
  a.nblocks = (long)B * Hkv * (T / 32);
  a.D = D;
  return finish(hsk::launch_quant_b32(a, (hipStream_t)stream));
}

size_t attn_decode_int8kv_workspace_size(int B, int Hq, int Hkv, int D, int T8, int Th) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || D <= 0 || T8 < 0 || Th <= 0) return 0;
  if ((long long)T8 + 2ll * Th >= (1ll << 31)) return 0;
  return int8_ws_bytes(B, Hq, Hkv, D, T8, Th);
}

int attn_decode_int8kv(const void* q, const int8_t* k_codes, const float* k_scales, const int8_t* v_codes,
                       const float* v_scales, const void* k_hot, const void* v_hot, void* out, int B, int Hq,
                       int Hkv, int D, int T8, int Th, float scale, void* workspace, size_t workspace_bytes,
                       void* stream) {
  if (int rc = hsk::int8_decode_validate(q, k_codes, k_scales, v_codes, v_scales, k_hot, v_hot, out, B, Hq, Hkv,
                                         D, T8, Th, scale))
    return rc;
  const size_t need = int8_ws_bytes(B, Hq, Hkv, D, T8, Th);
  if (!workspace || workspace_bytes < need) return HSK_ERR_WORKSPACE;
  if (!aligned16(workspace)) return HSK_ERR_ALIGN;
  hsk::Int8DecodeArgs a{};
  a.q = (const uint16_t*)q;
  a.kc = k_codes; a.ks = k_scales; a.vc = v_codes; a.vs = v_scales;
  a.kh = (const uint16_t*)k_hot;
  a.vh = (const uint16_t*)v_hot;
  a.out = (uint16_t*)out;
  a.ws = (float*)workspace;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.D = D; a.T8 = T8; a.Th = Th;
  a.scale_log2 = log2e_times(scale);
  hsk::int8_decode_plan(B, Hkv, T8, Th, &a.nsplit, &a.wsplit);
  return finish(hsk::launch_int8_decode(a, (hipStream_t)stream));
}

size_t blocksparse_workspace_size(int L, int Hq, int Hkv, int D, int block, int topk) {
  (void)topk;
  if (L <= 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || block <= 0) return 0;
  return bs_ws_bytes(L, Hq, Hkv, D, block);
}

int blocksparse_select_attend(const void* q, const void* k, const void* v, void* out, int32_t* sel, int L,
                              int Hq, int Hkv, int D, int block, int topk, int window, float scale,
                              void* workspace, size_t workspace_bytes, void* stream) {
  if (!q || !k || !v || !out) return HSK_ERR_NULL;
  if (topk > 0 && !sel) return HSK_ERR_NULL;
  if (L <= 0 || window < 1 || topk < 0) return HSK_ERR_SHAPE;
  if (int rc = check_heads(Hq, Hkv, D)) return rc;
  if (block != 64 || topk > 256) return HSK_ERR_UNSUPPORTED;
  if (L % block != 0) return HSK_ERR_SHAPE;
  if (L / block > 4096 || (long long)L * Hkv * D * 2 >= (1ll << 32)) return HSK_ERR_UNSUPPORTED;
  if (!std::isfinite(scale) || scale <= 0.f) return HSK_ERR_SHAPE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || (sel && !aligned4(sel)))
    return HSK_ERR_ALIGN;
  const size_t need = bs_ws_bytes(L, Hq, Hkv, D, block);
  if (!workspace || workspace_bytes < need) return HSK_ERR_WORKSPACE;
  if (!aligned16(workspace)) return HSK_ERR_ALIGN;
  hsk::BlockSparseArgs a{};
  a.q = (const uint16_t*)q;
  a.k = (const uint16_t*)k;
  a.v = (const uint16_t*)v;
  a.out = (uint16_t*)out;
  a.sel = sel;
  a.L = L; a.Hq = Hq; a.Hkv = Hkv; a.D = D; a.block = block; a.topk = topk;
  a.window = window >= L ? L + 256 : window;
  a.nb = L / block;
  a.nbp = (a.nb + 63) / 64 * 64;
  a.qsum = (double*)workspace;
  a.ksum = a.qsum + (size_t)Hq * a.nbp * D;
  a.scores = a.ksum + (size_t)Hkv * a.nbp * D;
  a.scale_log2 = log2e_times(scale);
  return finish(hsk::launch_blocksparse(a, (hipStream_t)stream));
}

int swa_window_safe_len(const int32_t* slot_pos, const int32_t* match_len, int32_t* safe_len, int B, int W,
                        void* stream) {
  if (B < 0 || W < 1 || W > 65536) return HSK_ERR_SHAPE;
  if (B == 0) return HSK_OK;  // nothing is read or written
  if (!slot_pos || !match_len || !safe_len) return HSK_ERR_NULL;
  if (!aligned4(slot_pos) || !aligned4(match_len) || !aligned4(safe_len)) return HSK_ERR_ALIGN;
  hsk::WindowSafeArgs a{};
  a.slot_pos = slot_pos;
  a.match_len = match_len;
  a.safe_len = safe_len;
  a.B = B;
  a.W = W;
  return finish(hsk::launch_window_safe(a, (hipStream_t)stream));
}

int kv_block_means_int8(const int8_t* codes, const float* scales, float* means, int B, int Hkv, int T8, int D,
                        void* stream) {
  if (B <= 0 || Hkv <= 0 || T8 < 0 || T8 % 32 != 0) return HSK_ERR_SHAPE;
  if (!head_dim_ok(D)) return HSK_ERR_UNSUPPORTED;
  // one thread per (sequence, KV head, block, d): the grid counts them in 256s
  if ((long long)B * Hkv >= (1ll << 31) || (long long)B * Hkv * (T8 / 32) * D >= (1ll << 39))
    return HSK_ERR_UNSUPPORTED;
  if (T8 == 0) return HSK_OK;
  if (!codes || !scales || !means) return HSK_ERR_NULL;
  if (!aligned4(scales) || !aligned4(means)) return HSK_ERR_ALIGN;
  hsk::BlockMeansArgs a{};
  a.codes = codes; a.scales = scales; a.means = means;
  a.units = B * Hkv; a.T8 = T8; a.D = D;
  return finish(hsk::launch_block_means(a, (hipStream_t)stream));
}

size_t attn_decode_int8kv_sparse_workspace_size(int B, int Hq, int Hkv, int D, int T8, int Th, int topk) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || D <= 0 || T8 < 0 || Th <= 0 || topk < 0) return 0;
  return sparse_plan(B, Hq, Hkv, D, T8, Th, topk).bytes;
}

int attn_decode_int8kv_sparse(const void* q, const int8_t* k_codes, const float* k_scales, const int8_t* v_codes,
                              const float* v_scales, const float* k_means, const void* k_hot, const void* v_hot,
                              void* out, int32_t* sel, int B, int Hq, int Hkv, int D, int T8, int Th, int topk,
                              float scale, void* workspace, size_t workspace_bytes, void* stream) {
  if (!q || !k_hot || !v_hot || !out) return HSK_ERR_NULL;
  if (topk > 0 && !sel) return HSK_ERR_NULL;
  if (T8 > 0 && (!k_codes || !k_scales || !v_codes || !v_scales || !k_means)) return HSK_ERR_NULL;
  if (B <= 0 || T8 < 0 || T8 % 32 != 0 || Th <= 0 || topk < 0) return HSK_ERR_SHAPE;
  if (int rc = check_heads(Hq, Hkv, D)) return rc;
  if (Hq / Hkv > 16 || topk > 256 || T8 / 32 > 4096) return HSK_ERR_UNSUPPORTED;
  if ((long long)T8 * D >= (1ll << 31)) return HSK_ERR_UNSUPPORTED;
  if (!std::isfinite(scale)) return HSK_ERR_SHAPE;
  if (!aligned16(q) || !aligned16(k_hot) || !aligned16(v_hot) || !aligned16(out) || (sel && !aligned4(sel)))
    return HSK_ERR_ALIGN;
  if (T8 > 0 && (!aligned16(k_codes) || !aligned16(v_codes) || !aligned4(k_scales) || !aligned4(v_scales) ||
                 !aligned4(k_means)))
    return HSK_ERR_ALIGN;
  const SparsePlan p = sparse_plan(B, Hq, Hkv, D, T8, Th, topk);
  if (!workspace || workspace_bytes < p.bytes) return HSK_ERR_WORKSPACE;
  if (!aligned16(workspace)) return HSK_ERR_ALIGN;
  char* ws = (char*)workspace;
  hsk::SparseDecodeArgs a{};
  a.q = (const uint16_t*)q;
  a.kc = k_codes; a.ks = k_scales; a.vc = v_codes; a.vs = v_scales; a.means = k_means;
  a.kh = (const uint16_t*)k_hot; a.vh = (const uint16_t*)v_hot;
  a.out = (uint16_t*)out;
  a.sel = sel;
  a.scores = (double*)(ws + p.off_scores);
  a.ulist = (int32_t*)(ws + p.off_list);
  a.umask = (uint32_t*)(ws + p.off_mask);
  a.ucount = (int32_t*)(ws + p.off_count);
  a.ws = (float*)(ws + p.off_rec);
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.D = D; a.T8 = T8; a.Th = Th; a.topk = topk;
  a.nblk = p.nblk; a.lmax = p.lmax;
  a.epsplit = p.epsplit; a.nss = p.nss; a.hsplit = p.hsplit; a.nsh = p.nsh;
  a.scale_log2 = log2e_times(scale);
  hipStream_t s = (hipStream_t)stream;
  if (topk > 0) {
    const hipError_t e = hsk::launch_sparse_select(a, s);
    if (e != hipSuccess) return HSK_ERR_HIP;
  }
  return finish(hsk::launch_sparse_decode(a, s));
}

}  // extern "C"
