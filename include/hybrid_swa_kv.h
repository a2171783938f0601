/*
 * hybrid_swa_kv — C ABI of the MI355X (gfx950) hybrid long-context attention path.
 *
 * The operations follow three public pages:
 *   [K25-arch] "Kimi K2.5 model architecture deep-dive: industrial optimisation
 *              for ultra-long context" (framerc.cn)
 *   [MiMo-inf] IT之家 article on the Xiaomi MiMo-V2.5 inference system (hnjmgj.com)
 *   [S35-K25]  "2026 LLM architecture overview (III): Step 3.5 Flash & Kimi K2.5"
 *              (codearts.csdn.net)
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every tensor pointer is a DEVICE pointer owned by the caller, all on the
 *   current HIP device (hipSetDevice), to which `stream` must belong too: the
 *   kernels are launched there.  The library
 *   never allocates, frees or keeps device memory between calls, holds no global
 *   state, and is reentrant -- except attn_decode_int8kv_noalloc, which uses a
 *   static device array of its own (see there).  Work is enqueued on `stream` (a hipStream_t passed
 *   as void*; NULL = the null stream) and the call returns without waiting.
 * - Tensors are dense, row-major, contiguous; base pointers must be 16-byte
 *   aligned.  bf16 means IEEE bfloat16 bit patterns (uint16).
 * - Attention: query head h reads KV head h / (Hq / Hkv) (contiguous GQA groups);
 *   Hq % Hkv == 0 and Hq / Hkv <= 16.  head_dim D is 64 or 128.  Scores are
 *   scale * q.k; softmax and accumulation are fp32; outputs are rounded once
 *   (round-to-nearest-even) to the output dtype.
 * - Return value: HSK_OK (0) or an error code.  Argument errors (NULL pointers,
 *   bad shapes, misalignment, unsupported sizes, short workspace) are detected on
 *   the host before anything is enqueued; HSK_ERR_HIP reports a launch failure
 *   (hipGetLastError after the launch).  No C++ exception crosses the ABI.
 * - Values stored in device memory (e.g. `pos`) are preconditions the host does
 *   not read.
 */
#ifndef HYBRID_SWA_KV_H
#define HYBRID_SWA_KV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum hsk_status {
  HSK_OK = 0,
  HSK_ERR_NULL = 1,        /* a required pointer is NULL */
  HSK_ERR_SHAPE = 2,       /* a size is non-positive or sizes are inconsistent */
  HSK_ERR_UNSUPPORTED = 3, /* valid but not implemented (D, group size, dtype, block) */
  HSK_ERR_ALIGN = 4,       /* a pointer is not 16-byte aligned */
  HSK_ERR_WORKSPACE = 5,   /* workspace NULL or smaller than *_workspace_size() */
  HSK_ERR_HIP = 6          /* the HIP runtime reported an error */
};

enum hsk_dtype { HSK_F32 = 0, HSK_BF16 = 1 };

/* Human-readable text for a status code (static storage, never NULL). */
const char* hsk_strerror(int status);

/* ABI version: increases when a signature or a layout changes. */
int hsk_abi_version(void);

/*
 * swa_prefill — causal sliding-window or full causal GQA attention over a prompt.
 *
 * [MiMo-inf] section 1: 60 of 70 layers attend a 128-token sliding window, the
 * other 10 attend the full causal prefix; [K25-arch] section 2.2 "direction two":
 * a local window of 1024 tokens.  Key j is visible to query i iff
 * 0 <= i - j < window (the window counts the query itself); window <= 0 or
 * window >= L means full causal attention (j <= i).
 *
 * q   [B, L, Hq,  D]  dtype        (token-major)
 * k,v [B, L, Hkv, D]  dtype
 * out [B, L, Hq,  D]  dtype, written
 * dtype HSK_BF16 (MFMA path) or HSK_F32 (exact-fp32 path for small cases:
 * B * L * Hq <= 2^26, else HSK_ERR_UNSUPPORTED).
 * scale > 0 (the softmax scale, usually 1/sqrt(D)).
 * ring_k, ring_v: optional (both NULL or both set), [B, Hkv, ring_w, D] dtype.
 *   When set, the K/V of positions max(0, L - ring_w) .. L-1 are also copied to
 *   slot (position mod ring_w), the sliding-window pool of [MiMo-inf] section 2
 *   ("dual pools"); other slots are left untouched.
 */
int swa_prefill(const void* q, const void* k, const void* v, void* out,
                int B, int L, int Hq, int Hkv, int D, int window, float scale, int dtype,
                void* ring_k, void* ring_v, int ring_w, void* stream);

/*
 * swa_prefill_chunk — one chunk of a sliding-window prefill, continuing from a ring.
 *
 * [K25-arch] section 4.2 prefills long inputs in chunks (prefill_chunk_size
 * 4096); [MiMo-inf] section 2 keeps a sliding-window layer's KV in a W-slot
 * ring (slot = position mod W).  The chunk holds positions pos0 .. pos0+C-1 of
 * every sequence; query i attends positions max(0, i-W+1) .. i; positions below
 * pos0 are read from the ring, which on entry holds positions max(0, pos0-W) ..
 * pos0-1 at slot position mod W.  On return the ring holds positions
 * max(0, pos0+C-W) .. pos0+C-1 (the chunk's rows written after its attention,
 * in stream order).  bf16 only.
 *
 * q, out       [B, C, Hq, D] bf16 (token-major, as in swa_prefill)
 * k, v         [B, C, Hkv, D] bf16, the chunk's own K/V
 * ring_k/v     [B, Hkv, W, D] bf16, read and updated in place
 * pos0         position of the chunk's first row; W the window and ring size
 * Limits: pos0 and W multiples of 64, 64 <= W <= 65536, else HSK_ERR_UNSUPPORTED;
 * scale > 0 and finite; pointers 16-byte aligned.
 */
int swa_prefill_chunk(const void* q, const void* k, const void* v, void* out,
                      void* ring_k, void* ring_v,
                      int B, int C, int Hq, int Hkv, int D, int W, int pos0, float scale,
                      void* stream);

/*
 * swa_decode_ring — one decode token per sequence against a sliding-window ring.
 *
 * [MiMo-inf] section 2 ("dual pools"): the SWA pool holds exactly W tokens per
 * sequence in a ring buffer; the full-attention index maps positions to slots.
 * Here slot = position mod W.  For each sequence b with p = pos[b] >= 0:
 *   1. ring_k/ring_v[b, :, p mod W, :] <- k_new/v_new[b]   (every other slot kept)
 *   2. slot_out[b] <- p mod W                               (if slot_out != NULL)
 *   3. out[b, h] = attention of q[b, h] over positions max(0, p-W+1) .. p, i.e.
 *      the W most recent tokens including the new one; slot s holds position
 *      p - ((p - s) mod W), and slots whose position would be negative are not
 *      attended.  The new token's K/V is taken from k_new/v_new.
 * A sequence with pos[b] < 0 has no token to decode and is skipped: its ring
 * rows and slot_out[b] keep their contents and out[b] is all zero.
 *
 * q           [B, Hq,  D]     bf16
 * k_new,v_new [B, Hkv, D]     bf16
 * ring_k,v    [B, Hkv, W, D]  bf16, updated in place
 * pos         [B] int32 (device), out [B, Hq, D] bf16, slot_out [B] int32 or NULL.
 * W in [1, 65536]; B <= 65535, else HSK_ERR_UNSUPPORTED.  Here Hq / Hkv may
 * exceed 16 when it is a multiple of 16.
 */
int swa_decode_ring(const void* q, const void* k_new, const void* v_new,
                    void* ring_k, void* ring_v, const int32_t* pos,
                    void* out, int32_t* slot_out,
                    int B, int Hq, int Hkv, int D, int W, float scale, void* stream);

/*
 * kv_quant_int8_b32 — INT8 block-wise encoding of a KV region.
 *
 * [K25-arch] section 2.2 "direction one" (warm region stored as INT8 with
 * block-wise quantisation) and section 2.3 (one scale per 32 tokens).  For every
 * (b, head, 32-token block n), over the 32 x D values X of that block:
 *   a = max |X|;  a == 0 -> scale 0, codes 0;
 *   else scale = fl32(a / 127) (correctly rounded),
 *        code  = clamp(rint(fl32(x / scale)), -127, 127), rint = half to even.
 * Call once for K and once for V.
 *
 * x      [B, Hkv, T, D] bf16          (T % 32 == 0)
 * codes  [B, Hkv, T, D] int8, written
 * scales [B, Hkv, T/32] fp32, written
 * Limits: B * Hkv * T / 32 < 2^31 blocks, else HSK_ERR_UNSUPPORTED; T == 0 is a
 * no-op.
 */
int kv_quant_int8_b32(const void* x, int8_t* codes, float* scales,
                      int B, int Hkv, int T, int D, void* stream);

/*
 * attn_decode_int8kv — full-attention decode over an INT8 region plus a bf16 tail.
 *
 * [K25-arch] section 2.2 "direction one": the newest tokens are kept as
 * full-precision KV (the hot zone, 2048 tokens in section 4.2), older ones as
 * INT8 with one scale per 32 tokens.  Positions 0 .. T8-1 are the dequantised
 * values code * scale, positions T8 .. T8+Th-1 the bf16 rows.  The query is
 * the token at position T8+Th-1 (its own K/V is the last hot row), so every
 * cached position is visible.  Split along the keys; partial (max, sum, acc)
 * records go to `workspace` and are merged in a fixed order (deterministic).
 *
 * q                [B, Hq, D] bf16
 * k_codes, v_codes [B, Hkv, T8, D] int8     (T8 % 32 == 0, T8 >= 0)
 * k_scales,v_scales[B, Hkv, T8/32] fp32     (may be NULL when T8 == 0)
 * k_hot, v_hot     [B, Hkv, Th, D] bf16     (Th >= 1)
 * out              [B, Hq, D] bf16, written
 * workspace        device scratch of attn_decode_int8kv_workspace_size(...) bytes
 * Limits: Hq / Hkv <= 16, T8 * D < 2^31 and T8 + 2 Th < 2^31 per (sequence,
 * KV head), else HSK_ERR_UNSUPPORTED (the workspace size query returns 0).
 */
int attn_decode_int8kv(const void* q,
                       const int8_t* k_codes, const float* k_scales,
                       const int8_t* v_codes, const float* v_scales,
                       const void* k_hot, const void* v_hot, void* out,
                       int B, int Hq, int Hkv, int D, int T8, int Th, float scale,
                       void* workspace, size_t workspace_bytes, void* stream);

size_t attn_decode_int8kv_workspace_size(int B, int Hq, int Hkv, int D, int T8, int Th);

/*
 * attn_decode_int8kv_noalloc — attn_decode_int8kv with no workspace argument.
 *
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc).  Same
 * arguments, semantics, kernels and results as attn_decode_int8kv, bit for bit;
 * the split records go to a static device array of
 * ATTN_DECODE_INT8KV_NOALLOC_MAX_WORKSPACE bytes inside the library (one per
 * GPU, held until the process ends) instead of a caller workspace.
 * Nothing is allocated and nothing must be cleared between calls.
 * Every call on one GPU shares that GPU's array: calls that overlap on one GPU
 * (on different streams or from different host threads) race and must not be
 * issued; calls ordered on one stream are fine.
 * Errors: as attn_decode_int8kv; HSK_ERR_WORKSPACE when
 * attn_decode_int8kv_workspace_size(...) exceeds the array (B * Hkv units of
 * Hq / Hkv heads and about 2048 / (B * Hkv) splits, (D + 2) floats per split and
 * head: e.g. 4.3 MB for B 16, 32/8 heads, D 128), checked before any HIP call;
 * HSK_ERR_HIP when the array's device address cannot be obtained.
 */
#define ATTN_DECODE_INT8KV_NOALLOC_MAX_WORKSPACE ((size_t)32 << 20)

int attn_decode_int8kv_noalloc(const void* q,
                               const int8_t* k_codes, const float* k_scales,
                               const int8_t* v_codes, const float* v_scales,
                               const void* k_hot, const void* v_hot, void* out,
                               int B, int Hq, int Hkv, int D, int T8, int Th, float scale,
                               void* stream);

/*
 * kv_block_means_int8 — the K block means stored with the INT8 blocks.
 *
 * For the block-sparse decode below ([K25-arch] section 2.2: a query keeps its
 * top-64 long-range keys; section 2.3: 32-token INT8 blocks): per (sequence,
 * KV head, 32-token block) and d, mean = fl32(fl32(sum of the 32 codes) * scale)
 * / 32 -- the code sum is an exact integer, so one fp32 rounding; the division
 * by 32 is exact (bit-exact output).
 *
 * codes  [B, Hkv, T8, D] int8;  scales [B, Hkv, T8/32] fp32
 * means  [B, Hkv, D, T8/32] fp32, written (d-major)
 * Errors: HSK_ERR_SHAPE unless B, Hkv > 0 and T8 % 32 == 0; HSK_ERR_UNSUPPORTED
 * for D other than 64 or 128, or B * Hkv * (T8/32) * D >= 2^39; T8 == 0 is then
 * a no-op (the pointers may be NULL); else HSK_ERR_NULL for a NULL pointer and
 * HSK_ERR_ALIGN for scales or means not 4-byte aligned.
 */
int kv_block_means_int8(const int8_t* codes, const float* scales, float* means,
                        int B, int Hkv, int T8, int D, void* stream);

/*
 * attn_decode_int8kv_sparse — top-k block-sparse decode over the hot + INT8 pool.
 *
 * [K25-arch] section 2.2 joins the hot/warm KV ("direction one") with a local
 * window plus top-64 long-range attention ("direction two").  Here the local
 * window is the bf16 hot tail (always attended) and the long-range candidates
 * are the 32-token INT8 blocks: per query head, score(j) = q . mean_j in fp64
 * (means from kv_block_means_int8); the topk highest are kept, ties to the lower
 * block, all blocks when there are at most topk.  The query (position T8+Th-1)
 * attends the hot tail and the tokens of its kept blocks.
 *
 * q [B, Hq, D] bf16; codes/scales as attn_decode_int8kv; k_means [B, Hkv, D, T8/32]
 * fp32; k_hot, v_hot [B, Hkv, Th, D] bf16; out [B, Hq, D] bf16, written;
 * sel [B, Hq, topk] int32, written: kept blocks ascending, -1 padded (bit-exact
 * up to fp64 near-ties).  workspace: attn_decode_int8kv_sparse_workspace_size(...).
 * Limits: Hq / Hkv <= 16, topk <= 256, T8 / 32 <= 4096, T8 * D < 2^31.
 */
int attn_decode_int8kv_sparse(const void* q,
                              const int8_t* k_codes, const float* k_scales,
                              const int8_t* v_codes, const float* v_scales,
                              const float* k_means, const void* k_hot, const void* v_hot,
                              void* out, int32_t* sel,
                              int B, int Hq, int Hkv, int D, int T8, int Th, int topk, float scale,
                              void* workspace, size_t workspace_bytes, void* stream);

size_t attn_decode_int8kv_sparse_workspace_size(int B, int Hq, int Hkv, int D, int T8, int Th, int topk);

/*
 * blocksparse_select_attend — top-k block-sparse causal attention.
 *
 * [K25-arch] section 2.2 "direction two": a local sliding window plus sparse
 * long-range attention to the top-64 most relevant keys (section 2.3).  Here the
 * sparse part works on whole key blocks of `block` tokens:
 *   1. per query head h and query block qb, per KV head g and key block kb:
 *      sums of Q and K over the block, in fp64;
 *   2. score(h, qb, kb) = (sumQ/block) . (sumK/block), fp64, for kb < qb only;
 *   3. S(h, qb) = the `topk` highest scores, ties to the lower kb; every earlier
 *      block when qb <= topk;
 *   4. key j is visible to query i iff 0 <= i - j < window, or j's block is in
 *      S(h, i / block).
 * sel receives S ascending, padded with -1 (bit-exact integer output).
 *
 * q   [L, Hq,  D] bf16;  k, v [L, Hkv, D] bf16;  out [L, Hq, D] bf16, written
 * sel [Hq, L/block, topk] int32, written
 * block == 64;  L % block == 0;  0 <= topk <= 256;  window >= 1;  scale > 0.
 * workspace: blocksparse_workspace_size(...) bytes: fp64 block sums of Q and K
 * and the per-head triangle of block scores (Hq * nb * (nb - 1) / 2 doubles,
 * about 0.5 GB at L = 131072, Hq = 32).
 */
int blocksparse_select_attend(const void* q, const void* k, const void* v, void* out,
                              int32_t* sel, int L, int Hq, int Hkv, int D,
                              int block, int topk, int window, float scale,
                              void* workspace, size_t workspace_bytes, void* stream);

size_t blocksparse_workspace_size(int L, int Hq, int Hkv, int D, int block, int topk);

/*
 * swa_window_safe_len — longest reusable prefix whose sliding-window KV survives.
 *
 * [MiMo-inf] section 2, prefix cache: under sliding-window layers a token-level
 * prefix match does not mean the KV is still there; the match is cut to the
 * "window-safe length", whose last W tokens still have valid SWA slots.  Here a
 * prefix of length l needs positions max(0, l - W) .. l - 1, and position p is
 * present when slot p mod W holds p.  safe_len[b] is the largest l <= match_len[b]
 * whose needed positions are all present (0 if none; match_len < 0 counts as 0).
 *
 * slot_pos   [B, W] int32: the position each SWA slot holds, -1 for an empty slot
 * match_len  [B] int32: the token-level prefix match length
 * safe_len   [B] int32, written (bit-exact integer output)
 * Errors: HSK_ERR_SHAPE unless 0 <= B and 1 <= W <= 65536; B == 0 is a no-op
 * (pointers may then be NULL); otherwise pointers non-NULL and 4-byte aligned.
 */
int swa_window_safe_len(const int32_t* slot_pos, const int32_t* match_len, int32_t* safe_len,
                        int B, int W, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* HYBRID_SWA_KV_H */
