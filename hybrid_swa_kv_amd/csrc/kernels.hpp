// Host-side launch interface between the C ABI (abi.cpp) and the kernels.
// Every launcher assumes its arguments were validated by the ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace hsk {

struct PrefillArgs {
  const uint16_t* q;  // bf16 bits, or fp32 reinterpreted, [B, L, Hq, D]
  const uint16_t* k;  // [B, L, Hkv, D]
  const uint16_t* v;
  uint16_t* o;
  int B, L, Hq, Hkv, D;
  int window;        // effective window, >= 1 (full causal passed as L + 1 or more)
  float scale;       // softmax scale
  float scale_log2;  // scale * log2(e)
  int nqb, total;    // filled by the launcher
  // chunk mode (ring_k != nullptr): the L rows are positions pos0 .. pos0+L-1 and
  // positions before pos0 are read from the ring [B, Hkv, window, D] at slot
  // position mod window (pos0 and window multiples of 64)
  const uint16_t* ring_k;
  const uint16_t* ring_v;
  int pos0;
};

struct RingCopyArgs {
  const void* k;  // [B, L, Hkv, D]
  const void* v;
  void* ring_k;   // [B, Hkv, W, D]
  void* ring_v;
  int B, L, Hkv, W, row_bytes;
  int pos0;       // absolute position of row 0 of k / v
};

struct RingDecodeArgs {
  const uint16_t* q;      // [B, Hq, D]
  const uint16_t* k_new;  // [B, Hkv, D]
  const uint16_t* v_new;
  uint16_t* ring_k;       // [B, Hkv, W, D]
  uint16_t* ring_v;
  const int32_t* pos;     // [B]
  uint16_t* out;          // [B, Hq, D]
  int32_t* slot_out;      // [B] or null
  int B, Hq, Hkv, D, W;
  int G;                  // Hq / Hkv
  float scale_log2;
};

struct QuantArgs {
  const uint16_t* x;  // [B, Hkv, T, D]
  int8_t* codes;      // [B, Hkv, T, D]
  float* scales;      // [B, Hkv, T/32]
  long nblocks;       // B * Hkv * T / 32
  int D;
};

struct Int8DecodeArgs {
  const uint16_t* q;  // [B, Hq, D]
  const int8_t* kc;   // [B, Hkv, T8, D]
  const float* ks;    // [B, Hkv, T8/32]
  const int8_t* vc;
  const float* vs;
  const uint16_t* kh;  // [B, Hkv, Th, D]
  const uint16_t* vh;
  uint16_t* out;       // [B, Hq, D]
  float* ws;           // partials [B*Hkv][nsplit][G][D + 2]
  int B, Hq, Hkv, D, T8, Th;
  float scale_log2;
  // Split plan: an INT8 token weighs 1 (its 256 bytes of K and V codes) and a
  // hot token 2; split s covers weights [s wsplit, (s+1) wsplit) of the order
  // INT8 tokens 0 .. T8-1, then hot tokens 0 .. Th-1.
  int nsplit, wsplit;
};

struct BlockSparseArgs {
  const uint16_t* q;  // [L, Hq, D]
  const uint16_t* k;  // [L, Hkv, D]
  const uint16_t* v;
  uint16_t* out;      // [L, Hq, D]
  int32_t* sel;       // [Hq, nb, topk]
  double* qsum;       // [Hq, nbp, D] block sums of Q (blocks past nb unused)
  double* ksum;       // [Hkv, nbp, D] block sums of K
  double* scores;     // [Hq][nb (nb - 1) / 2] packed lower triangle of sumQ . sumK
  int L, Hq, Hkv, D, block, topk, window, nb;
  int nbp;            // nb rounded up to a multiple of 64
  float scale_log2;
};

struct WindowSafeArgs {
  const int32_t* slot_pos;   // [B, W] position held by each SWA slot, -1 empty
  const int32_t* match_len;  // [B]
  int32_t* safe_len;         // [B]
  int B, W;
};

struct BlockMeansArgs {
  const int8_t* codes;  // [B, Hkv, T8, D]
  const float* scales;  // [B, Hkv, T8/32]
  float* means;         // [B, Hkv, D, T8/32] (d-major)
  int units, T8, D;     // units = B * Hkv
};

// Block-sparse decode over the hot + INT8 pool.  Per (sequence, KV head) unit the
// selection writes the union of the group's kept blocks, ascending, with a bit
// per head that kept each block.
struct SparseDecodeArgs {
  const uint16_t* q;     // [B, Hq, D]
  const int8_t* kc;      // [B, Hkv, T8, D]
  const float* ks;       // [B, Hkv, T8/32]
  const int8_t* vc;
  const float* vs;
  const float* means;    // [B, Hkv, D, T8/32] K block means
  const uint16_t* kh;    // [B, Hkv, Th, D]
  const uint16_t* vh;
  uint16_t* out;         // [B, Hq, D]
  int32_t* sel;          // [B, Hq, topk]
  int32_t* ulist;        // [units, lmax] kept blocks of the group, ascending
  uint32_t* umask;       // [units, lmax] bit per head of the group
  int32_t* ucount;       // [units]
  double* scores;        // [B, Hq, nblk] block scores
  float* ws;             // split records, as the dense decode
  int B, Hq, Hkv, D, T8, Th, topk, nblk, lmax;
  int epsplit, nss;      // union entries per sparse split, sparse splits per unit
  int hsplit, nsh;       // hot tokens per hot split, hot splits per unit
  float scale_log2;
};

// Host-side argument checks of attn_decode_int8kv, everything but the workspace
// (an HSK_* status; no HIP call).
int int8_decode_validate(const void* q, const int8_t* k_codes, const float* k_scales, const int8_t* v_codes,
                         const float* v_scales, const void* k_hot, const void* v_hot, const void* out, int B,
                         int Hq, int Hkv, int D, int T8, int Th, float scale);

hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t s);
hipError_t launch_prefill_f32(const PrefillArgs& a, hipStream_t s);
hipError_t launch_prefill_ring(const RingCopyArgs& a, hipStream_t s);
hipError_t launch_ring_decode(const RingDecodeArgs& a, hipStream_t s);
hipError_t launch_quant_b32(const QuantArgs& a, hipStream_t s);
void int8_decode_plan(int B, int Hkv, int T8, int Th, int* nsplit, int* wsplit);
hipError_t launch_int8_decode(const Int8DecodeArgs& a, hipStream_t s);
hipError_t launch_blocksparse(const BlockSparseArgs& a, hipStream_t s);
hipError_t launch_window_safe(const WindowSafeArgs& a, hipStream_t s);
hipError_t launch_block_means(const BlockMeansArgs& a, hipStream_t s);
hipError_t launch_sparse_select(const SparseDecodeArgs& a, hipStream_t s);  // scores, then selection
hipError_t launch_sparse_decode(const SparseDecodeArgs& a, hipStream_t s);

}  // namespace hsk
