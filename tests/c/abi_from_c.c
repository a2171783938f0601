/* Calls the library from plain C through include/hybrid_swa_kv.h: the ABI
 * version, the status strings and host-side argument checks (every call below
 * is rejected before any device work, so no GPU is needed).  Prints "ok" and
 * exits 0 when every check holds. */
#include <stdio.h>
#include <string.h>

#include "hybrid_swa_kv.h"

static int failures = 0;

static void expect(const char* what, int got, int want) {
  if (got != want) {
    printf("FAIL %s: got %d (%s), want %d\n", what, got, hsk_strerror(got), want);
    ++failures;
  }
}

int main(void) {
  /* a fake 16-byte-aligned "device pointer" and a misaligned one (never dereferenced) */
  void* p = (void*)(uintptr_t)4096;
  void* mis = (void*)(uintptr_t)4100;
  const int32_t* pos = (const int32_t*)p;
  size_t need;

  if (hsk_abi_version() < 1) { printf("FAIL abi version\n"); ++failures; }
  if (strcmp(hsk_strerror(HSK_OK), "ok") != 0 || hsk_strerror(12345) == NULL) {
    printf("FAIL strerror\n");
    ++failures;
  }

  expect("prefill NULL q", swa_prefill(NULL, p, p, p, 1, 8, 2, 2, 128, 0, 1.0f, HSK_BF16, NULL, NULL, 0, NULL),
         HSK_ERR_NULL);
  expect("prefill D 96", swa_prefill(p, p, p, p, 1, 8, 2, 2, 96, 0, 1.0f, HSK_BF16, NULL, NULL, 0, NULL),
         HSK_ERR_UNSUPPORTED);
  expect("prefill misaligned", swa_prefill(p, mis, p, p, 1, 8, 2, 2, 128, 0, 1.0f, HSK_BF16, NULL, NULL, 0, NULL),
         HSK_ERR_ALIGN);
  expect("chunk W 100", swa_prefill_chunk(p, p, p, p, p, p, 1, 64, 8, 2, 128, 100, 0, 1.0f, NULL),
         HSK_ERR_UNSUPPORTED);
  expect("ring W 0", swa_decode_ring(p, p, p, p, p, pos, p, NULL, 2, 8, 2, 128, 0, 1.0f, NULL), HSK_ERR_SHAPE);
  expect("quant T 33", kv_quant_int8_b32(p, (int8_t*)p, (float*)p, 1, 1, 33, 128, NULL), HSK_ERR_SHAPE);
  expect("quant empty", kv_quant_int8_b32(p, (int8_t*)p, (float*)p, 1, 1, 0, 128, NULL), HSK_OK);

  need = attn_decode_int8kv_workspace_size(16, 32, 8, 128, 63488, 2048);
  if (need == 0) { printf("FAIL workspace size\n"); ++failures; }
  expect("int8 short workspace",
         attn_decode_int8kv(p, (const int8_t*)p, (const float*)p, (const int8_t*)p, (const float*)p, p, p, p, 16, 32,
                            8, 128, 63488, 2048, 1.0f, p, need - 1, NULL),
         HSK_ERR_WORKSPACE);
  expect("noalloc group 17",
         attn_decode_int8kv_noalloc(p, (const int8_t*)p, (const float*)p, (const int8_t*)p, (const float*)p, p, p, p,
                                    1, 34, 2, 128, 64, 8, 1.0f, NULL),
         HSK_ERR_UNSUPPORTED);
  expect("blocksparse block 32",
         blocksparse_select_attend(p, p, p, p, (int32_t*)p, 4096, 8, 2, 128, 32, 16, 512, 1.0f, p, 1u << 30, NULL),
         HSK_ERR_UNSUPPORTED);
  expect("window safe W 0", swa_window_safe_len(pos, pos, (int32_t*)p, 1, 0, NULL), HSK_ERR_SHAPE);
  expect("means T8 48", kv_block_means_int8((const int8_t*)p, (const float*)p, (float*)p, 2, 2, 48, 128, NULL),
         HSK_ERR_SHAPE);
  expect("sparse topk 300",
         attn_decode_int8kv_sparse(p, (const int8_t*)p, (const float*)p, (const int8_t*)p, (const float*)p,
                                   (const float*)p, p, p, p, (int32_t*)p, 2, 8, 2, 128, 64, 16, 300, 1.0f, p, 1u << 20,
                                   NULL),
         HSK_ERR_UNSUPPORTED);

  if (failures) return 1;
  printf("ok\n");
  return 0;
}
