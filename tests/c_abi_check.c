/*
 * C99 consumer of include/packed_bit_gemv.h, linked against the built
 * library: the boundary is usable from plain C. Every entry-point call below
 * is invalid on purpose (null pointer, bad shape or misalignment), so the
 * library returns from its argument checks before any HIP call and nothing
 * needs a GPU. Prints "ok" and exits 0 when every return value is the
 * documented one.
 */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "packed_bit_gemv.h"

static int failures = 0;

static void expect(const char* what, long long got, long long want) {
  if (got != want) {
    printf("FAIL %s: got %lld, want %lld\n", what, got, want);
    ++failures;
  }
}

int main(void) {
  /* fake 256-byte-aligned addresses: only ever passed with an invalid argument */
  const uintptr_t base = (uintptr_t)1 << 20;
  const uint32_t* packed = (const uint32_t*)base;
  const int8_t* w = (const int8_t*)base;
  const float* scale = (const float*)(base + 0x1000);
  const uint16_t* x = (const uint16_t*)(base + 0x2000);
  float* y = (float*)(base + 0x3000);
  uint16_t* h = (uint16_t*)(base + 0x4000);
  uint64_t* keys = (uint64_t*)(base + 0x5000);
  int32_t* token = (int32_t*)(base + 0x6000);
  const int32_t* tokens = (const int32_t*)(base + 0x7000);

  expect("abi version", pbg_abi_version(), PBG_ABI_VERSION);
  expect("words_per_row(1)", pbg_words_per_row(1), 4);
  expect("words_per_row(64)", pbg_words_per_row(64), 4);
  expect("words_per_row(65)", pbg_words_per_row(65), 8);
  expect("words_per_row(4096)", pbg_words_per_row(4096), 256);
  expect("words_per_row(0)", pbg_words_per_row(0), 0);
  expect("strerror(ok) non-empty", pbg_strerror(PBG_OK) != NULL && strlen(pbg_strerror(PBG_OK)) > 0, 1);
  expect("strerror(unknown) non-null", pbg_strerror(12345) != NULL, 1);

  expect("gemv null", ternary_gemv(NULL, scale, 8, 64, x, y, 0), PBG_ERR_NULL);
  expect("gemv n = 0", ternary_gemv(packed, scale, 0, 64, x, y, 0), PBG_ERR_SHAPE);
  expect("gemv k too large", ternary_gemv(packed, scale, 8, PBG_MAX_K + 1, x, y, 0), PBG_ERR_SHAPE);
  expect("gemv packed misaligned", ternary_gemv((const uint32_t*)(base + 4), scale, 8, 64, x, y, 0), PBG_ERR_ALIGN);
  expect("small m = 0", ternary_gemm_small(packed, scale, 8, 64, x, 0, y, 0), PBG_ERR_SHAPE);
  expect("small m = 9", ternary_gemm_small(packed, scale, 8, 64, x, PBG_MAX_M + 1, y, 0), PBG_ERR_SHAPE);
  expect("splitk workspace bytes", pbg_splitk_workspace_bytes(4096, 12288), 8 * 8 * (4096 + 64));
  expect("splitk null workspace", ternary_gemm_splitk(packed, scale, 8, 64, x, 1, y, NULL, 1 << 20, 0), PBG_ERR_NULL);
  expect("splitk workspace misaligned",
         ternary_gemm_splitk(packed, scale, 8, 64, x, 1, y, (void*)(base + 0x9010), 1 << 20, 0), PBG_ERR_ALIGN);
  expect("splitk workspace too small",
         ternary_gemm_splitk(packed, scale, 4096, 12288, x, 8, y, (void*)(base + 0x9000), 1024, 0),
         PBG_ERR_WORKSPACE);
  expect("words_per_row3(4096)", pbg_words_per_row3(4096), 384);
  expect("pack3 null codes", pack_ternary3(NULL, 8, 64, (uint32_t*)base, (int32_t*)(base + 0x1000),
                                            (int64_t*)(base + 0x2000), NULL, 0), PBG_ERR_NULL);
  expect("gemv3 k = 0", ternary3_gemv(packed, scale, 8, 0, x, y, 0), PBG_ERR_SHAPE);
  expect("gemm3 small m = 9", ternary3_gemm_small(packed, scale, 8, 64, x, PBG_MAX_M + 1, y, 0), PBG_ERR_SHAPE);
  expect("head null y", int8_head_gemv(w, scale, 8, 64, x, 1, NULL, 0), PBG_ERR_NULL);
  expect("head w misaligned", int8_head_gemv(w + 8, scale, 8, 64, x, 1, y, 0), PBG_ERR_ALIGN);
  expect("argmax keys misaligned", int8_head_argmax(w, scale, 8, 64, x, 1, (uint64_t*)(base + 0x5004), token,
                                                    y, 0), PBG_ERR_ALIGN);
  expect("argmax null token", int8_head_argmax(w, scale, 8, 64, x, 1, keys, NULL, y, 0), PBG_ERR_NULL);
  expect("argmax noalloc m = 9", int8_head_argmax_noalloc(w, scale, 8, 64, x, PBG_MAX_M + 1, token, y, 0),
         PBG_ERR_SHAPE);
  expect("argmax noalloc null w", int8_head_argmax_noalloc(NULL, scale, 8, 64, x, 1, token, y, 0), PBG_ERR_NULL);
  expect("argmax noalloc scratch size", PBG_NOALLOC_SCRATCH_BYTES, 262144);
  expect("embedding m = 0", int8_embedding_gather(w, scale, 8, 64, tokens, 0, y, 0), PBG_ERR_SHAPE);
  expect("pack null codes", pack_ternary(NULL, 8, 64, (uint32_t*)base, (int32_t*)(base + 0x1000), NULL, NULL, 0),
         PBG_ERR_NULL);
  expect("gate_up d_model not multiple of 8",
         ternary_swiglu_gate_up(packed, scale, packed, scale, 100, 64, x, h, 0), PBG_ERR_SHAPE);
  expect("ffn d_model too large",
         ternary_ffn_swiglu(packed, scale, packed, scale, packed, scale, PBG_FFN_MAX_MODEL + 8, 64, x, h, y, 0),
         PBG_ERR_SHAPE);
  expect("gate_up small m = 9",
         ternary_swiglu_gate_up_small(packed, scale, packed, scale, 4096, 64, x, PBG_MAX_M + 1, h, 0), PBG_ERR_SHAPE);
  expect("ffn small null y",
         ternary_ffn_swiglu_small(packed, scale, packed, scale, packed, scale, 4096, 64, x, 4, h, NULL, 0),
         PBG_ERR_NULL);
  expect("3-bit gate_up d_model not multiple of 8",
         ternary3_swiglu_gate_up(packed, scale, packed, scale, 100, 64, x, h, 0), PBG_ERR_SHAPE);
  expect("3-bit ffn d_model too large",
         ternary3_ffn_swiglu(packed, scale, packed, scale, packed, scale, PBG_FFN_MAX_MODEL + 8, 64, x, h, y, 0),
         PBG_ERR_SHAPE);
  expect("3-bit gate_up small m = 0",
         ternary3_swiglu_gate_up_small(packed, scale, packed, scale, 4096, 64, x, 0, h, 0), PBG_ERR_SHAPE);
  expect("3-bit ffn small null down",
         ternary3_ffn_swiglu_small(packed, scale, packed, scale, NULL, scale, 4096, 64, x, 4, h, y, 0), PBG_ERR_NULL);
  expect("stream read bytes not a multiple of 16", pbg_stream_read(w, 1000, (uint32_t*)(base + 0x8000), 0),
         PBG_ERR_SHAPE);
  expect("stream read src misaligned", pbg_stream_read(w + 8, 1024, (uint32_t*)(base + 0x8000), 0), PBG_ERR_ALIGN);
  if (failures == 0) printf("ok\n");
  return failures == 0 ? 0 : 1;
}
