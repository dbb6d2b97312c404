/*
 * Host-side argument checks of every libmoesq entry point, for a build of
 * the library's host code with AddressSanitizer and UndefinedBehavior-
 * Sanitizer (tests/test_host_sanitizers.py builds and runs it on the CPU).
 * Every call here is rejected, or is a no-op, before any HIP call, so the
 * program needs no GPU.  It exits 0 when every status matches; a sanitizer
 * finding aborts it.
 */
#include <stdio.h>
#include <string.h>

#include "moesq.h"

static int failures = 0;

static void expect(const char *what, moesq_status_t got, moesq_status_t want) {
  const char *detail = moesq_last_error();
  if (got != want) {
    printf("FAIL %s: status %d, expected %d (%s)\n", what, (int)got, (int)want, detail);
    ++failures;
  } else if (want != MOESQ_OK && (!detail || !detail[0])) {
    printf("FAIL %s: error without a detail string\n", what);
    ++failures;
  }
}

#define P(x) ((void *)(uintptr_t)(x))

static moesq_weights_t weights(int32_t E, int32_t N, int32_t K, int32_t layout, int null_bufs) {
  moesq_weights_t w;
  memset(&w, 0, sizeof w);
  const uint8_t *b = null_bufs ? NULL : (const uint8_t *)P(0x1000);
  w.values = b;
  w.masks = b;
  w.scales = b;
  w.global_scale = null_bufs ? NULL : (const float *)P(0x1000);
  w.E = E;
  w.N = N;
  w.K = K;
  w.layout = layout;
  return w;
}

int main(void) {
  int32_t *ip = (int32_t *)P(0x10);
  uint16_t *hp = (uint16_t *)P(0x10);
  uint8_t *bp = (uint8_t *)P(0x10);
  float *fp = (float *)P(0x10);
  moesq_weights_t w = weights(8, 128, 256, MOESQ_LAYOUT_CANONICAL, 0);

  /* routing */
  expect("route E=0", moesq_route(NULL, 4, 2, 0, ip, ip, ip, NULL, 0, NULL), MOESQ_ERR_SHAPE);
  expect("route E>max", moesq_route(NULL, 4, 2, MOESQ_MAX_EXPERTS + 1, ip, ip, ip, NULL, 0, NULL),
         MOESQ_ERR_SHAPE);
  expect("route k>E", moesq_route(NULL, 4, 9, 8, ip, ip, ip, NULL, 0, NULL), MOESQ_ERR_SHAPE);
  expect("route T<0", moesq_route(NULL, -1, 2, 8, ip, ip, ip, NULL, 0, NULL), MOESQ_ERR_SHAPE);
  expect("route ids NULL", moesq_route(NULL, 4, 2, 8, ip, ip, ip, NULL, 0, NULL), MOESQ_ERR_NULL);
  expect("route T*k overflow", moesq_route(ip, 1 << 30, 4, 8, ip, ip, ip, NULL, 0, NULL),
         MOESQ_ERR_SHAPE);
  expect("route_noalloc offsets NULL", moesq_route_noalloc(ip, 4, 2, 8, NULL, ip, ip, NULL),
         MOESQ_ERR_NULL);
  expect("route_noalloc beyond scratch",
         moesq_route_noalloc(ip, 600000, 1, 1024, ip, ip, ip, NULL), MOESQ_ERR_SHAPE);
  if (moesq_route_workspace_bytes(64, 2, 8) != 0) {
    printf("FAIL workspace of a small routing\n");
    ++failures;
  }

  /* dispatch and combine */
  expect("permute K%8", moesq_permute(hp, ip, 4, 2, 12, hp, NULL), MOESQ_ERR_SHAPE);
  expect("permute x NULL", moesq_permute(NULL, ip, 4, 2, 16, hp, NULL), MOESQ_ERR_NULL);
  expect("permute empty", moesq_permute(NULL, NULL, 0, 2, 16, NULL, NULL), MOESQ_OK);
  expect("unpermute N%8", moesq_unpermute(hp, ip, NULL, 4, 2, 12, hp, NULL), MOESQ_ERR_SHAPE);
  expect("unpermute k<1", moesq_unpermute(hp, ip, NULL, 4, 0, 16, hp, NULL), MOESQ_ERR_SHAPE);

  /* grouped GEMM */
  moesq_weights_t bad = weights(8, 128, 48, MOESQ_LAYOUT_CANONICAL, 0);
  expect("spgemm K%32", moesq_grouped_spgemm(hp, ip, 4, &bad, 0, hp, NULL, 0, NULL), MOESQ_ERR_SHAPE);
  bad = weights(8, 128, 256, 7, 0);
  expect("spgemm layout", moesq_grouped_spgemm(hp, ip, 4, &bad, 0, hp, NULL, 0, NULL),
         MOESQ_ERR_LAYOUT);
  bad = weights(8, 128, 256, MOESQ_LAYOUT_CANONICAL, 1);
  expect("spgemm NULL weights", moesq_grouped_spgemm(hp, ip, 4, &bad, 0, hp, NULL, 0, NULL),
         MOESQ_ERR_NULL);
  bad = weights(8, 48, 256, MOESQ_LAYOUT_CANONICAL, 0);
  expect("spgemm SwiGLU N%32", moesq_grouped_spgemm(hp, ip, 4, &bad, MOESQ_EPI_SWIGLU, hp, NULL, 0, NULL),
         MOESQ_ERR_SHAPE);
  bad = weights(8, 1 << 16, 1 << 17, MOESQ_LAYOUT_CANONICAL, 0);
  expect("spgemm 2 GiB expert", moesq_grouped_spgemm(hp, ip, 4, &bad, 0, hp, NULL, 0, NULL),
         MOESQ_ERR_SHAPE);
  expect("spgemm epilogue", moesq_grouped_spgemm(hp, ip, 4, &w, 5, hp, NULL, 0, NULL), MOESQ_ERR_ARG);
  expect("spgemm flat without perm",
         moesq_grouped_spgemm(hp, ip, 4, &w, MOESQ_OUT_FLAT, hp, NULL, 0, NULL), MOESQ_ERR_ARG);
  expect("spgemm M<0", moesq_grouped_spgemm(hp, ip, -1, &w, 0, hp, NULL, 0, NULL), MOESQ_ERR_SHAPE);
  expect("spgemm M=0", moesq_grouped_spgemm(NULL, ip, 0, &w, 0, NULL, NULL, 0, NULL), MOESQ_OK);
  expect("spgemm NULL descriptor", moesq_grouped_spgemm(hp, ip, 4, NULL, 0, hp, NULL, 0, NULL),
         MOESQ_ERR_NULL);
  expect("gather T<0", moesq_grouped_spgemm_gather(hp, ip, -1, 2, ip, &w, 0, hp, NULL, 0, NULL),
         MOESQ_ERR_SHAPE);
  expect("gather perm NULL", moesq_grouped_spgemm_gather(hp, NULL, 4, 2, ip, &w, 0, hp, NULL, 0, NULL),
         MOESQ_ERR_NULL);
  expect("fused route k>E",
         moesq_route_grouped_spgemm(ip, hp, 4, 9, &w, 0, hp, ip, ip, ip, NULL), MOESQ_ERR_SHAPE);
  expect("fused route ids NULL",
         moesq_route_grouped_spgemm(NULL, hp, 4, 2, &w, 0, hp, ip, ip, ip, NULL), MOESQ_ERR_NULL);

  /* W4A4 */
  expect("quantize K%32", moesq_quantize_activations(hp, 4, 48, bp, bp, fp, NULL), MOESQ_ERR_SHAPE);
  expect("quantize misaligned", moesq_quantize_activations((uint16_t *)P(0x18), 4, 64, bp, bp, fp, NULL),
         MOESQ_ERR_ARG);
  expect("quantize T=0", moesq_quantize_activations(NULL, 0, 64, NULL, NULL, NULL, NULL), MOESQ_OK);
  moesq_act4_t act = {bp, bp, fp, 8, 256};
  moesq_act4_t act_k = {bp, bp, fp, 8, 128};
  moesq_act4_t act_rows = {bp, bp, fp, 7, 256};
  expect("act4 NULL descriptor", moesq_grouped_spgemm_act4(NULL, NULL, 0, 1, ip, 8, &w, 0, hp, NULL),
         MOESQ_ERR_NULL);
  expect("act4 K differs", moesq_grouped_spgemm_act4(&act_k, NULL, 0, 1, ip, 8, &w, 0, hp, NULL),
         MOESQ_ERR_SHAPE);
  expect("act4 rows", moesq_grouped_spgemm_act4(&act_rows, NULL, 0, 1, ip, 8, &w, 0, hp, NULL),
         MOESQ_ERR_SHAPE);
  expect("act4 M != T*k", moesq_grouped_spgemm_act4(&act, ip, 4, 2, ip, 9, &w, 0, hp, NULL),
         MOESQ_ERR_SHAPE);

  /* packing, tiling, decode, validation, the read utility */
  expect("pack K%32", moesq_pack_weights(fp, 1, 16, 48, bp, bp, bp, fp, NULL), MOESQ_ERR_SHAPE);
  expect("pack paired E=0", moesq_pack_weights_paired(fp, 0, 16, 64, bp, bp, bp, fp, NULL),
         MOESQ_ERR_SHAPE);
  moesq_weights_t pt = weights(8, 128, 256, MOESQ_LAYOUT_PAIRED_TILED, 0);
  expect("tile a tiled source", moesq_tile_weights(&pt, bp, bp, bp, NULL), MOESQ_ERR_LAYOUT);
  expect("decode expert out of range", moesq_decode_weights(&w, 8, hp, NULL), MOESQ_ERR_ARG);
  expect("validate E=0 with ids", moesq_validate(ip, 4, 2, 0, NULL, NULL, NULL, NULL), MOESQ_ERR_SHAPE);
  expect("stream_read misaligned", moesq_stream_read(P(0x18), 16, (uint32_t *)P(0x10), NULL),
         MOESQ_ERR_ARG);

  for (int st = -7; st <= 1; ++st) {
    const char *name = moesq_status_string((moesq_status_t)st);
    if (!name || !name[0]) {
      printf("FAIL status string %d\n", st);
      ++failures;
    }
  }
  if (moesq_version() < 100) {
    printf("FAIL version\n");
    ++failures;
  }
  printf("%s: %d failure(s)\n", failures ? "FAILED" : "ok", failures);
  return failures ? 1 : 0;
}
