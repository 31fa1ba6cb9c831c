/* Host-only checks of the moeq C ABI under AddressSanitizer / UBSan (no GPU): shape and
   argument validation with fake device pointers (nothing is launched), the host
   repack and the host MXFP4 -> NVFP4 conversion on exact-size heap buffers. */
#include <stdio.h>
#include <stdlib.h>
#include <string.h>
#include <stdint.h>
#include "moeq.h"

static int fails = 0;
#define CHECK(c) do { if (!(c)) { printf("FAIL %s:%d %s\n", __FILE__, __LINE__, #c); fails++; } } while (0)

int main(void) {
  for (int fmt = 0; fmt <= 9; fmt++)
    for (int r = 1; r <= 4096; r *= 4)
      for (int c = 16; c <= 8192; c *= 2)
        for (int p = -1; p <= 2; p++) (void)moeq_plane_bytes(fmt, r, c, p);
  CHECK(moeq_packed_bytes(1, 2048, 4096) == 2048 * 4096 / 2 + 2048 * 4096 / 32);
  CHECK(moeq_plane_bytes(8, 24, 512, 0) == 0);
  /* host repack on exact-size buffers */
  for (int fmt = 3; fmt <= 4; fmt++) {
    int rows = 3, cols = 768, bs = fmt == 3 ? 84 : 66;
    size_t nb = (size_t)rows * (cols / 256);
    uint8_t* blocks = malloc(nb * bs);
    uint8_t* d = malloc(moeq_plane_bytes(fmt, rows, cols, 0));
    uint8_t* s = malloc(moeq_plane_bytes(fmt, rows, cols, 1));
    for (size_t i = 0; i < nb * bs; i++) blocks[i] = (uint8_t)(i * 131u);
    CHECK(moeq_pack_ggml(fmt, blocks, rows, cols, d, s) == MOEQ_OK);
    CHECK(moeq_pack_ggml(fmt, blocks, rows, 700, d, s) == MOEQ_E_SHAPE);
    CHECK(moeq_pack_ggml(1, blocks, rows, cols, d, s) == MOEQ_E_FMT);
    free(blocks); free(d); free(s);
  }
  /* host MXFP4 -> NVFP4 on exact-size buffers, lossless and lossy */
  {
    int rows = 5, cols = 96;
    uint8_t* nib = malloc(rows * cols / 2);
    uint8_t* e8 = malloc(rows * cols / 32);
    uint8_t* nib2 = malloc(rows * cols / 2);
    uint8_t* e4 = malloc(rows * cols / 16);
    float s2;
    for (int i = 0; i < rows * cols / 2; i++) nib[i] = (uint8_t)(i * 7);
    for (int i = 0; i < rows * cols / 32; i++) e8[i] = (uint8_t)(110 + i % 18);
    CHECK(moeq_mxfp4_to_nvfp4(nib, e8, rows, cols, nib2, e4, &s2) == MOEQ_OK);
    CHECK(memcmp(nib, nib2, rows * cols / 2) == 0);
    e8[3] = 255;
    CHECK(moeq_mxfp4_to_nvfp4(nib, e8, rows, cols, nib2, e4, &s2) == MOEQ_E_LOSSY);
    e8[3] = 0; e8[4] = 200;
    CHECK(moeq_mxfp4_to_nvfp4(nib, e8, rows, cols, nib2, e4, &s2) == MOEQ_E_LOSSY);
    CHECK(moeq_mxfp4_to_nvfp4(nib, e8, rows, 100, nib2, e4, &s2) == MOEQ_E_SHAPE);
    free(nib); free(e8); free(nib2); free(e4);
  }
  /* validation with fake device pointers: every call must return before any launch */
  {
    moeq_weight w = {1, 256, 512, 2, (void*)0x10000, 1 << 20, (void*)0x20000, 1 << 20, (float*)0x30000, (uint8_t*)0x40000};
    moeq_layer L;
    memset(&L, 0, sizeof(L));
    L.hidden = 1024; L.inter = 512; L.n_experts = 8; L.top_k = 2;
    moeq_weight g = {1, 512, 1024, 8, (void*)0x10000, 1 << 20, (void*)0x20000, 1 << 16, 0, 0};
    moeq_weight dn = {1, 1024, 512, 8, (void*)0x10000, 1 << 20, (void*)0x20000, 1 << 16, 0, 0};
    L.gate = g; L.up = g; L.down = dn;
    size_t n1 = moeq_workspace_bytes(&L, 1), n64 = moeq_workspace_bytes(&L, 64), n4k = moeq_workspace_bytes(&L, 4096);
    CHECK(n1 > 0 && n64 > n1 && n4k > n64);
    void* p = (void*)0x100000;
    CHECK(moeq_expert_forward(&L, p, p, p, 1, p, p, n1 - 1, NULL) == MOEQ_E_WORKSPACE);
    CHECK(moeq_expert_forward(&L, p, p, p, -1, p, p, n1, NULL) == MOEQ_E_INVAL);
    CHECK(moeq_expert_forward(&L, p, p, p, 0, p, p, n1, NULL) == MOEQ_OK);
    CHECK(moeq_expert_forward_noalloc(&L, p, p, p, 100000, p, NULL, NULL) == MOEQ_E_SCRATCH);
    CHECK(moeq_linear(&w, 5, p, 1, p, NULL) == MOEQ_E_INVAL);
    w.fmt = 8; w.cols = 640;
    CHECK(moeq_linear(&w, 0, p, 1, p, NULL) == MOEQ_E_SHAPE);
    CHECK(moeq_mxfp8_to_tiled(p, p, 16, 640, 1, p, p, NULL) == MOEQ_E_SHAPE);
    CHECK(moeq_mxfp4_to_nvfp4_device(p, p, 16, 48, 1, p, p, p, p, NULL) == MOEQ_E_SHAPE);
    CHECK(moeq_nvfp4_to_mxfp4_device(p, p, p, 16, 64, -1, p, p, p, NULL) == MOEQ_E_INVAL);
    L.top_k = 17;
    CHECK(moeq_workspace_bytes(&L, 1) == 0);
    L.top_k = 2; L.n_experts = 2000;
    CHECK(moeq_workspace_bytes(&L, 1) == 0);
  }
  for (int i = -9; i <= 1; i++) CHECK(moeq_status_string(i) != NULL);
  printf("%s (%d failures)\n", fails ? "FAILED" : "ok", fails);
  return fails != 0;
}
