/* A plain C99 caller of the library: it includes only include/veda.h, links libveda.so,
 * and exercises the host-side entry points that need no device (version, status text,
 * layer checks, workspace size, index count, and validation failures of the compute
 * calls, which return before any device call).  Prints one line per check and exits
 * with the number of failed checks. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "veda.h"

static int failures = 0;

static void expect(const char* what, long long got, long long want) {
  printf("%-58s %s (got %lld, want %lld)\n", what, got == want ? "ok" : "FAIL", got, want);
  if (got != want) ++failures;
}

/* the 1344x768 5.17 s layer: 129024 video tokens, then 512 text and 1024 audio tokens */
static veda_layer t2v_layer(void) {
  veda_layer L;
  memset(&L, 0, sizeof L);
  L.B = 1;
  L.H = 40;
  L.d = 128;
  L.p = 64;
  L.tile = 128;
  L.n_seg = 1;
  L.n_tokens = 129024 + 1536;
  L.stride_h = 128;
  L.stride_n = 40 * 128;
  L.stride_b = L.stride_n * L.n_tokens;
  L.query.start = 0;
  L.query.len = 129024;
  L.seg[0].start = 0;
  L.seg[0].len = 129024;
  L.budget[0] = 50;
  L.wdtype = VEDA_W_BF16;
  return L;
}

int main(void) {
  void* fake = (void*)(uintptr_t)0x10000;     /* never dereferenced: validation fails first */
  veda_range dense[2] = {{129024, 512}, {129536, 1024}};
  veda_layer L = t2v_layer();

  expect("veda_abi_version() == VEDA_ABI_VERSION", veda_abi_version(), VEDA_ABI_VERSION);
  expect("status text of VEDA_OK is not empty", veda_status_string(VEDA_OK)[0] != 0, 1);
  expect("layer valid for selection", veda_layer_check(&L, 1), VEDA_OK);
  expect("Ktot = 50", veda_k_total(&L), 50);
  /* q_hat [1,40,1008,64] + k_hat [1,40,1008,64] in fp32 */
  expect("selection workspace >= 2 * 40 * 1008 * 64 * 4 bytes",
         veda_select_workspace_bytes(&L) >= (size_t)2 * 40 * 1008 * 64 * 4, 1);

  veda_layer bad = L;
  bad.d = 96;
  expect("d = 96 is unsupported", veda_layer_check(&bad, 0), VEDA_EUNSUPPORTED);
  bad = L;
  bad.query.start = bad.n_tokens - 10;
  expect("query past the sequence", veda_layer_check(&bad, 0), VEDA_ERANGE);

  expect("veda_select without q", veda_select(&L, NULL, fake, fake, fake, fake, NULL, fake, 1u << 30, NULL),
         VEDA_EINVAL);
  expect("veda_sparse_attn with a dense range overlapping the video",
         veda_sparse_attn(&L, fake, fake, fake, fake, NULL, (veda_range[]){{128000, 2000}}, 1, 0.0f, fake, NULL,
                          NULL),
         VEDA_ERANGE);
  expect("veda_sparse_attn with a negative scale",
         veda_sparse_attn(&L, fake, fake, fake, fake, NULL, dense, 2, -1.0f, fake, NULL, NULL), VEDA_EINVAL);
  expect("veda_sparse_attn with an order but no index",
         veda_sparse_attn(&L, fake, fake, fake, NULL, fake, dense, 2, 0.0f, fake, NULL, NULL), VEDA_EINVAL);
  expect("veda_tile_order without an index", veda_tile_order(&L, NULL, fake, NULL), VEDA_EINVAL);
  expect("veda_sparse_attn_fp8qk without scales",
         veda_sparse_attn_fp8qk(&L, fake, fake, fake, NULL, NULL, fake, NULL, dense, 2, 0.0f, fake, NULL, NULL),
         VEDA_EINVAL);
  expect("veda_dequant_fp8_e4m3 of nothing is a no-op", veda_dequant_fp8_e4m3(fake, fake, 0, 0, NULL), VEDA_OK);
  return failures;
}
