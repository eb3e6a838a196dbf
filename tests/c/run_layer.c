/* A plain C99 host program that runs the selection and the block-sparse attention of one
 * layer through the C ABI, with device memory from the HIP runtime API only (no PyTorch).
 *
 * usage: run_layer <input file> <output file>
 * input:  veda_layer (raw struct), int32 n_dense, veda_range dense[n_dense],
 *         then bf16 q, k, v [B, n_tokens, H, d] and bf16 wq, wk [H, p, d] (raw bits)
 * output: int32 idx [B, H, Tq, Ktot], then bf16 out [B, n_tokens, H, d]
 * Exit status: 0 on success, else the failing step's number. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "veda.h"

static void* read_all(FILE* f, size_t n) {
  void* p = malloc(n ? n : 1);
  if (p && n && fread(p, 1, n, f) != n) {
    free(p);
    return NULL;
  }
  return p;
}

/* device copy of n host bytes (host NULL: uninitialised device memory) */
static void* upload(const void* host, size_t n) {
  void* d = NULL;
  if (hipMalloc(&d, n ? n : 16) != hipSuccess) return NULL;
  if (n && host && hipMemcpy(d, host, n, hipMemcpyHostToDevice) != hipSuccess) return NULL;
  return d;
}

int main(int argc, char** argv) {
  if (argc != 3) return 1;
  FILE* in = fopen(argv[1], "rb");
  if (!in) return 2;
  veda_layer L;
  int32_t n_dense = 0;
  if (fread(&L, sizeof L, 1, in) != 1 || fread(&n_dense, 4, 1, in) != 1 || n_dense < 0 || n_dense > 8) return 3;
  veda_range dense[8];
  if (n_dense && fread(dense, sizeof(veda_range), (size_t)n_dense, in) != (size_t)n_dense) return 3;
  const size_t tensor = (size_t)L.B * (size_t)L.n_tokens * (size_t)L.H * (size_t)L.d * 2;
  const size_t weights = (size_t)L.H * (size_t)L.p * (size_t)L.d * 2;
  void* hq = read_all(in, tensor);
  void* hk = read_all(in, tensor);
  void* hv = read_all(in, tensor);
  void* hwq = read_all(in, weights);
  void* hwk = read_all(in, weights);
  fclose(in);
  if (!hq || !hk || !hv || !hwq || !hwk) return 4;

  void* q = upload(hq, tensor);
  void* k = upload(hk, tensor);
  void* v = upload(hv, tensor);
  void* wq = upload(hwq, weights);
  void* wk = upload(hwk, weights);
  void* out = upload(NULL, tensor);
  const int64_t tq = (L.query.len + L.tile - 1) / L.tile;
  const size_t idx_bytes = (size_t)L.B * (size_t)L.H * (size_t)tq * (size_t)veda_k_total(&L) * 4;
  void* idx = upload(NULL, idx_bytes);
  const size_t ws_bytes = veda_select_workspace_bytes(&L);
  void* ws = upload(NULL, ws_bytes);
  if (!q || !k || !v || !wq || !wk || !out || !idx || !ws) return 5;
  if (hipMemset(out, 0, tensor) != hipSuccess) return 5;

  int st = veda_select(&L, q, k, wq, wk, (int32_t*)idx, NULL, ws, ws_bytes, NULL);
  if (st != VEDA_OK) {
    fprintf(stderr, "veda_select: %s\n", veda_status_string(st));
    return 6;
  }
  st = veda_sparse_attn(&L, q, k, v, (const int32_t*)idx, NULL, dense, n_dense, 0.0f, out, NULL, NULL);
  if (st != VEDA_OK) {
    fprintf(stderr, "veda_sparse_attn: %s\n", veda_status_string(st));
    return 7;
  }
  if (hipDeviceSynchronize() != hipSuccess) return 8;

  void* hidx = malloc(idx_bytes ? idx_bytes : 1);
  void* hout = malloc(tensor);
  if (!hidx || !hout) return 9;
  if (hipMemcpy(hidx, idx, idx_bytes, hipMemcpyDeviceToHost) != hipSuccess) return 9;
  if (hipMemcpy(hout, out, tensor, hipMemcpyDeviceToHost) != hipSuccess) return 9;
  FILE* o = fopen(argv[2], "wb");
  if (!o || fwrite(hidx, 1, idx_bytes, o) != idx_bytes || fwrite(hout, 1, tensor, o) != tensor) return 10;
  fclose(o);
  hipFree(q);
  hipFree(k);
  hipFree(v);
  hipFree(wq);
  hipFree(wk);
  hipFree(out);
  hipFree(idx);
  hipFree(ws);
  free(hq);
  free(hk);
  free(hv);
  free(hwq);
  free(hwk);
  free(hidx);
  free(hout);
  printf("run_layer: ok\n");
  return 0;
}
