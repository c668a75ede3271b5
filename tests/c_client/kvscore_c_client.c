/*
 * A plain C client of libkvscore: the whole hot path through the C ABI alone (no torch, no
 * Python), with device memory and a stream from the HIP runtime's C API.
 *
 *   kvscore_c_client IN OUT
 *
 * IN (little-endian binary): int32 S, L, Hq, Hkv, d, W, mode; int64 cu_seqlens[S+1];
 * float64 ratio, frac; then q_win bf16 [L][S][Hq][W][d] and k, v bf16 [L][Hkv][N][d]
 * (head-major, N = cu_seqlens[S]). The budgets of sequence s come from kvscore_budget with
 * a flat profile and a total of floor(frac * L * n_s) slots.
 *
 * OUT: int32 budgets [S][L]; int64 segment offsets [U+1]; float32 score [L][Hkv][N];
 * int32 kept positions [R]; bf16 k_out, v_out [R][d] (R = offsets[U]).
 *
 * Exit status 0 on success; otherwise the failing call and kvscore_last_error() are
 * printed to stderr.
 */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "kvscore.h"

#define HIP_OK(x)                                                            \
  do {                                                                       \
    hipError_t e_ = (x);                                                     \
    if (e_ != hipSuccess) {                                                  \
      fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_));                \
      return 2;                                                              \
    }                                                                        \
  } while (0)
#define KV_OK(x)                                                             \
  do {                                                                       \
    int rc_ = (x);                                                           \
    if (rc_ != 0) {                                                          \
      fprintf(stderr, "%s -> %d: %s\n", #x, rc_, kvscore_last_error());      \
      return 3;                                                              \
    }                                                                        \
  } while (0)

static int read_all(FILE* f, void* p, size_t n) { return fread(p, 1, n, f) == n ? 0 : -1; }
static int write_all(FILE* f, const void* p, size_t n) { return fwrite(p, 1, n, f) == n ? 0 : -1; }

static void* dev_alloc(size_t n, hipError_t* err) {
  void* p = NULL;
  *err = hipMalloc(&p, n ? n : 1);
  return p;
}

int main(int argc, char** argv) {
  if (argc != 3) {
    fprintf(stderr, "usage: %s IN OUT\n", argv[0]);
    return 1;
  }
  FILE* in = fopen(argv[1], "rb");
  if (!in) {
    perror(argv[1]);
    return 1;
  }
  int32_t hdr[7];
  if (read_all(in, hdr, sizeof hdr)) return 1;
  const int S = hdr[0], L = hdr[1], Hq = hdr[2], Hkv = hdr[3], d = hdr[4], W = hdr[5], mode = hdr[6];
  if (S < 1 || S > KVSCORE_MAX_SEQS) return 1;
  int64_t cu[KVSCORE_MAX_SEQS + 1];
  double ratio, frac;
  if (read_all(in, cu, sizeof(int64_t) * (S + 1)) || read_all(in, &ratio, 8) || read_all(in, &frac, 8)) return 1;
  const int64_t N = cu[S], U = (int64_t)L * S * Hkv, rows = (int64_t)L * S * Hq * W;
  const size_t qn = (size_t)rows * d * 2, kvn = (size_t)L * Hkv * N * d * 2;
  unsigned char* hq = malloc(qn);
  unsigned char* hk = malloc(kvn);
  unsigned char* hv = malloc(kvn);
  if (!hq || !hk || !hv || read_all(in, hq, qn) || read_all(in, hk, kvn) || read_all(in, hv, kvn)) return 1;
  fclose(in);

  kvscore_problem p;
  memset(&p, 0, sizeof p);
  p.num_seqs = S;
  p.num_layers = L;
  p.num_q_heads = Hq;
  p.num_kv_heads = Hkv;
  p.head_dim = d;
  p.window = W;
  p.cu_seqlens = cu;
  p.k_strides[0] = p.v_strides[0] = (int64_t)Hkv * N * d;
  p.k_strides[1] = p.v_strides[1] = N * d;
  p.k_strides[2] = p.v_strides[2] = d;
  p.mode = mode;
  p.softmax_scale = 0.f;

  /* budgets: a flat profile, floor(frac * L * n_s) slots per sequence, each layer in [W, n_s] */
  int32_t* budgets = malloc(sizeof(int32_t) * S * L);
  double* prof = calloc((size_t)L, sizeof(double));
  if (!budgets || !prof) return 1;
  for (int s = 0; s < S; ++s) {
    const int64_t n = cu[s + 1] - cu[s];
    KV_OK(kvscore_budget(prof, L, ratio, INFINITY, (int64_t)floor(frac * L * n), W, (int32_t)n, budgets + s * L));
  }
  int64_t* off = malloc(sizeof(int64_t) * (U + 1));
  if (!off) return 1;
  KV_OK(kvscore_segment_offsets(&p, budgets, off));
  const int64_t R = off[U];

  hipStream_t st;
  HIP_OK(hipStreamCreate(&st));
  hipError_t e = hipSuccess;
  void *q = dev_alloc(qn, &e), *k = NULL, *v = NULL;
  HIP_OK(e);
  k = dev_alloc(kvn, &e);
  HIP_OK(e);
  v = dev_alloc(kvn, &e);
  HIP_OK(e);
  const int Tq = kvscore_num_query_tiles(&p);
  if (Tq < 1) {
    fprintf(stderr, "kvscore_num_query_tiles: %s\n", kvscore_last_error());
    return 3;
  }
  float *a = dev_alloc(sizeof(float) * rows * d, &e), *lse = NULL, *dom = NULL, *partial = NULL, *score = NULL;
  HIP_OK(e);
  lse = dev_alloc(sizeof(float) * rows, &e);
  HIP_OK(e);
  dom = dev_alloc(sizeof(float) * rows, &e);
  HIP_OK(e);
  int32_t* jstar = dev_alloc(sizeof(int32_t) * rows, &e);
  HIP_OK(e);
  partial = dev_alloc(sizeof(float) * L * Hkv * (size_t)Tq * N, &e);
  HIP_OK(e);
  score = dev_alloc(sizeof(float) * L * Hkv * (size_t)N, &e);
  HIP_OK(e);
  const size_t ws_fwd = kvscore_workspace_size(&p, KVSCORE_WS_ATTN_FWD);
  const size_t ws_sc = kvscore_workspace_size(&p, KVSCORE_WS_SCORE);
  void* wf = dev_alloc(ws_fwd, &e);
  HIP_OK(e);
  void* wsc = dev_alloc(ws_sc, &e);
  HIP_OK(e);
  int64_t* doff = dev_alloc(sizeof(int64_t) * (U + 1), &e);
  HIP_OK(e);
  int32_t* kept = dev_alloc(sizeof(int32_t) * R, &e);
  HIP_OK(e);
  void* kout = dev_alloc((size_t)R * d * 2, &e);
  HIP_OK(e);
  void* vout = dev_alloc((size_t)R * d * 2, &e);
  HIP_OK(e);

  HIP_OK(hipMemcpyAsync(q, hq, qn, hipMemcpyHostToDevice, st));
  HIP_OK(hipMemcpyAsync(k, hk, kvn, hipMemcpyHostToDevice, st));
  HIP_OK(hipMemcpyAsync(v, hv, kvn, hipMemcpyHostToDevice, st));
  HIP_OK(hipMemcpyAsync(doff, off, sizeof(int64_t) * (U + 1), hipMemcpyHostToDevice, st));

  KV_OK(kvscore_attn_fwd(&p, q, k, v, a, lse, jstar, dom, ws_fwd ? wf : NULL, ws_fwd, st));
  KV_OK(kvscore_score(&p, q, k, v, a, lse, jstar, partial, wsc, ws_sc, st));
  KV_OK(kvscore_merge(&p, partial, jstar, dom, score, st));
  KV_OK(kvscore_topk(&p, score, budgets, doff, kept, 1, 0, NULL, 0, st));
  KV_OK(kvscore_compact(&p, k, v, budgets, doff, kept, kout, vout, st));

  float* hscore = malloc(sizeof(float) * L * Hkv * (size_t)N);
  int32_t* hkept = malloc(sizeof(int32_t) * (R ? R : 1));
  unsigned char* hko = malloc((size_t)R * d * 2 + 1);
  unsigned char* hvo = malloc((size_t)R * d * 2 + 1);
  if (!hscore || !hkept || !hko || !hvo) return 1;
  HIP_OK(hipMemcpyAsync(hscore, score, sizeof(float) * L * Hkv * (size_t)N, hipMemcpyDeviceToHost, st));
  HIP_OK(hipMemcpyAsync(hkept, kept, sizeof(int32_t) * R, hipMemcpyDeviceToHost, st));
  HIP_OK(hipMemcpyAsync(hko, kout, (size_t)R * d * 2, hipMemcpyDeviceToHost, st));
  HIP_OK(hipMemcpyAsync(hvo, vout, (size_t)R * d * 2, hipMemcpyDeviceToHost, st));
  HIP_OK(hipStreamSynchronize(st));

  FILE* out = fopen(argv[2], "wb");
  if (!out) {
    perror(argv[2]);
    return 1;
  }
  if (write_all(out, budgets, sizeof(int32_t) * S * L) || write_all(out, off, sizeof(int64_t) * (U + 1)) ||
      write_all(out, hscore, sizeof(float) * L * Hkv * (size_t)N) || write_all(out, hkept, sizeof(int32_t) * R) ||
      write_all(out, hko, (size_t)R * d * 2) || write_all(out, hvo, (size_t)R * d * 2))
    return 1;
  fclose(out);

  hipFree(q);
  hipFree(k);
  hipFree(v);
  hipFree(a);
  hipFree(lse);
  hipFree(dom);
  hipFree(jstar);
  hipFree(partial);
  hipFree(score);
  hipFree(wf);
  hipFree(wsc);
  hipFree(doff);
  hipFree(kept);
  hipFree(kout);
  hipFree(vout);
  HIP_OK(hipStreamDestroy(st));
  free(hq);
  free(hk);
  free(hv);
  free(budgets);
  free(prof);
  free(off);
  free(hscore);
  free(hkept);
  free(hko);
  free(hvo);
  return 0;
}
