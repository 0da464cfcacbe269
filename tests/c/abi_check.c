/*
 * abi_check.c -- drives libidx through its C ABI alone (include/idx.h and the
 * HIP runtime; no Python, no PyTorch) on a batch whose answer is known in
 * closed form, and exits 0 when every check holds.
 *
 * Two decode requests of 300 and 9000 positions (one new token each, the
 * last position).  A few "planted" positions have K rows of all ones, every
 * other K row is zero; q is all ones and every head weight is one.  With the
 * score of IndexCache's lightning indexer, I[s] = ks[s] * sum_h w_h *
 * max(0, q8_h . k8_s), a zero row scores exactly 0 and every planted row
 * scores the same positive value.  The top-k row (k = 16, ties to the lower
 * position, ascending) is therefore the planted positions plus the lowest
 * zero-score positions.  Checked:
 *   idx_quant_write_k, idx_quant_q_fold_w, idx_score_topk (fused), idx_logits
 *   + idx_topk (must equal the fused rows), the logits themselves,
 *   idx_topk_to_physical, and one argument error (k = 0).
 */
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "idx.h"

#define NREQ 2
#define K 16
#define HEADS 64
#define DIM 128
#define BS 64

static int failures = 0;

#define HIP_OK(call)                                                        \
  do {                                                                      \
    hipError_t e_ = (call);                                                 \
    if (e_ != hipSuccess) {                                                 \
      fprintf(stderr, "%s:%d: %s\n", __FILE__, __LINE__, hipGetErrorString(e_)); \
      exit(2);                                                              \
    }                                                                       \
  } while (0)

#define IDX_OK_(call)                                                       \
  do {                                                                      \
    idx_status_t s_ = (call);                                               \
    if (s_ != IDX_OK) {                                                     \
      fprintf(stderr, "%s:%d: %s\n", __FILE__, __LINE__, idx_status_str(s_)); \
      exit(2);                                                              \
    }                                                                       \
  } while (0)

static void expect(int cond, const char* what, int t, int j) {
  if (!cond) {
    if (failures < 20) fprintf(stderr, "FAIL %s (token %d, entry %d)\n", what, t, j);
    ++failures;
  }
}

static void* dev_alloc(size_t bytes) {
  void* p = NULL;
  HIP_OK(hipMalloc(&p, bytes > 0 ? bytes : 1));
  return p;
}

static void* dev_copy(const void* host, size_t bytes) {
  void* p = dev_alloc(bytes);
  HIP_OK(hipMemcpy(p, host, bytes, hipMemcpyHostToDevice));
  return p;
}

static int cmp_int(const void* a, const void* b) {
  const int x = *(const int*)a, y = *(const int*)b;
  return (x > y) - (x < y);
}

int main(void) {
  const int32_t seq_lens[NREQ] = {300, 9000};
  const int32_t qsl[NREQ + 1] = {0, 1, 2};
  static const int planted0[] = {7, 123, 299};
  static const int planted1[] = {0, 4095, 4096, 8999};
  const int* planted[NREQ] = {planted0, planted1};
  const int nplanted[NREQ] = {3, 4};

  /* block tables: request 0 owns blocks 0..4, request 1 blocks 5..145 in reverse */
  const int64_t stride = (9000 + BS - 1) / BS;
  const int64_t num_blocks = 5 + stride;
  int32_t* bt = calloc((size_t)(NREQ * stride), sizeof(int32_t));
  for (int j = 0; j < 5; ++j) bt[j] = j;
  for (int j = 0; j < stride; ++j) bt[stride + j] = (int32_t)(5 + (stride - 1 - j));

  /* every position's K row (bf16 bits) and its slot */
  const int64_t rows = seq_lens[0] + seq_lens[1];
  uint16_t* kb = calloc((size_t)(rows * DIM), sizeof(uint16_t));
  int64_t* slots = malloc((size_t)rows * sizeof(int64_t));
  int64_t i = 0;
  for (int r = 0; r < NREQ; ++r)
    for (int p = 0; p < seq_lens[r]; ++p, ++i) {
      slots[i] = (int64_t)bt[r * stride + p / BS] * BS + p % BS;
      for (int q = 0; q < nplanted[r]; ++q)
        if (planted[r][q] == p)
          for (int d = 0; d < DIM; ++d) kb[i * DIM + d] = 0x3F80;   /* 1.0 */
    }
  uint16_t* qb = malloc(sizeof(uint16_t) * NREQ * HEADS * DIM);
  float* wraw = malloc(sizeof(float) * NREQ * HEADS);
  for (int j = 0; j < NREQ * HEADS * DIM; ++j) qb[j] = 0x3F80;
  for (int j = 0; j < NREQ * HEADS; ++j) wraw[j] = 1.0f;

  hipStream_t st;
  HIP_OK(hipStreamCreate(&st));
  idx_kcache_t cache = {(uint8_t*)dev_alloc((size_t)num_blocks * BS * 132), num_blocks, BS};
  HIP_OK(hipMemset(cache.data, 0, (size_t)num_blocks * BS * 132));
  uint16_t* d_kb = dev_copy(kb, sizeof(uint16_t) * rows * DIM);
  int64_t* d_slots = dev_copy(slots, sizeof(int64_t) * rows);
  IDX_OK_(idx_quant_write_k(d_kb, rows, DIM, DIM, d_slots, cache, st));

  uint16_t* d_qb = dev_copy(qb, sizeof(uint16_t) * NREQ * HEADS * DIM);
  float* d_wraw = dev_copy(wraw, sizeof(float) * NREQ * HEADS);
  uint8_t* d_q8 = dev_alloc((size_t)NREQ * HEADS * DIM);
  float* d_w = dev_alloc(sizeof(float) * NREQ * HEADS);
  IDX_OK_(idx_quant_q_fold_w(d_qb, d_wraw, NREQ, HEADS, DIM, 0.08838834764831845f, d_q8, d_w, NULL,
                             st));

  idx_batch_t b;
  b.seq_lens = dev_copy(seq_lens, sizeof(seq_lens));
  b.query_start_loc = dev_copy(qsl, sizeof(qsl));
  b.block_table = dev_copy(bt, sizeof(int32_t) * NREQ * stride);
  b.block_table_stride = stride;
  b.num_reqs = NREQ;
  b.num_tokens = NREQ;
  b.max_seq_len = 9000;
  b.max_query_len = 1;
  b.num_decode_tokens = 0;

  /* fused score + top-k */
  const size_t ws_bytes = idx_score_topk_workspace_size(&b, K);
  void* ws = dev_alloc(ws_bytes);
  int32_t* d_topk = dev_alloc(sizeof(int32_t) * NREQ * K);
  IDX_OK_(idx_score_topk(d_q8, d_w, HEADS, DIM, cache, &b, K, d_topk, K, ws, ws_bytes, st));

  /* unfused: scores, then top-k */
  float* d_logits = dev_alloc(sizeof(float) * NREQ * 9000);
  IDX_OK_(idx_logits(d_q8, d_w, HEADS, DIM, cache, &b, d_logits, 9000, st));
  const size_t ws2_bytes = idx_topk_workspace_size(&b, K);
  void* ws2 = dev_alloc(ws2_bytes);
  int32_t* d_topk2 = dev_alloc(sizeof(int32_t) * NREQ * K);
  IDX_OK_(idx_topk(d_logits, 9000, &b, K, d_topk2, K, ws2, ws2_bytes, st));

  /* logical -> physical */
  int32_t* d_phys = dev_alloc(sizeof(int32_t) * NREQ * K);
  int32_t* d_valid = dev_alloc(sizeof(int32_t) * NREQ);
  IDX_OK_(idx_topk_to_physical(d_topk, K, &b, BS, num_blocks, K, 0, d_phys, K, d_valid, st));

  /* an argument error enqueues nothing */
  expect(idx_score_topk(d_q8, d_w, HEADS, DIM, cache, &b, 0, d_topk, K, ws, ws_bytes, st) != IDX_OK,
         "k = 0 rejected", -1, -1);
  HIP_OK(hipStreamSynchronize(st));

  int32_t topk[NREQ * K], topk2[NREQ * K], phys[NREQ * K], valid[NREQ];
  float* logits = malloc(sizeof(float) * NREQ * 9000);
  HIP_OK(hipMemcpy(topk, d_topk, sizeof(topk), hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(topk2, d_topk2, sizeof(topk2), hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(phys, d_phys, sizeof(phys), hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(valid, d_valid, sizeof(valid), hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(logits, d_logits, sizeof(float) * NREQ * 9000, hipMemcpyDeviceToHost));

  for (int t = 0; t < NREQ; ++t) {
    /* expected row: planted positions plus the lowest zero-score positions, ascending */
    int want[K], nw = 0;
    for (int q = 0; q < nplanted[t]; ++q) want[nw++] = planted[t][q];
    for (int p = 0; nw < K; ++p) {
      int is_planted = 0;
      for (int q = 0; q < nplanted[t]; ++q) is_planted |= planted[t][q] == p;
      if (!is_planted) want[nw++] = p;
    }
    qsort(want, K, sizeof(int), cmp_int);
    const float* lg = logits + (size_t)t * 9000;
    const float top = lg[planted[t][0]];
    expect(top > 0.0f, "planted score positive", t, planted[t][0]);
    for (int p = 0; p < seq_lens[t]; ++p) {
      int is_planted = 0;
      for (int q = 0; q < nplanted[t]; ++q) is_planted |= planted[t][q] == p;
      if (is_planted)
        expect(lg[p] == top, "planted scores equal", t, p);
      else
        expect(lg[p] == 0.0f, "zero row scores 0", t, p);
    }
    for (int j = 0; j < K; ++j) {
      const int pos = want[j];
      expect(topk[t * K + j] == pos, "fused top-k row", t, j);
      expect(topk2[t * K + j] == pos, "unfused top-k row", t, j);
      expect(phys[t * K + j] == bt[t * stride + pos / BS] * BS + pos % BS, "physical slot", t, j);
    }
    expect(valid[t] == K, "valid count", t, -1);
  }

  if (failures == 0) printf("abi_check: ok (%s)\n", idx_version());
  else fprintf(stderr, "abi_check: %d failures\n", failures);
  return failures == 0 ? 0 : 1;
}
