/*
 * abi_check.c: the C ABI of libcpattn (include/cp_attn.h) driven from plain
 * C99, with device memory from the HIP runtime's C API and nothing else, no
 * Python and no torch.
 *
 * Every check has a closed-form answer worked out on the host in double
 * precision, so no reference implementation is needed:
 *  - Q = 0 makes every score 0: each row's weights are uniform over the keys
 *    it sees, O_i is the mean of those value rows and LSE_i = ln(count)
 *    (softmax definition; Context parallelism guide (diffusers), section Ring
 *    Attention for the chunked form).
 *  - The ring over three uneven chunks gives the same rows.
 *  - seq2head then head2seq is the identity, and seq2head moves every element
 *    to out[p][b][q*S_l + s][h][d] from in[q][b][s][p*H_l + h][d]
 *    (Context parallelism guide (diffusers), section Ulysses Attention).
 *  - The uneven regroupings and the K/V gather, on two stacked tensors, move
 *    every element by their index formulas (Context parallelism guide
 *    (diffusers), section Ulysses Anything Attention; Sequence Parallelism
 *    page (SGLang Diffusion), K/V gather) and the uneven pair round-trips.
 *  - With Q = 0 and 128 keys the backward is: dV_j = (1/128) sum_i dO_i,
 *    dK_j = 0, dQ_i = scale sum_j (1/128)(<dO_i, v_j> - Delta_i) k_j with
 *    Delta_i = <dO_i, mean_j v_j> (derivative of the same softmax).
 *  - A rejected call returns its status, sets cp_last_error and leaves the
 *    output untouched.
 * Tolerances: the uniform forward is exact up to fp32 summation (1e-4 on values
 * of size ~1); the backward rounds dS to bf16 (relative 2^-8), so it is held to
 * 1e-2 of the largest reference value.
 *
 * Exit status 0 when every check passes.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "cp_attn.h"

static int failures = 0;

#define CHECK_HIP(x)                                                          \
  do {                                                                        \
    hipError_t e_ = (x);                                                      \
    if (e_ != hipSuccess) {                                                   \
      fprintf(stderr, "HIP error %d at %s:%d\n", (int)e_, __FILE__, __LINE__); \
      exit(2);                                                                \
    }                                                                         \
  } while (0)

static void expect(int ok, const char* what) {
  if (!ok) {
    fprintf(stderr, "FAILED: %s\n", what);
    ++failures;
  }
}

/* bf16 encoding by round-to-nearest-even of the fp32 bits (inputs are finite). */
static uint16_t to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
static double from_bf16(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* Seeded values in [-1, 1): a 64-bit linear congruential generator. */
static uint64_t lcg_state = 0x9e3779b97f4a7c15ull;
static float next_uniform(void) {
  lcg_state = lcg_state * 6364136223846793005ull + 1442695040888963407ull;
  return (float)((double)(lcg_state >> 11) / 9007199254740992.0 * 2.0 - 1.0);
}

static void* dev_alloc(size_t bytes) {
  void* p = NULL;
  CHECK_HIP(hipMalloc(&p, bytes ? bytes : 16));
  return p;
}

/* ---------------------------------------------------------------- forward */
static void check_forward(void) {
  enum { Sq = 70, Skv = 150, H = 3, D = 128 };
  const size_t nq = (size_t)Sq * H * D, nk = (size_t)Skv * H * D;
  uint16_t* hq = calloc(nq, 2);
  uint16_t* hk = malloc(nk * 2);
  uint16_t* hv = malloc(nk * 2);
  for (size_t x = 0; x < nk; ++x) hk[x] = to_bf16(next_uniform());
  for (size_t x = 0; x < nk; ++x) hv[x] = to_bf16(next_uniform());
  void *q = dev_alloc(nq * 2), *k = dev_alloc(nk * 2), *v = dev_alloc(nk * 2);
  float* o = dev_alloc(nq * 4);
  float* lse = dev_alloc((size_t)H * Sq * 4);
  CHECK_HIP(hipMemcpy(q, hq, nq * 2, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(k, hk, nk * 2, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(v, hv, nk * 2, hipMemcpyHostToDevice));
  float* ho = malloc(nq * 4);
  float* hl = malloc((size_t)H * Sq * 4);

  for (int causal = 0; causal <= 1; ++causal) {
    cp_status st = cp_attn_chunk_partial(q, k, v, o, lse, 1, H, Sq, Skv, D, CP_BF16, CP_F32,
                                         0.125f, causal, 0, 0, NULL);
    expect(st == CP_OK, "cp_attn_chunk_partial returns CP_OK");
    CHECK_HIP(hipDeviceSynchronize());
    CHECK_HIP(hipMemcpy(ho, o, nq * 4, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(hl, lse, (size_t)H * Sq * 4, hipMemcpyDeviceToHost));
    double err_o = 0.0, err_l = 0.0;
    for (int i = 0; i < Sq; ++i)
      for (int h = 0; h < H; ++h) {
        const int n = causal ? (i + 1 < Skv ? i + 1 : Skv) : Skv;  /* keys row i sees */
        err_l = fmax(err_l, fabs(hl[h * Sq + i] - log((double)n)));
        for (int d = 0; d < D; ++d) {
          double mean = 0.0;
          for (int j = 0; j < n; ++j) mean += from_bf16(hv[((size_t)j * H + h) * D + d]);
          mean /= n;
          err_o = fmax(err_o, fabs(ho[((size_t)i * H + h) * D + d] - mean));
        }
      }
    expect(err_o <= 1e-4, causal ? "causal uniform O" : "uniform O");
    expect(err_l <= 1e-4, causal ? "causal LSE = ln(visible keys)" : "LSE = ln(keys)");
    printf("ok: chunk partial %s, max-abs O %.2e, LSE %.2e\n", causal ? "causal" : "non-causal",
           err_o, err_l);
  }

  /* ring over three uneven chunks (pointers into the same K/V), bf16 out */
  const int64_t lens[3] = {61, 0, 89};
  cp_kv_chunk chunks[3];
  int64_t start = 0;
  for (int c = 0; c < 3; ++c) {
    chunks[c].k = (const char*)k + (size_t)start * H * D * 2;
    chunks[c].v = (const char*)v + (size_t)start * H * D * 2;
    chunks[c].len = lens[c];
    chunks[c].pos0 = start;
    start += lens[c];
  }
  size_t ws_bytes = cp_ring_attention_workspace_bytes(3, 1, H, Sq, D);
  void* ws = ws_bytes ? dev_alloc(ws_bytes) : NULL;
  void* ob = dev_alloc(nq * 2);
  cp_status st = cp_ring_attention(q, chunks, 3, ob, lse, 1, H, Sq, D, CP_BF16, 0.125f, 0, 0, ws,
                                   ws_bytes, NULL);
  expect(st == CP_OK, "cp_ring_attention returns CP_OK");
  CHECK_HIP(hipDeviceSynchronize());
  uint16_t* hob = malloc(nq * 2);
  CHECK_HIP(hipMemcpy(hob, ob, nq * 2, hipMemcpyDeviceToHost));
  double err = 0.0;
  for (int i = 0; i < Sq; ++i)
    for (int h = 0; h < H; ++h)
      for (int d = 0; d < D; ++d) {
        double mean = 0.0;
        for (int j = 0; j < Skv; ++j) mean += from_bf16(hv[((size_t)j * H + h) * D + d]);
        mean /= Skv;
        err = fmax(err, fabs(from_bf16(hob[((size_t)i * H + h) * D + d]) - mean));
      }
  expect(err <= 4e-3, "ring O (bf16 output: half a bf16 step of values below 1)");
  printf("ok: ring over chunks of 61, 0 and 89 keys, max-abs O %.2e\n", err);

  /* a rejected call: status, error text, output untouched */
  CHECK_HIP(hipMemset(o, 0x5a, nq * 4));
  st = cp_attn_chunk_partial(q, k, v, o, lse, 1, H, Sq, Skv, 96, CP_BF16, CP_F32, 0.125f, 0, 0, 0,
                             NULL);
  expect(st == CP_E_UNSUPPORTED, "head dim 96 is CP_E_UNSUPPORTED");
  expect(strlen(cp_last_error()) > 0, "cp_last_error describes the rejection");
  CHECK_HIP(hipMemcpy(ho, o, nq * 4, hipMemcpyDeviceToHost));
  int untouched = 1;
  for (size_t x = 0; x < nq; ++x) {
    uint32_t u;
    memcpy(&u, &ho[x], 4);
    if (u != 0x5a5a5a5au) untouched = 0;
  }
  expect(untouched, "a rejected call leaves the output untouched");
  printf("ok: rejected call (\"%s\")\n", cp_last_error());

  free(hq), free(hk), free(hv), free(ho), free(hl), free(hob);
  hipFree(q), hipFree(k), hipFree(v), hipFree(o), hipFree(lse), hipFree(ob);
  if (ws) hipFree(ws);
}

/* --------------------------------------------------------------- relayout */
static void check_relayout(void) {
  enum { P = 4, B = 2, S_l = 13, H = 8, D = 64 };
  const int H_l = H / P;
  const size_t n = (size_t)P * B * S_l * H * D;
  uint16_t* hin = malloc(n * 2);
  uint16_t* hout = malloc(n * 2);
  for (size_t x = 0; x < n; ++x) hin[x] = (uint16_t)(x * 2654435761u >> 7);
  void *in = dev_alloc(n * 2), *mid = dev_alloc(n * 2), *back = dev_alloc(n * 2);
  CHECK_HIP(hipMemcpy(in, hin, n * 2, hipMemcpyHostToDevice));
  expect(cp_ulysses_seq2head(in, mid, P, B, S_l, H, D, CP_BF16, NULL) == CP_OK, "seq2head");
  expect(cp_ulysses_head2seq(mid, back, P, B, S_l, H, D, CP_BF16, NULL) == CP_OK, "head2seq");
  CHECK_HIP(hipDeviceSynchronize());
  CHECK_HIP(hipMemcpy(hout, mid, n * 2, hipMemcpyDeviceToHost));
  int perm_ok = 1;
  for (int p = 0; p < P; ++p)
    for (int b = 0; b < B; ++b)
      for (int q = 0; q < P; ++q)
        for (int s = 0; s < S_l; ++s)
          for (int h = 0; h < H_l; ++h)
            for (int d = 0; d < D; ++d) {
              const size_t o = ((((size_t)p * B + b) * (P * S_l) + q * S_l + s) * H_l + h) * D + d;
              const size_t i = ((((size_t)q * B + b) * S_l + s) * H + p * H_l + h) * D + d;
              if (hout[o] != hin[i]) perm_ok = 0;
            }
  expect(perm_ok, "seq2head moves in[q][b][s][p*H_l+h][d] to out[p][b][q*S_l+s][h][d]");
  CHECK_HIP(hipMemcpy(hout, back, n * 2, hipMemcpyDeviceToHost));
  expect(memcmp(hout, hin, n * 2) == 0, "head2seq(seq2head(x)) == x");
  printf("ok: Ulysses regrouping, P=%d B=%d S_l=%d H=%d D=%d, bit for bit\n", P, B, S_l, H, D);
  free(hin), free(hout);
  hipFree(in), hipFree(mid), hipFree(back);
}

/* ------------------------------------------- uneven regroupings, stacked */
static void check_uneven_relayout(void) {
  enum { P = 3, B = 2, D = 24, COUNT = 2 };
  const int64_t s_lens[P] = {5, 0, 4}, h_counts[P] = {2, 3, 0};
  int64_t s_off[P + 1] = {0}, h_off[P + 1] = {0};
  for (int r = 0; r < P; ++r) {
    s_off[r + 1] = s_off[r] + s_lens[r];
    h_off[r + 1] = h_off[r] + h_counts[r];
  }
  const int64_t S = s_off[P], H = h_off[P];
  const size_t n = (size_t)B * S * H * D; /* elements of one tensor */
  uint16_t* hin = malloc(COUNT * n * 2);
  uint16_t* hout = malloc(COUNT * n * 2);
  for (size_t x = 0; x < COUNT * n; ++x) hin[x] = (uint16_t)(x * 40503u + 7u);
  void *in = dev_alloc(COUNT * n * 2), *mid = dev_alloc(COUNT * n * 2);
  void *back = dev_alloc(COUNT * n * 2), *gath = dev_alloc(COUNT * n * 2);
  CHECK_HIP(hipMemcpy(in, hin, COUNT * n * 2, hipMemcpyHostToDevice));
  expect(cp_ulysses_anything_seq2head_n(in, mid, COUNT, P, B, s_lens, h_counts, D, CP_BF16,
                                        NULL) == CP_OK, "anything seq2head_n");
  expect(cp_ulysses_anything_head2seq_n(mid, back, COUNT, P, B, s_lens, h_counts, D, CP_BF16,
                                        NULL) == CP_OK, "anything head2seq_n");
  expect(cp_kv_gather_n(in, gath, COUNT, P, B, s_lens, H, D, CP_BF16, NULL) == CP_OK,
         "kv_gather_n");
  CHECK_HIP(hipDeviceSynchronize());
  CHECK_HIP(hipMemcpy(hout, mid, COUNT * n * 2, hipMemcpyDeviceToHost));
  int perm_ok = 1;
  for (int t = 0; t < COUNT; ++t)
    for (int p = 0; p < P; ++p)
      for (int q = 0; q < P; ++q)
        for (int b = 0; b < B; ++b)
          for (int64_t s = 0; s < s_lens[q]; ++s)
            for (int64_t h = 0; h < h_counts[p]; ++h)
              for (int d = 0; d < D; ++d) {
                /* group p = [B][S][h_counts[p]][D] at B*S*h_off[p]*D; shard q =
                   [B][s_lens[q]][H][D] at B*s_off[q]*H*D */
                const size_t o = t * n + (size_t)(B * S * h_off[p] * D) +
                                 (size_t)(((b * S + s_off[q] + s) * h_counts[p] + h) * D + d);
                const size_t i = t * n + (size_t)(B * s_off[q] * H * D) +
                                 (size_t)(((b * s_lens[q] + s) * H + h_off[p] + h) * D + d);
                if (hout[o] != hin[i]) perm_ok = 0;
              }
  expect(perm_ok, "anything seq2head_n moves in_q[b][s][h0_p+h][d] to out_p[b][off_q+s][h][d]");
  CHECK_HIP(hipMemcpy(hout, back, COUNT * n * 2, hipMemcpyDeviceToHost));
  expect(memcmp(hout, hin, COUNT * n * 2) == 0, "anything head2seq_n(seq2head_n(x)) == x");
  CHECK_HIP(hipMemcpy(hout, gath, COUNT * n * 2, hipMemcpyDeviceToHost));
  int gather_ok = 1;
  for (int t = 0; t < COUNT; ++t)
    for (int q = 0; q < P; ++q)
      for (int b = 0; b < B; ++b)
        for (int64_t s = 0; s < s_lens[q]; ++s)
          for (int64_t h = 0; h < H; ++h)
            for (int d = 0; d < D; ++d) {
              const size_t o = t * n + (size_t)(((b * S + s_off[q] + s) * H + h) * D + d);
              const size_t i = t * n + (size_t)(B * s_off[q] * H * D) +
                               (size_t)(((b * s_lens[q] + s) * H + h) * D + d);
              if (hout[o] != hin[i]) gather_ok = 0;
            }
  expect(gather_ok, "kv_gather_n moves in_q[b][s][h][d] to out[b][off_q+s][h][d]");
  printf("ok: uneven regrouping and K/V gather of %d stacked tensors, s_lens {5,0,4}, "
         "h_counts {2,3,0}, bit for bit\n", COUNT);
  free(hin), free(hout);
  hipFree(in), hipFree(mid), hipFree(back), hipFree(gath);
}

/* --------------------------------------------------------------- backward */
static void check_backward(void) {
  enum { Sq = 70, Skv = 128, H = 2, D = 128 };
  const float scale = 0.0883883476f; /* 1/sqrt(128) */
  const size_t nq = (size_t)Sq * H * D, nk = (size_t)Skv * H * D;
  uint16_t* hq = calloc(nq, 2);
  uint16_t* hk = malloc(nk * 2);
  uint16_t* hv = malloc(nk * 2);
  uint16_t* hdo = malloc(nq * 2);
  for (size_t x = 0; x < nk; ++x) hk[x] = to_bf16(next_uniform());
  for (size_t x = 0; x < nk; ++x) hv[x] = to_bf16(next_uniform());
  for (size_t x = 0; x < nq; ++x) hdo[x] = to_bf16(next_uniform());
  /* saved statistics of the uniform forward: LSE = ln(128), Delta_i = <dO_i, mean v> */
  float* hl = malloc((size_t)H * Sq * 4);
  float* hdelta = malloc((size_t)H * Sq * 4);
  double* vbar = calloc((size_t)H * D, sizeof(double));
  for (int h = 0; h < H; ++h)
    for (int d = 0; d < D; ++d) {
      for (int j = 0; j < Skv; ++j) vbar[h * D + d] += from_bf16(hv[((size_t)j * H + h) * D + d]);
      vbar[h * D + d] /= Skv;
    }
  for (int h = 0; h < H; ++h)
    for (int i = 0; i < Sq; ++i) {
      double dl = 0.0;
      for (int d = 0; d < D; ++d) dl += from_bf16(hdo[((size_t)i * H + h) * D + d]) * vbar[h * D + d];
      hl[h * Sq + i] = (float)log((double)Skv);
      hdelta[h * Sq + i] = (float)dl;
    }
  void *q = dev_alloc(nq * 2), *k = dev_alloc(nk * 2), *v = dev_alloc(nk * 2),
       *dout = dev_alloc(nq * 2);
  float *lse = dev_alloc((size_t)H * Sq * 4), *delta = dev_alloc((size_t)H * Sq * 4);
  float *dq = dev_alloc(nq * 4), *dk = dev_alloc(nk * 4), *dv = dev_alloc(nk * 4);
  CHECK_HIP(hipMemcpy(q, hq, nq * 2, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(k, hk, nk * 2, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(v, hv, nk * 2, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(dout, hdo, nq * 2, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(lse, hl, (size_t)H * Sq * 4, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(delta, hdelta, (size_t)H * Sq * 4, hipMemcpyHostToDevice));
  cp_status st = cp_attn_chunk_backward(q, k, v, dout, lse, delta, dq, dk, dv, 1, H, Sq, Skv, D,
                                        CP_BF16, scale, 0, 0, 0, 0, NULL);
  expect(st == CP_OK, "cp_attn_chunk_backward returns CP_OK");
  CHECK_HIP(hipDeviceSynchronize());
  float* hdq = malloc(nq * 4);
  float* hdk = malloc(nk * 4);
  float* hdv = malloc(nk * 4);
  CHECK_HIP(hipMemcpy(hdq, dq, nq * 4, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(hdk, dk, nk * 4, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(hdv, dv, nk * 4, hipMemcpyDeviceToHost));
  double max_dk = 0.0, err_dv = 0.0, ref_dv = 0.0, err_dq = 0.0, ref_dq = 0.0;
  for (size_t x = 0; x < nk; ++x) max_dk = fmax(max_dk, fabs(hdk[x]));
  for (int h = 0; h < H; ++h)
    for (int d = 0; d < D; ++d) {
      double want = 0.0;
      for (int i = 0; i < Sq; ++i) want += from_bf16(hdo[((size_t)i * H + h) * D + d]);
      want /= Skv;
      ref_dv = fmax(ref_dv, fabs(want));
      for (int j = 0; j < Skv; ++j) err_dv = fmax(err_dv, fabs(hdv[((size_t)j * H + h) * D + d] - want));
    }
  for (int i = 0; i < Sq; ++i)
    for (int h = 0; h < H; ++h) {
      double ds[Skv];
      for (int j = 0; j < Skv; ++j) {
        double dp = 0.0;
        for (int d = 0; d < D; ++d)
          dp += from_bf16(hdo[((size_t)i * H + h) * D + d]) * from_bf16(hv[((size_t)j * H + h) * D + d]);
        ds[j] = (dp - hdelta[h * Sq + i]) / Skv;
      }
      for (int d = 0; d < D; ++d) {
        double want = 0.0;
        for (int j = 0; j < Skv; ++j) want += ds[j] * from_bf16(hk[((size_t)j * H + h) * D + d]);
        want *= scale;
        ref_dq = fmax(ref_dq, fabs(want));
        err_dq = fmax(err_dq, fabs(hdq[((size_t)i * H + h) * D + d] - want));
      }
    }
  expect(max_dk == 0.0, "dK = 0 when Q = 0");
  expect(err_dv <= 1e-2 * ref_dv + 1e-6, "dV = mean over rows of dO (uniform weights)");
  expect(err_dq <= 1e-2 * ref_dq + 1e-6, "dQ closed form");
  printf("ok: backward, max|dK| %.1e, dV max-abs %.2e (ref %.2e), dQ max-abs %.2e (ref %.2e)\n",
         max_dk, err_dv, ref_dv, err_dq, ref_dq);
  free(hq), free(hk), free(hv), free(hdo), free(hl), free(hdelta), free(vbar);
  free(hdq), free(hdk), free(hdv);
  hipFree(q), hipFree(k), hipFree(v), hipFree(dout), hipFree(lse), hipFree(delta);
  hipFree(dq), hipFree(dk), hipFree(dv);
}

int main(void) {
  printf("libcpattn ABI version %d\n", cp_abi_version());
  check_forward();
  check_relayout();
  check_uneven_relayout();
  check_backward();
  if (failures) {
    fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  printf("all C ABI checks passed\n");
  return 0;
}
