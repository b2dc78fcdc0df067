/* Drives every entry point of the CPU oracle on small inputs held in
 * exact-size heap buffers, for a build under AddressSanitizer and
 * UndefinedBehaviorSanitizer: an out-of-bounds access, a use after free or an
 * undefined operation (signed overflow, bad shift, misaligned load) aborts
 * the run.  Values are not checked here; the oracle's pins do that.  Also
 * checks that malformed arguments are rejected with a nonzero code.
 * Prints "oracle checks ok" and exits 0 on success. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "coli_oracle.h"

static uint64_t rng = 0x9E3779B97F4A7C15ull;
static float frand(void) { /* xorshift64*, uniform in [-1, 1) */
  rng ^= rng >> 12; rng ^= rng << 25; rng ^= rng >> 27;
  return (float)((double)((rng * 2685821657736338717ull) >> 11) / 9007199254740992.0 * 2.0 - 1.0);
}

static void *xmalloc(size_t n) {
  void *p = malloc(n ? n : 1);
  if (!p) { fprintf(stderr, "out of memory\n"); exit(2); }
  return p;
}

static float *frandv(size_t n, float scale) {
  float *p = xmalloc(n * sizeof(float));
  for (size_t i = 0; i < n; ++i) p[i] = scale * frand();
  return p;
}

#define CHECK(cond) do { if (!(cond)) { fprintf(stderr, "check failed: %s (line %d)\n", #cond, __LINE__); exit(1); } } while (0)

typedef struct { uint8_t *w; float *s; } packed_t;

static packed_t pack_rand(int bits, int64_t rows, int64_t cols) {
  packed_t p;
  float *w = frandv((size_t)(rows * cols), 0.05f);
  p.w = xmalloc((size_t)(rows * cols * bits / 8));
  p.s = xmalloc((size_t)rows * sizeof(float));
  CHECK(orc_quant_pack(bits, w, rows, cols, p.w, p.s) == 0);
  free(w);
  return p;
}

static void quant_and_pack(int bits) {
  const int64_t rows = 5, cols = 96;
  float *w = frandv(rows * cols, 1.0f);
  for (int64_t c = 0; c < cols; ++c) w[2 * cols + c] = 0.0f; /* an all-zero row */
  int8_t *codes = xmalloc(rows * cols), *back = xmalloc(rows * cols);
  float *s = xmalloc(rows * sizeof(float));
  uint8_t *pk = xmalloc(rows * cols * bits / 8);
  CHECK(orc_quant_rows(bits, w, rows, cols, codes, s) == 0);
  CHECK(orc_pack(bits, codes, rows, cols, pk) == 0);
  CHECK(orc_unpack(bits, pk, rows, cols, back) == 0);
  CHECK(memcmp(codes, back, rows * cols) == 0);
  CHECK(orc_quant_pack(bits, w, rows, cols, pk, s) == 0);
  CHECK(orc_quant_rows(bits, w, 0, cols, codes, s) == 0); /* no rows */
  CHECK(orc_quant_rows(3, w, rows, cols, codes, s) != 0);
  CHECK(orc_pack(bits, codes, rows, 0, pk) != 0);
  CHECK(orc_quant_pack(bits, NULL, rows, cols, pk, s) != 0);
  free(w); free(codes); free(back); free(s); free(pk);
}

static void products(int bits) {
  const int64_t rows = 7, cols = 128, T = 3;
  packed_t W = pack_rand(bits, rows, cols);
  float *x = frandv(T * cols, 2.0f);
  int8_t *xq = xmalloc(T * cols);
  float *xd = xmalloc(T * (cols / 32) * sizeof(float));
  int32_t *acc = xmalloc(T * rows * (cols / 32) * sizeof(int32_t));
  float *y = xmalloc(T * rows * sizeof(float));
  CHECK(orc_q8_0(x, T, cols, xq, xd) == 0);
  CHECK(orc_q8_0(x, 0, cols, xq, xd) == 0);
  CHECK(orc_q8_0(x, T, 40, xq, xd) != 0); /* not a whole number of blocks */
  CHECK(orc_qdot(bits, W.w, W.s, rows, cols, xq, xd, T, acc, y) == 0);
  CHECK(orc_qdot(bits, W.w, W.s, rows, cols, xq, xd, T, NULL, y) == 0);
  CHECK(orc_qdot(bits, W.w, W.s, rows, cols, xq, xd, T, acc, NULL) == 0);
  CHECK(orc_qdot(bits, W.w, W.s, rows, 48, xq, xd, T, acc, y) != 0);
  CHECK(orc_qdot_f32act(bits, W.w, W.s, rows, cols, x, T, y) == 0);
  CHECK(orc_qdot_f32act(bits, W.w, W.s, rows, cols, x, 0, y) == 0);
  free(W.w); free(W.s); free(x); free(xq); free(xd); free(acc); free(y);
}

static void logits_and_route(void) {
  const int64_t T = 4, E = 16, H = 64;
  float *x = frandv(T * H, 1.0f), *gw = frandv(E * H, 0.2f), *bias = frandv(E, 0.01f);
  float *lg = xmalloc(T * E * sizeof(float)), *sig = xmalloc(T * E * sizeof(float));
  CHECK(orc_logits(x, gw, T, E, H, lg) == 0);
  CHECK(orc_logits(x, gw, T, 0, H, lg) != 0);
  for (int variant = 0; variant < 4; ++variant) {
    orc_router_cfg c = {(int32_t)E, 4, 4, 2, 1, 2.5f, 0.0f, 1};
    if (variant == 1) { c.top_p = 0.7f; c.top_p_renorm = 1; }
    if (variant == 2) { c.top_p = 0.5f; c.top_p_renorm = 0; c.norm_topk_prob = 0; }
    if (variant == 3) { c.n_group = 1; c.topk_group = 1; c.top_k = 8; }
    int32_t *idx = xmalloc(T * c.top_k * sizeof(int32_t));
    float *w = xmalloc(T * c.top_k * sizeof(float));
    CHECK(orc_route(&c, lg, variant & 1 ? NULL : bias, T, idx, w, variant ? NULL : sig) == 0);
    CHECK(orc_route(&c, lg, bias, 0, idx, w, NULL) == 0);
    free(idx); free(w);
  }
  orc_router_cfg bad = {(int32_t)E, 4, 5, 2, 1, 2.5f, 0.0f, 1}; /* E % n_group != 0 */
  int32_t idx1[16]; float w1[16];
  CHECK(orc_route(&bad, lg, bias, 1, idx1, w1, NULL) != 0);
  free(x); free(gw); free(bias); free(lg); free(sig);
}

static void expert_and_layer(int bits) {
  const int32_t H = 64, I = 96, E = 16, k = 4;
  const int64_t T = 5;
  packed_t g[17], u[17], d[17];
  for (int e = 0; e <= E; ++e) {
    g[e] = pack_rand(bits, I, H);
    u[e] = pack_rand(bits, I, H);
    d[e] = pack_rand(bits, H, I);
  }
  float *x = frandv(T * H, 1.0f), *o = xmalloc(T * H * sizeof(float));
  float *h = xmalloc(T * I * sizeof(float));
  CHECK(orc_expert_ffn(bits, H, I, g[0].w, g[0].s, u[0].w, u[0].s, d[0].w, d[0].s, x, T, o, h) == 0);
  CHECK(orc_expert_ffn(bits, H, I, g[0].w, g[0].s, u[0].w, u[0].s, d[0].w, d[0].s, x, T, o, NULL) == 0);
  CHECK(orc_expert_ffn(bits, H, I, g[0].w, g[0].s, u[0].w, u[0].s, d[0].w, d[0].s, x, 0, o, NULL) == 0);
  CHECK(orc_expert_ffn(bits, 40, I, g[0].w, g[0].s, u[0].w, u[0].s, d[0].w, d[0].s, x, T, o, NULL) != 0);

  const uint8_t *wg[16], *wu[16], *wd[16];
  const float *sg[16], *su[16], *sd[16];
  for (int e = 0; e < E; ++e) {
    wg[e] = g[e].w; wu[e] = u[e].w; wd[e] = d[e].w;
    sg[e] = g[e].s; su[e] = u[e].s; sd[e] = d[e].s;
  }
  float *gw = frandv(E * H, 0.2f), *bias = frandv(E, 0.01f);
  orc_layer L;
  memset(&L, 0, sizeof L);
  L.hidden = H; L.inter = I; L.bits = bits;
  L.router = (orc_router_cfg){E, k, 4, 2, 1, 2.5f, 0.0f, 1};
  L.gate_w = gw; L.gate_bias = bias;
  L.w_gate = wg; L.s_gate = sg; L.w_up = wu; L.s_up = su; L.w_down = wd; L.s_down = sd;
  L.sh_gate = g[E].w; L.sh_up = u[E].w; L.sh_down = d[E].w;
  L.sh_s_gate = g[E].s; L.sh_s_up = u[E].s; L.sh_s_down = d[E].s;
  float *y = xmalloc(T * H * sizeof(float)), *w = xmalloc(T * k * sizeof(float));
  float *lg = xmalloc(T * E * sizeof(float));
  int32_t *idx = xmalloc(T * k * sizeof(int32_t));
  CHECK(orc_moe_forward(&L, x, T, NULL, y, idx, w, lg) == 0);
  CHECK(orc_moe_forward(&L, x, T, lg, y, NULL, NULL, NULL) == 0);
  CHECK(orc_moe_forward(&L, x, 0, NULL, y, NULL, NULL, NULL) == 0);
  L.router.top_p = 0.6f;
  CHECK(orc_moe_forward(&L, x, T, NULL, y, idx, w, lg) == 0);
  /* a selected expert with no tensors is an error */
  for (int64_t j = 0; j < T * k; ++j)
    if (idx[j] >= 0) { wg[idx[j]] = NULL; break; }
  CHECK(orc_moe_forward(&L, x, T, NULL, y, NULL, NULL, NULL) != 0);

  int32_t counts[16], offs[17], perm[5 * 4], uniq[16], n_uniq = 0;
  idx[1] = -1;
  CHECK(orc_union_tables(idx, T, k, E, counts, offs, perm, uniq, &n_uniq) == 0);
  CHECK(n_uniq >= 1 && n_uniq <= E && offs[E] <= T * k);
  idx[0] = E; /* out of range */
  CHECK(orc_union_tables(idx, T, k, E, counts, offs, perm, uniq, &n_uniq) != 0);

  for (int e = 0; e <= E; ++e) {
    free(g[e].w); free(g[e].s); free(u[e].w); free(u[e].s); free(d[e].w); free(d[e].s);
  }
  free(x); free(o); free(h); free(gw); free(bias); free(y); free(w); free(lg); free(idx);
}

static void fp8(void) {
  const int64_t rows = 130, cols = 200; /* ragged 128-blocks both ways */
  uint8_t *w8 = xmalloc(rows * cols);
  for (int64_t i = 0; i < rows * cols; ++i) w8[i] = (uint8_t)(i * 37);
  const int64_t br = (rows + 127) / 128, bc = (cols + 127) / 128;
  float *bs = frandv(br * bc, 1.0f);
  float *out = xmalloc(rows * cols * sizeof(float));
  CHECK(orc_dequant_fp8_block(w8, bs, rows, cols, out) == 0);
  CHECK(orc_dequant_fp8_block(w8, bs, rows, 0, out) != 0);
  for (int c = 0; c < 256; ++c) (void)orc_e4m3_value((uint8_t)c);
  free(w8); free(bs); free(out);
}

int main(void) {
  orc_set_num_threads(2);
  CHECK(orc_num_threads() == 2);
  const int bits[3] = {8, 4, 2};
  for (int i = 0; i < 3; ++i) {
    quant_and_pack(bits[i]);
    products(bits[i]);
    expert_and_layer(bits[i]);
  }
  logits_and_route();
  fp8();
  CHECK(orc_qmax(3) < 0);
  printf("oracle checks ok\n");
  return 0;
}
