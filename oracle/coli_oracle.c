/*
 * coli_oracle.c -- the CPU oracle for colibrì's routed-expert MoE layer.
 *
 * TEST INFRASTRUCTURE ONLY (see coli_oracle.h): plain loops, no SIMD
 * intrinsics, no BLAS, no -ffast-math, no FMA contraction.  OpenMP, where
 * used, only splits independent output rows or tokens, so results do not
 * depend on the thread count.
 *
 * The layer (colibrì README, "Implemented features": DeepSeek-V3-like
 * sigmoid router with noaux_tc and routed_scaling_factor, a shared expert;
 * integer dot-product kernels against Q8_0-style int8 activations; int8 /
 * packed int4 / packed int2 quantised kernels with one scale per row,
 * dequantised on use; batch-union MoE that reads each unique expert of a
 * batch once).  The SwiGLU expert form and the group-limited top-k
 * parameters are not spelled out on the pages beyond "DeepSeek-V3-like"; the
 * readings taken are stated at each function.
 *
 * Parity unpinned (no value on the pages to check against): the exact
 * weight-quantisation rule (symmetric absmax, qmax = 2^(b-1)-1, ternary
 * int2), the Q8_0 scale kept in fp32, the group score (sum of the two best
 * biased scores) and expert top-p renormalisation.  These are this oracle's
 * readings; tests pin that the code computes them, not that colibrì does.
 */
#include "coli_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int orc_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Every parallel loop of the oracle splits independent rows or experts, so
 * the thread count changes its speed, never its results. */
void orc_set_num_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

int orc_qmax(int bits) {
  switch (bits) {
    case 8: return 127;
    case 4: return 7;
    case 2: return 1;
    default: return -1;
  }
}

/* Round to nearest, ties to even, in binary32 (the default rounding mode). */
static float round_even_f32(float v) { return rintf(v); }

static float clamp_code(float v, int qmax) {
  if (v > (float)qmax) return (float)qmax;
  if (v < -(float)qmax) return -(float)qmax;
  return v;
}

/*
 * O1 -- weight quantisation with one scale per row (colibrì README,
 * "Implemented features", quantised kernels: int8 / int4 / int2 with a
 * per-row scale; CSDN feature, "pure C" section, same list).
 * Reading: symmetric absmax.  qmax = 2^(b-1)-1; s = amax/qmax in binary32;
 * q = clamp(round_half_even(w/s), -qmax, qmax) with w/s in binary32; a row
 * whose s is zero gets q = 0.  int2 is therefore ternary {-1, 0, 1}.
 */
int orc_quant_rows(int bits, const float *w, int64_t rows, int64_t cols,
                   int8_t *codes, float *scales) {
  int qmax = orc_qmax(bits);
  if (qmax < 0 || rows < 0 || cols <= 0 || !w || !codes || !scales)
    return ORC_EINVAL;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    const float *wr = w + r * cols;
    float amax = 0.0f;
    for (int64_t c = 0; c < cols; ++c) {
      float a = fabsf(wr[c]);
      if (a > amax) amax = a;
    }
    float s = amax / (float)qmax;
    scales[r] = s;
    for (int64_t c = 0; c < cols; ++c) {
      float q = 0.0f;
      if (s != 0.0f) q = clamp_code(round_even_f32(wr[c] / s), qmax);
      codes[r * cols + c] = (int8_t)q;
    }
  }
  return ORC_OK;
}

/*
 * O2 -- packing (colibrì README, "Implemented features": packed int4 and
 * int2, checked bit-identical to the int8 container).
 * Reading: row-major, row stride cols*b/8 bytes, lowest bits first.  int8:
 * the byte is the code.  int4: byte j holds element 2j in bits 0-3 and
 * element 2j+1 in bits 4-7.  int2: byte j holds element 4j+m in bits
 * 2m..2m+1.  Fields are two's complement; unpacking sign-extends.
 */
int orc_pack(int bits, const int8_t *codes, int64_t rows, int64_t cols,
             uint8_t *packed) {
  if (orc_qmax(bits) < 0 || rows < 0 || cols <= 0 || (cols * bits) % 8 ||
      !codes || !packed)
    return ORC_EINVAL;
  const int per = 8 / bits;            /* elements per byte */
  const int64_t stride = cols * bits / 8;
  const unsigned mask = (1u << bits) - 1u;
  for (int64_t r = 0; r < rows; ++r) {
    for (int64_t j = 0; j < stride; ++j) {
      unsigned byte = 0;
      for (int m = 0; m < per; ++m) {
        unsigned field = (unsigned)(uint8_t)codes[r * cols + j * per + m] & mask;
        byte |= field << (bits * m);
      }
      packed[r * stride + j] = (uint8_t)byte;
    }
  }
  return ORC_OK;
}

int orc_unpack(int bits, const uint8_t *packed, int64_t rows, int64_t cols,
               int8_t *codes) {
  if (orc_qmax(bits) < 0 || rows < 0 || cols <= 0 || (cols * bits) % 8 ||
      !codes || !packed)
    return ORC_EINVAL;
  const int per = 8 / bits;
  const int64_t stride = cols * bits / 8;
  const int mask = (1 << bits) - 1;
  const int sign = 1 << (bits - 1);
  for (int64_t r = 0; r < rows; ++r) {
    for (int64_t c = 0; c < cols; ++c) {
      int byte = packed[r * stride + c / per];
      int field = (byte >> (bits * (int)(c % per))) & mask;
      int v = (field & sign) ? field - (1 << bits) : field;
      codes[r * cols + c] = (int8_t)v;
    }
  }
  return ORC_OK;
}

int orc_quant_pack(int bits, const float *w, int64_t rows, int64_t cols,
                   uint8_t *packed, float *scales) {
  if (orc_qmax(bits) < 0 || rows < 0 || cols <= 0 || (cols * bits) % 8)
    return ORC_EINVAL;
  int8_t *codes = (int8_t *)malloc((size_t)(rows * cols > 0 ? rows * cols : 1));
  if (!codes) return ORC_EINVAL;
  int rc = orc_quant_rows(bits, w, rows, cols, codes, scales);
  if (rc == ORC_OK) rc = orc_pack(bits, codes, rows, cols, packed);
  free(codes);
  return rc;
}

/*
 * O11 -- FP8 checkpoint dequantisation (colibrì README, "Implemented
 * features": the offline FP8 -> int4 converter dequantises the checkpoint's
 * 128x128 block-scaled FP8 weights and requantises them into the engine's
 * container; with O1 + O2 that is the converter's arithmetic).
 * Reading: the FP8 format is OCP E4M3 with no infinities ("e4m3fn"): bit 7
 * the sign, bits 6..3 the exponent field e (bias 7), bits 2..0 the mantissa
 * field m.  e = 0: the subnormal m/8 * 2^-6; e = 15 with m = 7: NaN;
 * otherwise (1 + m/8) * 2^(e-7).  A block's scale multiplies every value of
 * its 128x128 tile (blocks start at row 0 and column 0; edge blocks are
 * partial).  The binary64 product of two binary32 numbers is exact, so
 * rounding it once gives the binary32 product.
 */
float orc_e4m3_value(uint8_t code) {
  const int sign = code >> 7, e = (code >> 3) & 15, m = code & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0) v = ldexp((double)m / 8.0, -6);
  else v = ldexp(1.0 + (double)m / 8.0, e - 7);
  return (float)(sign ? -v : v);
}

int orc_dequant_fp8_block(const uint8_t *w8, const float *block_scale, int64_t rows,
                          int64_t cols, float *out) {
  if (rows < 0 || cols <= 0 || !w8 || !block_scale || !out) return ORC_EINVAL;
  const int64_t nbc = (cols + 127) / 128;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    for (int64_t c = 0; c < cols; ++c) {
      const double v = (double)orc_e4m3_value(w8[r * cols + c]);
      const double s = (double)block_scale[(r / 128) * nbc + c / 128];
      out[r * cols + c] = (float)(v * s);
    }
  }
  return ORC_OK;
}

/*
 * O12 -- the f32-activation variant of the quantised product (colibrì
 * README, "Implemented features": for a single row the int4 kernel keeps
 * its activations in f32, measured faster there than the integer path).
 * Reading: the weight row is dequantised on use (code times the row scale)
 * against unquantised binary32 activations: y = fl32( s_r * sum_c code*x ),
 * the sum over c in increasing order and the product with s_r in binary64,
 * rounded to binary32 once.
 */
int orc_qdot_f32act(int bits, const uint8_t *w_packed, const float *w_scale,
                    int64_t rows, int64_t cols, const float *x, int64_t T, float *y) {
  if (orc_qmax(bits) < 0 || rows < 0 || cols <= 0 || (cols * bits) % 8 || T < 0 ||
      !w_packed || !w_scale || !x || !y)
    return ORC_EINVAL;
  const int64_t stride = cols * bits / 8;
  int rc = ORC_OK;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    int8_t *wrow = (int8_t *)malloc((size_t)cols);
    if (!wrow) { rc = ORC_EINVAL; continue; }
    orc_unpack(bits, w_packed + r * stride, 1, cols, wrow);
    for (int64_t t = 0; t < T; ++t) {
      double sum = 0.0;
      for (int64_t c = 0; c < cols; ++c) sum += (double)wrow[c] * (double)x[t * cols + c];
      y[t * rows + r] = (float)((double)w_scale[r] * sum);
    }
    free(wrow);
  }
  return rc;
}

/*
 * O3 -- Q8_0-style activation quantisation (colibrì README, "Implemented
 * features", integer dot-product kernels).
 * Reading: blocks of 32 consecutive values along the row starting at column
 * 0; d = amax/127 in binary32; q = clamp(round_half_even(x/d), -127, 127)
 * with x/d in binary32; a block whose d is zero gets q = 0.  d is kept as an
 * fp32 number (the "-style" leaves the storage type open).
 */
int orc_q8_0(const float *x, int64_t T, int64_t n, int8_t *q, float *d) {
  if (T < 0 || n <= 0 || n % 32 || !x || !q || !d) return ORC_EINVAL;
  const int64_t nb = n / 32;
  for (int64_t t = 0; t < T; ++t) {
    for (int64_t b = 0; b < nb; ++b) {
      const float *xb = x + t * n + b * 32;
      float amax = 0.0f;
      for (int i = 0; i < 32; ++i) {
        float a = fabsf(xb[i]);
        if (a > amax) amax = a;
      }
      float db = amax / 127.0f;
      d[t * nb + b] = db;
      for (int i = 0; i < 32; ++i) {
        float v = 0.0f;
        if (db != 0.0f) v = clamp_code(round_even_f32(xb[i] / db), 127);
        q[t * n + b * 32 + i] = (int8_t)v;
      }
    }
  }
  return ORC_OK;
}

/*
 * O4 -- quantised product (colibrì README, "Implemented features": integer
 * dot products of int8 activations with int8 / int4 / int2 weights, each row
 * dequantised on use with its scale).
 * Reading: per block b of 32, acc = sum of code products as an exact int32;
 * y = fl32( sum_b  s_r * d_b * acc_b ) with every product and the running
 * sum in binary64, blocks in increasing order, rounded to binary32 once.
 */
int orc_qdot(int bits, const uint8_t *w_packed, const float *w_scale,
             int64_t rows, int64_t cols, const int8_t *xq, const float *xd,
             int64_t T, int32_t *acc, float *y) {
  if (orc_qmax(bits) < 0 || rows < 0 || cols <= 0 || cols % 32 || T < 0 ||
      !w_packed || !w_scale || !xq || !xd)
    return ORC_EINVAL;
  const int64_t nb = cols / 32;
  const int64_t stride = cols * bits / 8;
  int rc = ORC_OK;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    int8_t *wrow = (int8_t *)malloc((size_t)cols);
    if (!wrow) { rc = ORC_EINVAL; continue; }
    orc_unpack(bits, w_packed + r * stride, 1, cols, wrow);
    for (int64_t t = 0; t < T; ++t) {
      const int8_t *xr = xq + t * cols;
      double sum = 0.0;
      for (int64_t b = 0; b < nb; ++b) {
        int32_t a = 0;
        for (int i = 0; i < 32; ++i)
          a += (int32_t)wrow[b * 32 + i] * (int32_t)xr[b * 32 + i];
        if (acc) acc[(t * rows + r) * nb + b] = a;
        sum += (double)w_scale[r] * (double)xd[t * nb + b] * (double)a;
      }
      if (y) y[t * rows + r] = (float)sum;
    }
    free(wrow);
  }
  return rc;
}

/*
 * O5 -- router logits (colibrì README, "Implemented features": the
 * DeepSeek-V3-like router).  Reading: the gate matrix is fp32 [E][H];
 * l = fl32 of the binary64 dot product taken in increasing i.
 */
int orc_logits(const float *x, const float *gate_w, int64_t T, int64_t E,
               int64_t H, float *logits) {
  if (!x || !gate_w || !logits || T < 0 || E <= 0 || H <= 0) return ORC_EINVAL;
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t) {
    for (int64_t e = 0; e < E; ++e) {
      double s = 0.0;
      for (int64_t i = 0; i < H; ++i)
        s += (double)x[t * H + i] * (double)gate_w[e * H + i];
      logits[t * E + e] = (float)s;
    }
  }
  return ORC_OK;
}

static int router_cfg_ok(const orc_router_cfg *c) {
  if (!c) return 0;
  if (c->n_experts <= 0 || c->top_k <= 0 || c->n_group <= 0) return 0;
  if (c->n_experts % c->n_group) return 0;
  if (c->topk_group <= 0 || c->topk_group > c->n_group) return 0;
  if (c->top_k > c->topk_group * (c->n_experts / c->n_group)) return 0;
  return 1;
}

/* Sigmoid in binary64, rounded once to binary32. */
static float sigmoid_f32(float l) {
  return (float)(1.0 / (1.0 + exp(-(double)l)));
}

/*
 * O6 + O7 -- the router (colibrì README, "Implemented features":
 * DeepSeek-V3-like sigmoid router, noaux_tc, routed_scaling_factor; README
 * "Quick start" knobs: adaptive expert top-p).
 * Readings:
 *  - sigma_e = fl32(1/(1+exp(-l_e))) in binary64;
 *  - noaux_tc: the bias only steers selection: c_e = sigma_e + bias_e (fp32);
 *    the weights use the unbiased sigma;
 *  - groups are contiguous runs of E/n_group experts; a group's score is the
 *    fp32 sum of its two largest c (its only c if the group has one expert);
 *  - the topk_group best groups are kept (score descending, lower group
 *    index first on ties); among their experts the top_k best c are chosen
 *    (c descending, lower expert index first on ties) -- this is the rank
 *    order of the output slots;
 *  - S = fp32 sum of the chosen sigma in rank order; w_j = (sigma_j/S)*rsf
 *    (each step binary32) when norm_topk_prob, else sigma_j*rsf; S = 0 gives
 *    zero weights;
 *  - expert top-p (only for 0 < p < 1): on the normalised p_j = sigma_j/S,
 *    visit slots by p descending (rank order on ties) adding p_j to an fp32
 *    running sum; keep the shortest such prefix whose sum reaches p (at least
 *    one slot); the other slots get idx -1 and w 0.  With renormalisation the
 *    kept weights become (sigma_j/S_kept)*rsf, S_kept summed over kept slots
 *    in rank order; without it they are left as above.
 */
int orc_route(const orc_router_cfg *cfg, const float *logits,
              const float *bias, int64_t T, int32_t *idx, float *w,
              float *sigma_out) {
  if (!router_cfg_ok(cfg) || !logits || !idx || !w || T < 0) return ORC_EINVAL;
  const int E = cfg->n_experts, k = cfg->top_k, G = cfg->n_group;
  const int per = E / G;
  float *sig = (float *)malloc(sizeof(float) * (size_t)E);
  float *c = (float *)malloc(sizeof(float) * (size_t)E);
  float *gs = (float *)malloc(sizeof(float) * (size_t)G);
  char *gkeep = (char *)malloc((size_t)G);
  char *taken = (char *)malloc((size_t)E);
  if (!sig || !c || !gs || !gkeep || !taken) {
    free(sig); free(c); free(gs); free(gkeep); free(taken);
    return ORC_EINVAL;
  }
  for (int64_t t = 0; t < T; ++t) {
    const float *lt = logits + t * E;
    for (int e = 0; e < E; ++e) {
      sig[e] = sigmoid_f32(lt[e]);
      c[e] = sig[e] + (bias ? bias[e] : 0.0f);
      if (sigma_out) sigma_out[t * E + e] = sig[e];
    }
    /* group scores */
    for (int g = 0; g < G; ++g) {
      int b1 = -1, b2 = -1;
      for (int e = g * per; e < (g + 1) * per; ++e) {
        if (b1 < 0 || c[e] > c[b1]) { b2 = b1; b1 = e; }
        else if (b2 < 0 || c[e] > c[b2]) { b2 = e; }
      }
      gs[g] = (per >= 2) ? c[b1] + c[b2] : c[b1];
      gkeep[g] = 0;
    }
    /* keep topk_group groups */
    for (int n = 0; n < cfg->topk_group; ++n) {
      int best = -1;
      for (int g = 0; g < G; ++g)
        if (!gkeep[g] && (best < 0 || gs[g] > gs[best])) best = g;
      gkeep[best] = 1;
    }
    /* top_k experts among the kept groups, in rank order */
    memset(taken, 0, (size_t)E);
    int32_t *it = idx + t * k;
    float *wt = w + t * k;
    for (int j = 0; j < k; ++j) {
      int best = -1;
      for (int e = 0; e < E; ++e) {
        if (!gkeep[e / per] || taken[e]) continue;
        if (best < 0 || c[e] > c[best]) best = e;
      }
      taken[best] = 1;
      it[j] = best;
    }
    /* weights */
    float S = 0.0f;
    for (int j = 0; j < k; ++j) S += sig[it[j]];
    for (int j = 0; j < k; ++j) {
      float v;
      if (cfg->norm_topk_prob)
        v = (S != 0.0f) ? (sig[it[j]] / S) * cfg->routed_scaling_factor : 0.0f;
      else
        v = sig[it[j]] * cfg->routed_scaling_factor;
      wt[j] = v;
    }
    /* expert top-p */
    if (cfg->top_p > 0.0f && cfg->top_p < 1.0f) {
      float pn[64];
      char keep[64], seen[64];
      if (k > 64) { free(sig); free(c); free(gs); free(gkeep); free(taken); return ORC_EINVAL; }
      for (int j = 0; j < k; ++j) {
        pn[j] = (S != 0.0f) ? sig[it[j]] / S : 0.0f;
        keep[j] = 0; seen[j] = 0;
      }
      float cum = 0.0f;
      for (int n = 0; n < k; ++n) {
        int best = -1;
        for (int j = 0; j < k; ++j)
          if (!seen[j] && (best < 0 || pn[j] > pn[best])) best = j;
        seen[best] = 1;
        keep[best] = 1;
        cum += pn[best];
        if (cum >= cfg->top_p) break;
      }
      float Sk = 0.0f;
      for (int j = 0; j < k; ++j)
        if (keep[j]) Sk += sig[it[j]];
      for (int j = 0; j < k; ++j) {
        if (!keep[j]) { it[j] = -1; wt[j] = 0.0f; continue; }
        if (cfg->top_p_renorm)
          wt[j] = (Sk != 0.0f) ? (sig[it[j]] / Sk) * cfg->routed_scaling_factor : 0.0f;
      }
    }
  }
  free(sig); free(c); free(gs); free(gkeep); free(taken);
  return ORC_OK;
}

/*
 * O8 -- one expert (colibrì README, "Implemented features": DeepSeek-V3-like
 * MoE whose expert matmuls run against Q8_0-style int8 activations).
 * Reading: SwiGLU, o = down( silu(gate.x) * up.x ) with no clamp; both
 * expert inputs (x and the intermediate h) are Q8_0-quantised; g and u are
 * O4 results (fp32); h = fl32(silu(g)*u) with silu(z) = z/(1+exp(-z)) and the
 * product in binary64.
 */
int orc_expert_ffn(int bits, int64_t H, int64_t I,
                   const uint8_t *wg, const float *sg,
                   const uint8_t *wu, const float *su,
                   const uint8_t *wd, const float *sd,
                   const float *x, int64_t T, float *o, float *h_out) {
  if (orc_qmax(bits) < 0 || H <= 0 || I <= 0 || H % 32 || I % 32 || T < 0 ||
      !wg || !sg || !wu || !su || !wd || !sd || !x || !o)
    return ORC_EINVAL;
  if (T == 0) return ORC_OK;
  int8_t *xq = (int8_t *)malloc((size_t)(T * H));
  float *xd = (float *)malloc(sizeof(float) * (size_t)(T * H / 32));
  float *g = (float *)malloc(sizeof(float) * (size_t)(T * I));
  float *u = (float *)malloc(sizeof(float) * (size_t)(T * I));
  float *h = (float *)malloc(sizeof(float) * (size_t)(T * I));
  int8_t *hq = (int8_t *)malloc((size_t)(T * I));
  float *hd = (float *)malloc(sizeof(float) * (size_t)(T * I / 32));
  int rc = ORC_EINVAL;
  if (xq && xd && g && u && h && hq && hd) {
    rc = orc_q8_0(x, T, H, xq, xd);
    if (!rc) rc = orc_qdot(bits, wg, sg, I, H, xq, xd, T, NULL, g);
    if (!rc) rc = orc_qdot(bits, wu, su, I, H, xq, xd, T, NULL, u);
    if (!rc) {
      for (int64_t i = 0; i < T * I; ++i) {
        double gd = (double)g[i];
        double silu = gd / (1.0 + exp(-gd));
        h[i] = (float)(silu * (double)u[i]);
      }
      if (h_out) memcpy(h_out, h, sizeof(float) * (size_t)(T * I));
      rc = orc_q8_0(h, T, I, hq, hd);
    }
    if (!rc) rc = orc_qdot(bits, wd, sd, H, I, hq, hd, T, NULL, o);
  }
  free(xq); free(xd); free(g); free(u); free(h); free(hq); free(hd);
  return rc;
}

/*
 * O9 -- the layer (colibrì README, "Implemented features": the router picks
 * experts, the shared expert always runs, and the batch-union MoE applies
 * each expert to every position routed to it -- a regrouping of the
 * per-token result, so the oracle computes each token on its own).
 * Reading: y_t = fl32( o_shared + sum over kept slots j in rank order of
 * w_j * o_{idx_j} ) in binary64; the shared expert has weight 1; no residual
 * and no normalisation belong to the layer.
 */
int orc_moe_forward(const orc_layer *L, const float *x, int64_t T,
                    const float *logits_in, float *y, int32_t *idx_out,
                    float *w_out, float *logits_out) {
  if (!L || !x || !y || T < 0 || !router_cfg_ok(&L->router)) return ORC_EINVAL;
  const int64_t H = L->hidden, I = L->inter;
  const int E = L->router.n_experts, k = L->router.top_k;
  if (H <= 0 || I <= 0 || orc_qmax(L->bits) < 0) return ORC_EINVAL;
  if (!logits_in && !L->gate_w) return ORC_EINVAL;
  if (!L->sh_gate || !L->sh_up || !L->sh_down || !L->sh_s_gate ||
      !L->sh_s_up || !L->sh_s_down || !L->w_gate || !L->w_up || !L->w_down ||
      !L->s_gate || !L->s_up || !L->s_down)
    return ORC_EINVAL;
  if (T == 0) return ORC_OK;

  float *lg = (float *)malloc(sizeof(float) * (size_t)(T * E));
  int32_t *idx = (int32_t *)malloc(sizeof(int32_t) * (size_t)(T * k));
  float *w = (float *)malloc(sizeof(float) * (size_t)(T * k));
  if (!lg || !idx || !w) { free(lg); free(idx); free(w); return ORC_EINVAL; }
  int rc = ORC_OK;
  if (logits_in) memcpy(lg, logits_in, sizeof(float) * (size_t)(T * E));
  else rc = orc_logits(x, L->gate_w, T, E, H, lg);
  if (!rc) rc = orc_route(&L->router, lg, L->gate_bias, T, idx, w, NULL);
  /* every selected expert must be present */
  for (int64_t i = 0; !rc && i < T * k; ++i) {
    int e = idx[i];
    if (e < 0) continue;
    if (!L->w_gate[e] || !L->w_up[e] || !L->w_down[e] || !L->s_gate[e] ||
        !L->s_up[e] || !L->s_down[e])
      rc = ORC_EINVAL;
  }
  float *osh = (float *)malloc(sizeof(float) * (size_t)H);
  float *oe = (float *)malloc(sizeof(float) * (size_t)(k * H));
  if (!osh || !oe) rc = ORC_EINVAL;
  for (int64_t t = 0; !rc && t < T; ++t) {
    const float *xt = x + t * H;
    rc = orc_expert_ffn(L->bits, H, I, L->sh_gate, L->sh_s_gate, L->sh_up,
                        L->sh_s_up, L->sh_down, L->sh_s_down, xt, 1, osh, NULL);
    for (int j = 0; !rc && j < k; ++j) {
      int e = idx[t * k + j];
      if (e < 0) continue;
      rc = orc_expert_ffn(L->bits, H, I, L->w_gate[e], L->s_gate[e],
                          L->w_up[e], L->s_up[e], L->w_down[e], L->s_down[e],
                          xt, 1, oe + j * H, NULL);
    }
    for (int64_t r = 0; !rc && r < H; ++r) {
      double acc = (double)osh[r];
      for (int j = 0; j < k; ++j) {
        if (idx[t * k + j] < 0) continue;
        acc += (double)w[t * k + j] * (double)oe[j * H + r];
      }
      y[t * H + r] = (float)acc;
    }
  }
  if (!rc) {
    if (idx_out) memcpy(idx_out, idx, sizeof(int32_t) * (size_t)(T * k));
    if (w_out) memcpy(w_out, w, sizeof(float) * (size_t)(T * k));
    if (logits_out) memcpy(logits_out, lg, sizeof(float) * (size_t)(T * E));
  }
  free(osh); free(oe); free(lg); free(idx); free(w);
  return rc;
}

/*
 * O10 -- batch-union bookkeeping (colibrì README, "Implemented features":
 * in prefill and MTP verification each unique expert of the batch is read
 * once and applied to all positions routed to it).
 * Reading: the (token, slot) pairs routed to each expert, listed expert by
 * expert in increasing expert id and, within an expert, in increasing
 * (token, slot) order; a slot dropped by top-p (idx -1) is in no list.
 */
int orc_union_tables(const int32_t *idx, int64_t T, int32_t k, int32_t E,
                     int32_t *counts, int32_t *offs, int32_t *perm,
                     int32_t *uniq, int32_t *n_uniq) {
  if (!idx || T < 0 || k <= 0 || E <= 0 || !counts || !offs || !perm ||
      !uniq || !n_uniq)
    return ORC_EINVAL;
  for (int64_t i = 0; i < T * k; ++i)
    if (idx[i] < -1 || idx[i] >= E) return ORC_EINVAL;
  for (int e = 0; e < E; ++e) counts[e] = 0;
  for (int64_t i = 0; i < T * k; ++i)
    if (idx[i] >= 0) counts[idx[i]]++;
  offs[0] = 0;
  for (int e = 0; e < E; ++e) offs[e + 1] = offs[e] + counts[e];
  int64_t p = 0;
  for (int e = 0; e < E; ++e)
    for (int64_t i = 0; i < T * k; ++i)
      if (idx[i] == e) perm[p++] = (int32_t)i;
  int32_t n = 0;
  for (int e = 0; e < E; ++e)
    if (counts[e] > 0) uniq[n++] = e;
  *n_uniq = n;
  return ORC_OK;
}
