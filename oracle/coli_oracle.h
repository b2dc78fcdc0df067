/*
 * coli_oracle.h -- the CPU oracle for colibrì's routed-expert MoE layer.
 *
 * TEST INFRASTRUCTURE ONLY.  This is the plain, slow reference that the GPU
 * library is checked against.  Only the test suite, the smoke check of the
 * package entry module and the CPU-baseline leg of the benchmark may load or
 * call it; the product library never links, includes or calls anything here,
 * and this file shares no code, header, table or helper with it.
 *
 * Sources (web pages about colibrì, the pure-C GLM-5.2 engine):
 *   [README]  the colibrì README (JustVugg/colibri), sections "思路" (Idea) and
 *             "已实现的功能" (Implemented features);
 *   [CSDN]    the CSDN feature "Colibrì：蜂鸟驮巨兽——纯C语言打造的7440亿参数MoE
 *             本地推理引擎", section "纯C语言的浪漫与偏执" (pure C);
 *   [LABHUB]  the labhub post on running GLM-5.2 on slow computers, sections
 *             "核心技巧" (core trick) and "让它变得可以忍受的那些装置" (devices).
 * Where the pages leave a step open, the reading taken is stated at the
 * function (and collected in the repository's design notes).
 *
 * Parity unpinned against colibrì itself (the pages print no values): the
 * weight-quantisation rule, the Q8_0 scale type, the group score and expert
 * top-p renormalisation are readings, pinned only against mathematics.
 *
 * Conventions: row-major arrays; int8 codes are two's complement; every
 * floating-point step is IEEE binary32 or binary64 as stated, built without
 * -ffast-math and without FMA contraction.  Functions return 0 on success
 * and ORC_EINVAL on a bad argument (nothing written in that case).
 */
#ifndef COLI_ORACLE_H
#define COLI_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ORC_OK 0
#define ORC_EINVAL 1

/* Largest code magnitude for a b-bit symmetric container: 127, 7, 1. */
int orc_qmax(int bits);

/* O1 weight quantisation, one fp32 scale per row. */
int orc_quant_rows(int bits, const float *w, int64_t rows, int64_t cols,
                   int8_t *codes, float *scales);

/* O2 packing of codes into bytes (row stride cols*bits/8) and back. */
int orc_pack(int bits, const int8_t *codes, int64_t rows, int64_t cols,
             uint8_t *packed);
int orc_unpack(int bits, const uint8_t *packed, int64_t rows, int64_t cols,
               int8_t *codes);

/* O1 followed by O2. */
int orc_quant_pack(int bits, const float *w, int64_t rows, int64_t cols,
                   uint8_t *packed, float *scales);

/* O3 Q8_0-style activation quantisation: blocks of 32 along each row. */
int orc_q8_0(const float *x, int64_t T, int64_t n, int8_t *q, float *d);

/* O4 quantised matrix-vector product.
 * acc[t][r][b] (optional): exact int32 sum over block b of code products.
 * y[t][r] (optional): fl32 of the fp64 sum over blocks of s_r*d[t][b]*acc. */
int orc_qdot(int bits, const uint8_t *w_packed, const float *w_scale,
             int64_t rows, int64_t cols, const int8_t *xq, const float *xd,
             int64_t T, int32_t *acc, float *y);

/* O12 the f32-activation variant of O4: y[t][r] = fl32(s_r * sum_c
 * code[r][c] * x[t][c]) with the sum and the product in fp64. */
int orc_qdot_f32act(int bits, const uint8_t *w_packed, const float *w_scale,
                    int64_t rows, int64_t cols, const float *x, int64_t T, float *y);

/* O5 router logits: l[t][e] = fl32(sum_i x[t][i]*Wg[e][i]) in fp64. */
int orc_logits(const float *x, const float *gate_w, int64_t T, int64_t E,
               int64_t H, float *logits);

typedef struct {
  int32_t n_experts;      /* E */
  int32_t top_k;          /* k */
  int32_t n_group;        /* groups of E/n_group contiguous experts */
  int32_t topk_group;     /* groups kept */
  int32_t norm_topk_prob; /* 1: normalise the selected scores to sum 1 */
  float routed_scaling_factor;
  float top_p;            /* expert top-p; off unless 0 < top_p < 1 */
  int32_t top_p_renorm;   /* 1: renormalise over the kept experts */
} orc_router_cfg;

/* O6/O7 routing.  idx/w are [T][k] in rank order; a slot dropped by top-p
 * holds idx -1 and weight 0.  sigma (optional) receives the [T][E] fp32
 * sigmoid scores. */
int orc_route(const orc_router_cfg *cfg, const float *logits,
              const float *bias, int64_t T, int32_t *idx, float *w,
              float *sigma);

/* O8 one SwiGLU expert over T tokens: x [T][H] -> o [T][H].
 * h (optional) receives the fp32 intermediate [T][I]. */
int orc_expert_ffn(int bits, int64_t H, int64_t I,
                   const uint8_t *wg, const float *sg,
                   const uint8_t *wu, const float *su,
                   const uint8_t *wd, const float *sd,
                   const float *x, int64_t T, float *o, float *h);

/* One layer.  Routed expert e's tensors are reached through per-expert
 * pointer tables so a caller may supply only the experts a batch uses; a
 * routed expert that is selected but has a NULL table entry is an error. */
typedef struct {
  int32_t hidden, inter, bits;
  orc_router_cfg router;
  const float *gate_w;    /* [E][H] fp32, may be NULL if logits are given */
  const float *gate_bias; /* [E] fp32 or NULL (= zero) */
  const uint8_t *const *w_gate; const float *const *s_gate; /* [E] -> [I][H*b/8], [I] */
  const uint8_t *const *w_up;   const float *const *s_up;   /* [E] -> [I][H*b/8], [I] */
  const uint8_t *const *w_down; const float *const *s_down; /* [E] -> [H][I*b/8], [H] */
  const uint8_t *sh_gate, *sh_up, *sh_down;                 /* shared expert */
  const float *sh_s_gate, *sh_s_up, *sh_s_down;
} orc_layer;

/* O9 the layer on T tokens, each token on its own (no grouping).
 * logits_in may be NULL (then O5 from gate_w).  idx_out, w_out, logits_out
 * are optional. */
int orc_moe_forward(const orc_layer *L, const float *x, int64_t T,
                    const float *logits_in, float *y, int32_t *idx_out,
                    float *w_out, float *logits_out);

/* O11 FP8 checkpoint dequantisation: w8 [rows][cols] OCP FP8 E4M3 ("e4m3fn")
 * codes, block_scale [ceil(rows/128)][ceil(cols/128)] fp32; out[r][c] =
 * e4m3(w8[r][c]) * block_scale[r/128][c/128] rounded once to binary32.  The
 * two NaN codes give NaN.  orc_e4m3_value decodes one code. */
float orc_e4m3_value(uint8_t code);
int orc_dequant_fp8_block(const uint8_t *w8, const float *block_scale, int64_t rows,
                          int64_t cols, float *out);

/* O10 batch-union tables from idx [T][k] (entries -1 are skipped):
 * counts[E], offs[E+1] (exclusive scan), perm[] = t*k+j of each routed pair
 * ordered by (expert, t, j), uniq[] = experts with a nonzero count in
 * increasing order, *n_uniq their number.  perm needs T*k entries and uniq
 * E entries. */
int orc_union_tables(const int32_t *idx, int64_t T, int32_t k, int32_t E,
                     int32_t *counts, int32_t *offs, int32_t *perm,
                     int32_t *uniq, int32_t *n_uniq);

/* Number of OpenMP threads the oracle runs with (1 without OpenMP). */
int orc_num_threads(void);

/* Sets the OpenMP thread count of later oracle calls (n <= 0: no change).
 * Results do not depend on it. */
void orc_set_num_threads(int n);

#ifdef __cplusplus
}
#endif
#endif
