/*
 * oracle.c -- plain, slow, scalar CPU oracle of the W8A8 INT8 fused-MoE layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code with
 * the HIP path: no kernels, headers, helpers or tables.
 *
 * Sources (the pages):
 *  - SGLang PR #3888 "[Feature] DeepSeek V3/R1 INT8 Quantization
 *    (channel-wise)", Modifications and Performance sections: the fused MoE
 *    kernel with channel-wise int8 weights and an int32 accumulator.
 *  - jiqizhixin, Meituan INT8 DeepSeek R1 article, section "Quantization
 *    exploration": block-wise quantization in [128,128] weight tiles with
 *    activations quantized online per token-group; channel-wise quantization
 *    with one weight group per output channel, activations quantized online
 *    per token, and a single dequantization after the INT8 matmul.
 *  - SGLang PR #8273 "support cutlass_moe_fp8 for deepepmoe", review on
 *    m_indices: expert offsets are the zero-padded cumulative sum of the
 *    per-expert token counts; the scatter emits the expert id of every row.
 *    Its highlights: MoE = scatter inputs, GEMM (w13), activation, GEMM (w2),
 *    gather outputs.
 * Where the pages are silent, the plainest reading is taken:
 *  - symmetric int8 in [-127, 127]; scale = max(max|x| / 127, 1e-8);
 *    q = round-half-even(x / scale) with an IEEE division;
 *  - w13 rows [0, I) are the gate, rows [I, 2I) the up projection;
 *    activation SiLU(gate) * up with silu(g) = g / (1 + exp(-g));
 *  - dequantization order ((float)acc * a_scale) * w_scale;
 *  - the intermediate is requantized per (token, expert) row (channel-wise) or
 *    per (row, 128-group) (block-wise), by the same rule as the activations;
 *  - combine: out = 0, then out = out + w_j * y_j for slots j = 0..k-1, fp32;
 *  - routing (the pages only name topk_idx): softmax top-k renormalised, or
 *    sigmoid scores with node-limited grouped selection (group score = sum of
 *    the group's two best scores), as in the DeepSeek-V3 technical report the
 *    article cites; ties go to the lower index everywhere.
 * Build: -O2 -fno-fast-math -ffp-contract=off, so every fp32 operation below
 * is one IEEE operation in the written order.  Outer loops run under OpenMP.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_EXPORT __attribute__((visibility("default")))

/* ------------------------------------------------------------------ quantization */

/* Symmetric INT8 quantization with one scale per br x bc block of a row-major
 * [rows, cols] fp32 matrix.  br=1, bc=cols: one scale per row (per-token
 * activations; per-output-channel weights, whose rows are output channels).
 * br=1, bc=128: per-token-group activations.  br=bc=128: block-wise weights.
 * Scale grid is [ceil(rows/br), ceil(cols/bc)], row-major. */
ORACLE_EXPORT void oracle_quant_blocks(const float* x, int64_t rows, int64_t cols, int64_t br,
                                       int64_t bc, int8_t* q, float* s) {
  const int64_t nbr = (rows + br - 1) / br, nbc = (cols + bc - 1) / bc;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t b = 0; b < nbr * nbc; ++b) {
    const int64_t bi = b / nbc, bj = b % nbc;
    const int64_t r0 = bi * br, r1 = (r0 + br < rows) ? r0 + br : rows;
    const int64_t c0 = bj * bc, c1 = (c0 + bc < cols) ? c0 + bc : cols;
    float amax = 0.0f;
    for (int64_t r = r0; r < r1; ++r)
      for (int64_t c = c0; c < c1; ++c) {
        float a = fabsf(x[r * cols + c]);
        if (a > amax) amax = a;
      }
    float sc = amax / 127.0f;
    if (sc < 1e-8f) sc = 1e-8f;
    s[b] = sc;
    for (int64_t r = r0; r < r1; ++r)
      for (int64_t c = c0; c < c1; ++c) {
        float v = nearbyintf(x[r * cols + c] / sc);
        if (v > 127.0f) v = 127.0f;
        if (v < -127.0f) v = -127.0f;
        q[r * cols + c] = (int8_t)v;
      }
  }
}

/* ------------------------------------------------------------------ routing */

/* a beats b: larger value first, equal values to the lower index. */
static int beats(float va, int64_t a, float vb, int64_t b) { return va > vb || (va == vb && a < b); }

/* Index of the best candidate (cand[i] != 0) of v[0..n), -1 if none. */
static int64_t best_of(const float* v, const unsigned char* cand, int64_t n) {
  int64_t best = -1;
  for (int64_t i = 0; i < n; ++i)
    if (cand[i] && (best < 0 || beats(v[i], i, v[best], best))) best = i;
  return best;
}

/* score_fn 0 = softmax, 1 = sigmoid.  n_group = 1 means ungrouped.
 * softmax: select the k largest logits.  renormalize: w_j = exp(l_j - m) / sum
 *   over the selected (m = largest selected), i.e. softmax over the selection;
 *   otherwise w_j = exp(l_j - m) / (sum over all E in index order).
 * sigmoid: s = 1/(1+exp(-l)), c = s + bias; group score = best + second best c
 *   of the group; keep the topk_group best groups; select the k best c among
 *   the kept groups' experts; w_j = s_j (/ sum of selected s if renormalize).
 * Finally w_j = w_j * routed_scaling.  Slots are in selection order. */
ORACLE_EXPORT void oracle_route(const float* logits, int64_t T, int64_t E, int64_t k, int32_t score_fn,
                                int64_t n_group, int64_t topk_group, int32_t renormalize,
                                float routed_scaling, const float* bias, int32_t* ids, float* w) {
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t t = 0; t < T; ++t) {
    const float* l = logits + t * E;
    float* s = (float*)malloc(sizeof(float) * E);
    float* c = (float*)malloc(sizeof(float) * E);
    unsigned char* cand = (unsigned char*)malloc(E);
    int32_t* sel = ids + t * k;
    float* wt = w + t * k;
    if (score_fn == 0) {
      for (int64_t e = 0; e < E; ++e) cand[e] = 1;
      for (int64_t j = 0; j < k; ++j) {
        int64_t b = best_of(l, cand, E);
        sel[j] = (int32_t)b;
        cand[b] = 0;
      }
      const float m = l[sel[0]];
      float sum = 0.0f;
      if (renormalize) {
        for (int64_t j = 0; j < k; ++j) sum = sum + expf(l[sel[j]] - m);
      } else {
        for (int64_t e = 0; e < E; ++e) sum = sum + expf(l[e] - m);
      }
      for (int64_t j = 0; j < k; ++j) wt[j] = (expf(l[sel[j]] - m) / sum) * routed_scaling;
    } else {
      for (int64_t e = 0; e < E; ++e) {
        s[e] = 1.0f / (1.0f + expf(-l[e]));
        c[e] = bias ? s[e] + bias[e] : s[e];
      }
      if (n_group > 1) {
        const int64_t gs = E / n_group;
        float* gscore = (float*)malloc(sizeof(float) * n_group);
        unsigned char* gcand = (unsigned char*)malloc(n_group);
        for (int64_t g = 0; g < n_group; ++g) {
          /* the group's best and second-best c */
          for (int64_t e = 0; e < gs; ++e) cand[e] = 1;
          int64_t b1 = best_of(c + g * gs, cand, gs);
          if (gs >= 2) {
            cand[b1] = 0;
            int64_t b2 = best_of(c + g * gs, cand, gs);
            gscore[g] = c[g * gs + b1] + c[g * gs + b2];
          } else {
            gscore[g] = c[g * gs + b1];
          }
          gcand[g] = 1;
        }
        for (int64_t e = 0; e < E; ++e) cand[e] = 0;
        for (int64_t j = 0; j < topk_group; ++j) {
          int64_t g = best_of(gscore, gcand, n_group);
          gcand[g] = 0;
          for (int64_t e = g * gs; e < (g + 1) * gs; ++e) cand[e] = 1;
        }
        free(gscore);
        free(gcand);
      } else {
        for (int64_t e = 0; e < E; ++e) cand[e] = 1;
      }
      for (int64_t j = 0; j < k; ++j) {
        int64_t b = best_of(c, cand, E);
        sel[j] = (int32_t)b;
        cand[b] = 0;
      }
      float sum = 0.0f;
      for (int64_t j = 0; j < k; ++j) sum = sum + s[sel[j]];
      for (int64_t j = 0; j < k; ++j) {
        float v = renormalize ? s[sel[j]] / sum : s[sel[j]];
        wt[j] = v * routed_scaling;
      }
    }
    free(s);
    free(c);
    free(cand);
  }
}

/* ------------------------------------------------------------------ align */

/* Stable grouping of the P = T*k (token, slot) pairs by expert (pair id
 * p = t*k + j).  counts[e]; offsets = [0, cumsum(counts)] (E+1 entries);
 * each expert's segment is padded to a multiple of block_m with the sentinel
 * P; padded_offsets = [0, cumsum(padded counts)]; tile_expert[i] = expert of
 * tile i; num_tiles = padded_offsets[E] / block_m.  Pair ids ascend within an
 * expert. */
ORACLE_EXPORT void oracle_align(const int32_t* ids, int64_t T, int64_t k, int64_t E, int64_t block_m,
                                int32_t* counts, int32_t* offsets, int32_t* padded_offsets,
                                int32_t* sorted_pair_ids, int32_t* tile_expert, int32_t* num_tiles) {
  const int64_t P = T * k;
  for (int64_t e = 0; e < E; ++e) counts[e] = 0;
  /* An expert id outside [0, E) names no expert: the pair is dropped (it takes no row). */
  for (int64_t p = 0; p < P; ++p)
    if (ids[p] >= 0 && ids[p] < E) counts[ids[p]] += 1;
  offsets[0] = 0;
  padded_offsets[0] = 0;
  for (int64_t e = 0; e < E; ++e) {
    offsets[e + 1] = offsets[e] + counts[e];
    int64_t pc = (counts[e] + block_m - 1) / block_m * block_m;
    padded_offsets[e + 1] = padded_offsets[e] + (int32_t)pc;
  }
  int64_t* fill = (int64_t*)malloc(sizeof(int64_t) * (E > 0 ? E : 1));
  for (int64_t e = 0; e < E; ++e) fill[e] = padded_offsets[e];
  for (int64_t p = 0; p < P; ++p)
    if (ids[p] >= 0 && ids[p] < E) sorted_pair_ids[fill[ids[p]]++] = (int32_t)p;
  for (int64_t e = 0; e < E; ++e)
    for (int64_t r = fill[e]; r < padded_offsets[e + 1]; ++r) sorted_pair_ids[r] = (int32_t)P;
  free(fill);
  for (int64_t e = 0; e < E; ++e)
    for (int64_t i = padded_offsets[e] / block_m; i < padded_offsets[e + 1] / block_m; ++i)
      tile_expert[i] = (int32_t)e;
  *num_tiles = (int32_t)(padded_offsets[E] / block_m);
}

/* ------------------------------------------------------------------ GEMM pieces */

/* Exact int8 x int8 dot product with int32 accumulation (|sum| <= K*127*127 < 2^31). */
static int32_t dot_i8(const int8_t* a, const int8_t* b, int64_t K) {
  int32_t acc = 0;
  for (int64_t i = 0; i < K; ++i) acc += (int32_t)a[i] * (int32_t)b[i];
  return acc;
}

static float silu_mul(float g, float u) { return (g / (1.0f + expf(-g))) * u; }

/* Requantize one row of fp32 values by the activation rule, per group of `group`
 * columns (group = n for a single scale). */
static void requant_row(const float* hf, int64_t n, int64_t group, int8_t* q, float* s) {
  for (int64_t g0 = 0, gi = 0; g0 < n; g0 += group, ++gi) {
    float amax = 0.0f;
    for (int64_t i = g0; i < g0 + group; ++i) {
      float a = fabsf(hf[i]);
      if (a > amax) amax = a;
    }
    float sc = amax / 127.0f;
    if (sc < 1e-8f) sc = 1e-8f;
    s[gi] = sc;
    for (int64_t i = g0; i < g0 + group; ++i) {
      float v = nearbyintf(hf[i] / sc);
      if (v > 127.0f) v = 127.0f;
      if (v < -127.0f) v = -127.0f;
      q[i] = (int8_t)v;
    }
  }
}

/* One expert row of the first GEMM + activation + requantization.
 * a: the token's int8 activations [H]; channel mode: a_s points at the token's
 * scale, w_s at the expert's [2I] channel scales; block mode: a_s -> [H/128],
 * w_s -> [2I/128, H/128].  Writes h_q [I] and h_s ([1] or [I/128]). */
static void w13_row(const int8_t* a, const float* a_s, const int8_t* w13, const float* w_s, int64_t H,
                    int64_t I, int32_t block, float* hf, int8_t* h_q, float* h_s) {
  for (int64_t n = 0; n < I; ++n) {
    float g, u;
    if (!block) {
      int32_t ag = dot_i8(a, w13 + n * H, H);
      int32_t au = dot_i8(a, w13 + (n + I) * H, H);
      g = ((float)ag * a_s[0]) * w_s[n];
      u = ((float)au * a_s[0]) * w_s[n + I];
    } else {
      const int64_t nkb = H / 128;
      g = 0.0f;
      u = 0.0f;
      for (int64_t kb = 0; kb < nkb; ++kb) {
        int32_t pg = dot_i8(a + kb * 128, w13 + n * H + kb * 128, 128);
        int32_t pu = dot_i8(a + kb * 128, w13 + (n + I) * H + kb * 128, 128);
        g = g + (((float)pg * a_s[kb]) * w_s[(n / 128) * nkb + kb]);
        u = u + (((float)pu * a_s[kb]) * w_s[((n + I) / 128) * nkb + kb]);
      }
    }
    hf[n] = silu_mul(g, u);
  }
  requant_row(hf, I, block ? 128 : I, h_q, h_s);
}

/* One expert row of the second GEMM, dequantized: y [H]. */
static void w2_row(const int8_t* hq, const float* h_s, const int8_t* w2, const float* w_s, int64_t H,
                   int64_t I, int32_t block, float* y) {
  for (int64_t n = 0; n < H; ++n) {
    if (!block) {
      int32_t acc = dot_i8(hq, w2 + n * I, I);
      y[n] = ((float)acc * h_s[0]) * w_s[n];
    } else {
      const int64_t nkb = I / 128;
      float acc_f = 0.0f;
      for (int64_t kb = 0; kb < nkb; ++kb) {
        int32_t part = dot_i8(hq + kb * 128, w2 + n * I + kb * 128, 128);
        acc_f = acc_f + (((float)part * h_s[kb]) * w_s[(n / 128) * nkb + kb]);
      }
      y[n] = acc_f;
    }
  }
}

/* ------------------------------------------------------------------ grouped (sorted-row) stages
 *
 * Experts' weights are passed as arrays of per-expert pointers (NULL for
 * experts that are not needed), so full-size checks can materialise only the
 * experts they touch.  Rows are the padded expert-sorted rows of the align
 * step; `rows` / `nrows` select which rows to compute (NULL = all rows below
 * num_tiles * block_m).  Pad rows (sentinel P) are skipped. */

static int64_t row_at(const int64_t* rows, int64_t i) { return rows ? rows[i] : i; }

/* Raw int32 accumulators.  gather = 1: A row of sorted row r is a[sorted[r] / k]
 * (first GEMM on the token activations); gather = 0: A row is a[r] (second GEMM
 * on the sorted intermediate).  out [*, N] int32 indexed by sorted row. */
ORACLE_EXPORT void oracle_grouped_gemm_i32(const int8_t* a, int64_t K, int32_t gather,
                                           const int8_t* const* w, int64_t N,
                                           const int32_t* sorted_pair_ids, const int32_t* tile_expert,
                                           int64_t block_m, int64_t P, int64_t k, const int64_t* rows,
                                           int64_t nrows, int32_t* out) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t i = 0; i < nrows; ++i) {
    const int64_t r = row_at(rows, i);
    const int64_t p = sorted_pair_ids[r];
    if (p >= P) continue;
    const int8_t* arow = gather ? a + (p / k) * K : a + r * K;
    const int8_t* we = w[tile_expert[r / block_m]];
    for (int64_t n = 0; n < N; ++n) out[r * N + n] = dot_i8(arow, we + n * K, K);
  }
}

/* First GEMM + SiLU(gate)*up + requantization over sorted rows.
 * channel: a_s [T], w13_s[e] -> [2I], h_s [rows]; block: a_s [T, H/128],
 * w13_s[e] -> [2I/128, H/128], h_s [rows, I/128]. */
ORACLE_EXPORT void oracle_w13_silu(const int8_t* a_q, const float* a_s, const int8_t* const* w13,
                                   const float* const* w13_s, const int32_t* sorted_pair_ids,
                                   const int32_t* tile_expert, int64_t block_m, int64_t T, int64_t k,
                                   int64_t H, int64_t I, int32_t block, const int64_t* rows, int64_t nrows,
                                   int8_t* h_q, float* h_s) {
  const int64_t P = T * k;
  const int64_t nsa = block ? H / 128 : 1, nsh = block ? I / 128 : 1;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t i = 0; i < nrows; ++i) {
    const int64_t r = row_at(rows, i);
    const int64_t p = sorted_pair_ids[r];
    if (p >= P) continue;
    const int64_t t = p / k, e = tile_expert[r / block_m];
    float* hf = (float*)malloc(sizeof(float) * I);
    w13_row(a_q + t * H, a_s + t * nsa, w13[e], w13_s[e], H, I, block, hf, h_q + r * I, h_s + r * nsh);
    free(hf);
  }
}

/* Second GEMM + top-k weighted combine.  out has one fp32 row of H per listed
 * token (tokens = NULL: all T tokens in order), fully overwritten.  pair_row is
 * built here from sorted_pair_ids (the inverse map). */
ORACLE_EXPORT void oracle_w2_combine(const int8_t* h_q, const float* h_s, const int8_t* const* w2,
                                     const float* const* w2_s, const int32_t* sorted_pair_ids,
                                     const int32_t* tile_expert, int32_t num_tiles, int64_t block_m,
                                     const float* topk_weights, int64_t T, int64_t k, int64_t H, int64_t I,
                                     int32_t block, const int64_t* tokens, int64_t ntok, float* out) {
  const int64_t P = T * k, R = (int64_t)num_tiles * block_m;
  const int64_t nsh = block ? I / 128 : 1;
  int64_t* pair_row = (int64_t*)malloc(sizeof(int64_t) * (P > 0 ? P : 1));
  for (int64_t p = 0; p < P; ++p) pair_row[p] = -1;
  for (int64_t r = 0; r < R; ++r)
    if (sorted_pair_ids[r] < P) pair_row[sorted_pair_ids[r]] = r;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t i = 0; i < ntok; ++i) {
    const int64_t t = tokens ? tokens[i] : i;
    float* y = (float*)malloc(sizeof(float) * H);
    float* o = out + i * H;
    for (int64_t n = 0; n < H; ++n) o[n] = 0.0f;
    for (int64_t j = 0; j < k; ++j) {
      const int64_t r = pair_row[t * k + j];
      if (r < 0) continue;
      const int64_t e = tile_expert[r / block_m];
      w2_row(h_q + r * I, h_s + r * nsh, w2[e], w2_s[e], H, I, block, y);
      const float wj = topk_weights[t * k + j];
      for (int64_t n = 0; n < H; ++n) o[n] = o[n] + (wj * y[n]);
    }
    free(y);
  }
  free(pair_row);
}

/* ------------------------------------------------------------------ dense per-token reference
 *
 * The whole layer for a list of tokens, computed straight from the routing
 * with no sorting: for token t, quantize its activations, then for each slot
 * j run the expert MLP on the int8 row and accumulate out = out + w_j * y_j.
 * x: fp32 activations of the listed tokens [ntok, H] (bf16 inputs widened
 * exactly by the caller); ids/weights [ntok, k]; out [ntok, H].  The
 * operations and their order are those of the sorted pipeline, so the two
 * results must agree bit for bit. */
ORACLE_EXPORT void oracle_moe_tokens(const float* x, int64_t ntok, int64_t H, int64_t I, int64_t k,
                                     const int32_t* ids, const float* topk_weights,
                                     const int8_t* const* w13, const float* const* w13_s,
                                     const int8_t* const* w2, const float* const* w2_s, int32_t block,
                                     float* out) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t t = 0; t < ntok; ++t) {
    const int64_t nsa = block ? H / 128 : 1, nsh = block ? I / 128 : 1;
    int8_t* aq = (int8_t*)malloc(H);
    float* as = (float*)malloc(sizeof(float) * nsa);
    float* hf = (float*)malloc(sizeof(float) * I);
    int8_t* hq = (int8_t*)malloc(I);
    float* hs = (float*)malloc(sizeof(float) * nsh);
    float* y = (float*)malloc(sizeof(float) * H);
    /* online activation quantization: one scale per token or per 128-group */
    requant_row(x + t * H, H, block ? 128 : H, aq, as);
    float* o = out + t * H;
    for (int64_t n = 0; n < H; ++n) o[n] = 0.0f;
    for (int64_t j = 0; j < k; ++j) {
      const int64_t e = ids[t * k + j];
      w13_row(aq, as, w13[e], w13_s[e], H, I, block, hf, hq, hs);
      w2_row(hq, hs, w2[e], w2_s[e], H, I, block, y);
      const float wj = topk_weights[t * k + j];
      for (int64_t n = 0; n < H; ++n) o[n] = o[n] + (wj * y[n]);
    }
    free(aq);
    free(as);
    free(hf);
    free(hq);
    free(hs);
    free(y);
  }
}

/* ------------------------------------------------------------------ dense linear
 *
 * The model's non-MoE projections in W8A8 INT8 (PR #3888 Modifications, "Norm Linear"; article,
 * "Quantization exploration": per-token activation scales, per-channel weight scales, one
 * dequantization after the INT8 matmul):
 *   out[m][n] = ((float)(a_q[m] . w[n]) * a_s[m]) * w_s[n]
 * a_q [M, K] int8, a_s [M], w [N, K] int8, w_s [N], out [M, N] fp32; `rows` / `nrows` select the
 * rows m to compute (NULL = all). */
ORACLE_EXPORT void oracle_linear(const int8_t* a_q, const float* a_s, const int8_t* w, const float* w_s, int64_t M,
                                 int64_t N, int64_t K, const int64_t* rows, int64_t nrows, float* out) {
  if (!rows) nrows = M;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t i = 0; i < nrows; ++i) {
    const int64_t m = row_at(rows, i);
    for (int64_t n = 0; n < N; ++n) {
      const int32_t acc = dot_i8(a_q + m * K, w + n * K, K);
      out[m * N + n] = ((float)acc * a_s[m]) * w_s[n];
    }
  }
}

/* ------------------------------------------------------------------ FP8 block-wise path
 *
 * SGLang PR #8273 "support cutlass_moe_fp8 for deepepmoe" (description, "New FP8 MoE Kernel"):
 * an MoE whose weights are FP8 with one scale per block and whose activations are FP8 with one
 * scale per token-group, multiplied by a block-scaled grouped GEMM (fp8_blockwise_scaled_grouped_mm
 * in its review).  The pages name the scheme and no arithmetic; the readings taken here:
 *  - FP8 is E4M3 as the OCP 8-bit floating-point specification defines it: sign bit, 4 exponent
 *    bits with bias 7, 3 mantissa bits, subnormals at exponent field 0, largest finite value 448,
 *    no infinities; codes 0x7F and 0xFF are NaN and are never produced.
 *  - Scales follow the INT8 rule with 448 (the largest finite E4M3 value) in place of 127:
 *    scale = max(max|x| / 448, 1e-8); code = the E4M3 value nearest to x / scale, ties to the
 *    even mantissa, with x / scale clamped to [-448, 448] first; a result of zero keeps the sign
 *    of x / scale.  Blocks are those of the INT8 block-wise path: 128 x 128 weight blocks and
 *    (token, 128-column) activation groups; the intermediate is requantized per (row, 128-group).
 *  - Block-scaled product: for each 128-wide K-block, part = sum of the products of the decoded
 *    values, computed exactly (every product of two E4M3 values is exact in a double, and 128 of
 *    them span fewer than 53 bits) and rounded once to fp32; then acc = acc + ((part * a_s) * w_s)
 *    in fp32, in ascending K-block order.  Everything after the sums is the INT8 block-wise path's
 *    arithmetic (SiLU(gate) * up, requantization, combine). */

/* Value of an E4M3 code (NaN codes never reach here). */
static double e4m3_decode(uint8_t c) {
  const int e = (c >> 3) & 15, m = c & 7;
  const double v = e == 0 ? ldexp((double)m, -9)      /* m/8 * 2^-6 */
                          : ldexp((double)(8 + m), e - 10); /* (1 + m/8) * 2^(e-7) */
  return (c & 0x80) ? -v : v;
}

/* The 256 code values, filled from e4m3_decode before any parallel use (the GEMMs and the
 * quantization look every code up many times). */
static double e4m3_table[256];
static int e4m3_table_ready = 0;
static void e4m3_table_init(void) {
  if (e4m3_table_ready) return;
  for (int c = 0; c < 256; ++c) e4m3_table[c] = e4m3_decode((uint8_t)c);
  e4m3_table_ready = 1;
}

/* E4M3 code nearest to x (x finite): clamp to [-448, 448], then the nearest of the 127
 * non-negative finite codes by magnitude, ties to the even code (consecutive codes alternate
 * mantissa parity, so the even code is the even mantissa). */
static uint8_t e4m3_encode(float x) {
  const int neg = signbit(x) != 0;
  double a = fabs((double)x);
  if (a > 448.0) a = 448.0;
  int lo = 0;
  for (int c = 0; c <= 0x7E; ++c)
    if (e4m3_table[c] <= a) lo = c;
  int code = lo;
  if (e4m3_table[lo] != a) {
    const int hi = lo + 1; /* a < 448 here, so lo < 0x7E */
    const double mid = (e4m3_table[lo] + e4m3_table[hi]) / 2.0; /* exact */
    if (a > mid || (a == mid && (hi & 1) == 0)) code = hi;
  }
  return (uint8_t)(code | (neg ? 0x80 : 0));
}

ORACLE_EXPORT void oracle_fp8_decode(const uint8_t* c, int64_t n, float* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = (float)e4m3_decode(c[i]);
}

ORACLE_EXPORT void oracle_fp8_encode(const float* x, int64_t n, uint8_t* out) {
  e4m3_table_init();
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = e4m3_encode(x[i]);
}

static float fp8_scale(float amax) {
  float sc = amax / 448.0f;
  if (sc < 1e-8f) sc = 1e-8f;
  return sc;
}

/* FP8 quantization with one scale per br x bc block of a row-major [rows, cols] fp32 matrix
 * (br=1, bc=128: per-token-group activations; br=bc=128: block-wise weights). */
ORACLE_EXPORT void oracle_fp8_quant_blocks(const float* x, int64_t rows, int64_t cols, int64_t br, int64_t bc,
                                           uint8_t* q, float* s) {
  e4m3_table_init();
  const int64_t nbr = (rows + br - 1) / br, nbc = (cols + bc - 1) / bc;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t b = 0; b < nbr * nbc; ++b) {
    const int64_t bi = b / nbc, bj = b % nbc;
    const int64_t r0 = bi * br, r1 = (r0 + br < rows) ? r0 + br : rows;
    const int64_t c0 = bj * bc, c1 = (c0 + bc < cols) ? c0 + bc : cols;
    float amax = 0.0f;
    for (int64_t r = r0; r < r1; ++r)
      for (int64_t c = c0; c < c1; ++c) {
        float a = fabsf(x[r * cols + c]);
        if (a > amax) amax = a;
      }
    const float sc = fp8_scale(amax);
    s[b] = sc;
    for (int64_t r = r0; r < r1; ++r)
      for (int64_t c = c0; c < c1; ++c) q[r * cols + c] = e4m3_encode(x[r * cols + c] / sc);
  }
}

/* One K-block's sum of products, exact, rounded once to fp32. */
static float fp8_part(const uint8_t* a, const uint8_t* b) {
  double sum = 0.0;
  for (int i = 0; i < 128; ++i) sum += e4m3_table[a[i]] * e4m3_table[b[i]];
  return (float)sum;
}

static void fp8_requant_row(const float* hf, int64_t n, uint8_t* q, float* s) {
  for (int64_t g0 = 0, gi = 0; g0 < n; g0 += 128, ++gi) {
    float amax = 0.0f;
    for (int64_t i = g0; i < g0 + 128; ++i) {
      float a = fabsf(hf[i]);
      if (a > amax) amax = a;
    }
    const float sc = fp8_scale(amax);
    s[gi] = sc;
    for (int64_t i = g0; i < g0 + 128; ++i) q[i] = e4m3_encode(hf[i] / sc);
  }
}

/* One expert row of the FP8 first GEMM: a [H] codes, a_s [H/128], w13 [2I, H] codes, w_s
 * [2I/128, H/128]; hf [I] scratch; writes h_q [I] codes and h_s [I/128]. */
static void fp8_w13_row(const uint8_t* a, const float* a_s, const uint8_t* w13, const float* w_s, int64_t H,
                        int64_t I, float* hf, uint8_t* h_q, float* h_s) {
  const int64_t nkb = H / 128;
  for (int64_t n = 0; n < I; ++n) {
    float g = 0.0f, u = 0.0f;
    for (int64_t kb = 0; kb < nkb; ++kb) {
      const float pg = fp8_part(a + kb * 128, w13 + n * H + kb * 128);
      const float pu = fp8_part(a + kb * 128, w13 + (n + I) * H + kb * 128);
      g = g + ((pg * a_s[kb]) * w_s[(n / 128) * nkb + kb]);
      u = u + ((pu * a_s[kb]) * w_s[((n + I) / 128) * nkb + kb]);
    }
    hf[n] = silu_mul(g, u);
  }
  fp8_requant_row(hf, I, h_q, h_s);
}

/* One expert row of the FP8 second GEMM: y [H]. */
static void fp8_w2_row(const uint8_t* hq, const float* h_s, const uint8_t* w2, const float* w_s, int64_t H,
                       int64_t I, float* y) {
  const int64_t nkb = I / 128;
  for (int64_t n = 0; n < H; ++n) {
    float acc = 0.0f;
    for (int64_t kb = 0; kb < nkb; ++kb) {
      const float part = fp8_part(hq + kb * 128, w2 + n * I + kb * 128);
      acc = acc + ((part * h_s[kb]) * w_s[(n / 128) * nkb + kb]);
    }
    y[n] = acc;
  }
}

/* FP8 first GEMM + SiLU(gate)*up + requantization over sorted rows (arguments as
 * oracle_w13_silu in block mode, codes in place of int8 values). */
ORACLE_EXPORT void oracle_fp8_w13_silu(const uint8_t* a_q, const float* a_s, const uint8_t* const* w13,
                                       const float* const* w13_s, const int32_t* sorted_pair_ids,
                                       const int32_t* tile_expert, int64_t block_m, int64_t T, int64_t k,
                                       int64_t H, int64_t I, const int64_t* rows, int64_t nrows, uint8_t* h_q,
                                       float* h_s) {
  e4m3_table_init();
  const int64_t P = T * k;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t i = 0; i < nrows; ++i) {
    const int64_t r = row_at(rows, i);
    const int64_t p = sorted_pair_ids[r];
    if (p >= P) continue;
    const int64_t t = p / k, e = tile_expert[r / block_m];
    float* hf = (float*)malloc(sizeof(float) * I);
    fp8_w13_row(a_q + t * H, a_s + t * (H / 128), w13[e], w13_s[e], H, I, hf, h_q + r * I, h_s + r * (I / 128));
    free(hf);
  }
}

/* FP8 second GEMM + top-k weighted combine (arguments as oracle_w2_combine in block mode). */
ORACLE_EXPORT void oracle_fp8_w2_combine(const uint8_t* h_q, const float* h_s, const uint8_t* const* w2,
                                         const float* const* w2_s, const int32_t* sorted_pair_ids,
                                         const int32_t* tile_expert, int32_t num_tiles, int64_t block_m,
                                         const float* topk_weights, int64_t T, int64_t k, int64_t H, int64_t I,
                                         const int64_t* tokens, int64_t ntok, float* out) {
  e4m3_table_init();
  const int64_t P = T * k, R = (int64_t)num_tiles * block_m;
  int64_t* pair_row = (int64_t*)malloc(sizeof(int64_t) * (P > 0 ? P : 1));
  for (int64_t p = 0; p < P; ++p) pair_row[p] = -1;
  for (int64_t r = 0; r < R; ++r)
    if (sorted_pair_ids[r] < P) pair_row[sorted_pair_ids[r]] = r;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t i = 0; i < ntok; ++i) {
    const int64_t t = tokens ? tokens[i] : i;
    float* y = (float*)malloc(sizeof(float) * H);
    float* o = out + i * H;
    for (int64_t n = 0; n < H; ++n) o[n] = 0.0f;
    for (int64_t j = 0; j < k; ++j) {
      const int64_t r = pair_row[t * k + j];
      if (r < 0) continue;
      const int64_t e = tile_expert[r / block_m];
      fp8_w2_row(h_q + r * I, h_s + r * (I / 128), w2[e], w2_s[e], H, I, y);
      const float wj = topk_weights[t * k + j];
      for (int64_t n = 0; n < H; ++n) o[n] = o[n] + (wj * y[n]);
    }
    free(y);
  }
  free(pair_row);
}

/* The whole FP8 layer for a list of tokens, straight from the routing (as oracle_moe_tokens):
 * FP8 quantization of the token per 128-group, then per slot the expert MLP and the combine. */
ORACLE_EXPORT void oracle_fp8_moe_tokens(const float* x, int64_t ntok, int64_t H, int64_t I, int64_t k,
                                         const int32_t* ids, const float* topk_weights,
                                         const uint8_t* const* w13, const float* const* w13_s,
                                         const uint8_t* const* w2, const float* const* w2_s, float* out) {
  e4m3_table_init();
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t t = 0; t < ntok; ++t) {
    uint8_t* aq = (uint8_t*)malloc(H);
    float* as = (float*)malloc(sizeof(float) * (H / 128));
    float* hf = (float*)malloc(sizeof(float) * I);
    uint8_t* hq = (uint8_t*)malloc(I);
    float* hs = (float*)malloc(sizeof(float) * (I / 128));
    float* y = (float*)malloc(sizeof(float) * H);
    fp8_requant_row(x + t * H, H, aq, as);
    float* o = out + t * H;
    for (int64_t n = 0; n < H; ++n) o[n] = 0.0f;
    for (int64_t j = 0; j < k; ++j) {
      const int64_t e = ids[t * k + j];
      fp8_w13_row(aq, as, w13[e], w13_s[e], H, I, hf, hq, hs);
      fp8_w2_row(hq, hs, w2[e], w2_s[e], H, I, y);
      const float wj = topk_weights[t * k + j];
      for (int64_t n = 0; n < H; ++n) o[n] = o[n] + (wj * y[n]);
    }
    free(aq);
    free(as);
    free(hf);
    free(hq);
    free(hs);
    free(y);
  }
}

/* ------------------------------------------------------------------ W4A8 path (int4 weights, FP8 activations)
 *
 * SGLang PR #8311 (w4a8 DeepSeek-R1 in DeepEP low-latency mode; its layer enables the path with a
 * w4afp8 flag): weights in 4-bit integers, activations in FP8.  The pages give no formats or
 * scales; the readings taken here:
 *  - weights: symmetric int4 in [-7, 7], one scale per (output row, 128-wide K group):
 *    scale = max(max|w| / 7, 1e-8), q = clamp(round-half-even(w / scale), -7, 7);
 *  - packing: two values per byte, 4 bytes per 8 consecutive K values: byte b of the group holds
 *    value 8g+b in its low nibble and value 8g+4+b in its high nibble; a nibble is sign (bit 3)
 *    and magnitude (bits 0-2), zero always as 0;
 *  - activations and the intermediate: the FP8 path's E4M3 per-token-group rule (above);
 *  - product per 128-wide K-block: the exact sum of decoded activation x integer weight products
 *    rounded once to fp32, then acc = acc + ((part * a_s[kb]) * w_s[n][kb]) in fp32, ascending
 *    K-blocks; after the sums the FP8 path's arithmetic (SiLU(gate) * up, FP8 requantization,
 *    combine). */

static int w4_nibble(int v) { return v < 0 ? (8 | -v) : v; }
static int w4_value(int nib) { return (nib & 8) ? -(nib & 7) : (nib & 7); }

/* Integer value of element k of a packed row. */
static int w4_at(const uint8_t* row, int64_t k) {
  const uint8_t byte = row[(k / 8) * 4 + (k % 4)];
  return w4_value((k % 8) < 4 ? (byte & 15) : (byte >> 4));
}

ORACLE_EXPORT void oracle_w4_unpack(const uint8_t* packed, int64_t rows, int64_t cols, int8_t* out) {
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t c = 0; c < cols; ++c) out[r * cols + c] = (int8_t)w4_at(packed + r * (cols / 2), c);
}

/* Int4 quantization of a row-major [rows, cols] fp32 matrix, one scale per (row, 128 columns);
 * cols a multiple of 128.  q: [rows, cols/2] packed bytes; s: [rows, cols/128]. */
ORACLE_EXPORT void oracle_w4_quant(const float* x, int64_t rows, int64_t cols, uint8_t* q, float* s) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    for (int64_t g0 = 0, gi = 0; g0 < cols; g0 += 128, ++gi) {
      float amax = 0.0f;
      for (int64_t c = g0; c < g0 + 128; ++c) {
        const float a = fabsf(x[r * cols + c]);
        if (a > amax) amax = a;
      }
      float sc = amax / 7.0f;
      if (sc < 1e-8f) sc = 1e-8f;
      s[r * (cols / 128) + gi] = sc;
      for (int64_t c = g0; c < g0 + 128; c += 8)
        for (int b = 0; b < 4; ++b) {
          int v[2];
          for (int h = 0; h < 2; ++h) {
            float t = nearbyintf(x[r * cols + c + 4 * h + b] / sc);
            if (t > 7.0f) t = 7.0f;
            if (t < -7.0f) t = -7.0f;
            v[h] = (int)t;
          }
          q[r * (cols / 2) + c / 2 + b] = (uint8_t)(w4_nibble(v[0]) | (w4_nibble(v[1]) << 4));
        }
    }
  }
}

/* One K-block of FP8 activations against int4 weights: exact, rounded once to fp32. */
static float w4_part(const uint8_t* a, const uint8_t* wrow, int64_t k0) {
  double sum = 0.0;
  for (int i = 0; i < 128; ++i) sum += e4m3_table[a[i]] * (double)w4_at(wrow, k0 + i);
  return (float)sum;
}

/* One expert row of the W4A8 first GEMM: a [H] FP8 codes, a_s [H/128], w13 [2I, H/2] packed,
 * w_s [2I, H/128]; writes h_q [I] FP8 codes and h_s [I/128]. */
static void w4_w13_row(const uint8_t* a, const float* a_s, const uint8_t* w13, const float* w_s, int64_t H,
                       int64_t I, float* hf, uint8_t* h_q, float* h_s) {
  const int64_t nkb = H / 128;
  for (int64_t n = 0; n < I; ++n) {
    float g = 0.0f, u = 0.0f;
    for (int64_t kb = 0; kb < nkb; ++kb) {
      const float pg = w4_part(a + kb * 128, w13 + n * (H / 2), kb * 128);
      const float pu = w4_part(a + kb * 128, w13 + (n + I) * (H / 2), kb * 128);
      g = g + ((pg * a_s[kb]) * w_s[n * nkb + kb]);
      u = u + ((pu * a_s[kb]) * w_s[(n + I) * nkb + kb]);
    }
    hf[n] = silu_mul(g, u);
  }
  fp8_requant_row(hf, I, h_q, h_s);
}

/* One expert row of the W4A8 second GEMM: y [H]. */
static void w4_w2_row(const uint8_t* hq, const float* h_s, const uint8_t* w2, const float* w_s, int64_t H,
                      int64_t I, float* y) {
  const int64_t nkb = I / 128;
  for (int64_t n = 0; n < H; ++n) {
    float acc = 0.0f;
    for (int64_t kb = 0; kb < nkb; ++kb) {
      const float part = w4_part(hq + kb * 128, w2 + n * (I / 2), kb * 128);
      acc = acc + ((part * h_s[kb]) * w_s[n * nkb + kb]);
    }
    y[n] = acc;
  }
}

/* W4A8 first GEMM over sorted rows (as oracle_fp8_w13_silu; w13[e] [2I, H/2] packed, w13_s[e]
 * [2I, H/128]). */
ORACLE_EXPORT void oracle_w4_w13_silu(const uint8_t* a_q, const float* a_s, const uint8_t* const* w13,
                                      const float* const* w13_s, const int32_t* sorted_pair_ids,
                                      const int32_t* tile_expert, int64_t block_m, int64_t T, int64_t k, int64_t H,
                                      int64_t I, const int64_t* rows, int64_t nrows, uint8_t* h_q, float* h_s) {
  e4m3_table_init();
  const int64_t P = T * k;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t i = 0; i < nrows; ++i) {
    const int64_t r = row_at(rows, i);
    const int64_t p = sorted_pair_ids[r];
    if (p >= P) continue;
    const int64_t t = p / k, e = tile_expert[r / block_m];
    float* hf = (float*)malloc(sizeof(float) * I);
    w4_w13_row(a_q + t * H, a_s + t * (H / 128), w13[e], w13_s[e], H, I, hf, h_q + r * I, h_s + r * (I / 128));
    free(hf);
  }
}

/* W4A8 second GEMM + top-k weighted combine (as oracle_fp8_w2_combine; w2[e] [H, I/2] packed,
 * w2_s[e] [H, I/128]). */
ORACLE_EXPORT void oracle_w4_w2_combine(const uint8_t* h_q, const float* h_s, const uint8_t* const* w2,
                                        const float* const* w2_s, const int32_t* sorted_pair_ids,
                                        const int32_t* tile_expert, int32_t num_tiles, int64_t block_m,
                                        const float* topk_weights, int64_t T, int64_t k, int64_t H, int64_t I,
                                        const int64_t* tokens, int64_t ntok, float* out) {
  e4m3_table_init();
  const int64_t P = T * k, R = (int64_t)num_tiles * block_m;
  int64_t* pair_row = (int64_t*)malloc(sizeof(int64_t) * (P > 0 ? P : 1));
  for (int64_t p = 0; p < P; ++p) pair_row[p] = -1;
  for (int64_t r = 0; r < R; ++r)
    if (sorted_pair_ids[r] < P) pair_row[sorted_pair_ids[r]] = r;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t i = 0; i < ntok; ++i) {
    const int64_t t = tokens ? tokens[i] : i;
    float* y = (float*)malloc(sizeof(float) * H);
    float* o = out + i * H;
    for (int64_t n = 0; n < H; ++n) o[n] = 0.0f;
    for (int64_t j = 0; j < k; ++j) {
      const int64_t r = pair_row[t * k + j];
      if (r < 0) continue;
      const int64_t e = tile_expert[r / block_m];
      w4_w2_row(h_q + r * I, h_s + r * (I / 128), w2[e], w2_s[e], H, I, y);
      const float wj = topk_weights[t * k + j];
      for (int64_t n = 0; n < H; ++n) o[n] = o[n] + (wj * y[n]);
    }
    free(y);
  }
  free(pair_row);
}

/* The whole W4A8 layer for a list of tokens, straight from the routing. */
ORACLE_EXPORT void oracle_w4_moe_tokens(const float* x, int64_t ntok, int64_t H, int64_t I, int64_t k,
                                        const int32_t* ids, const float* topk_weights, const uint8_t* const* w13,
                                        const float* const* w13_s, const uint8_t* const* w2,
                                        const float* const* w2_s, float* out) {
  e4m3_table_init();
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t t = 0; t < ntok; ++t) {
    uint8_t* aq = (uint8_t*)malloc(H);
    float* as = (float*)malloc(sizeof(float) * (H / 128));
    float* hf = (float*)malloc(sizeof(float) * I);
    uint8_t* hq = (uint8_t*)malloc(I);
    float* hs = (float*)malloc(sizeof(float) * (I / 128));
    float* y = (float*)malloc(sizeof(float) * H);
    fp8_requant_row(x + t * H, H, aq, as);
    float* o = out + t * H;
    for (int64_t n = 0; n < H; ++n) o[n] = 0.0f;
    for (int64_t j = 0; j < k; ++j) {
      const int64_t e = ids[t * k + j];
      w4_w13_row(aq, as, w13[e], w13_s[e], H, I, hf, hq, hs);
      w4_w2_row(hq, hs, w2[e], w2_s[e], H, I, y);
      const float wj = topk_weights[t * k + j];
      for (int64_t n = 0; n < H; ++n) o[n] = o[n] + (wj * y[n]);
    }
    free(aq);
    free(as);
    free(hf);
    free(hq);
    free(hs);
    free(y);
  }
}
