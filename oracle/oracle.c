/*
 * oracle.c -- plain, slow, fp64 CPU reference of one sparse Mixture-of-Experts
 * FFN layer.  TEST INFRASTRUCTURE ONLY: only the test-suite, the smoke check
 * and the CPU-baseline leg of the benchmark may load it.  It shares no code,
 * header, table or constant with the GPU library and includes nothing from it.
 *
 * What it follows (cited by page title and section):
 *  - "15. DeepSeek：MLA、MoE 与 MTP", section "V3 的 MoE：256 个专家怎样选 8 个":
 *    sigmoid scores of the router logits, a selection-only bias, groups of
 *    E/G experts scored by the sum of their two best biased scores, the best
 *    topk_group groups kept, top-k experts chosen among the kept groups, gates
 *    = unbiased scores of the chosen experts renormalised and multiplied by the
 *    routed scaling factor, output = gate-weighted sum of the chosen experts
 *    plus the shared experts.
 *  - "MoE架构揭秘：大模型参数激活率与专家路由机制解析", section 3.1: router =
 *    linear layer to E logits, softmax, top-k.
 *  - "GPT-4 Has 1.8 Trillion Parameters. It Uses 2% of Them Per Token",
 *    section 2.2 (expert capacity): an expert accepts at most C tokens; tokens
 *    beyond it go to their next-best expert; its MoEBlock sketch takes the
 *    softmax over the top-k logits, i.e. renormalised softmax gates.
 *  - same DeepSeek page, section "671B 和 37B 的参数账": an expert is three
 *    H x I matrices (gate, up, down); the router is E x H.
 *  - "MoE on KnightLi的博客", activation-function section: SwiGLU expert FFN.
 *  - same DeepSeek page, section "V4：放弃潜向量，改用压缩注意力", the FFN
 *    paragraph, and the page's table of generations: V4 scores with
 *    sqrt(softplus(l)) plus the selection bias and no group limit, and its
 *    first layers choose experts by a fixed token-id table (tid2eid) with the
 *    router only weighting them.
 *
 * Readings where the pages are silent (each also listed in the design notes):
 *  - ties in every ranking are broken by the lower index;
 *  - softmax routing selects on the fp32 logits (softmax is monotone);
 *  - selection always works on fp32 values; sigmoid selection uses the fp32
 *    sigmoid defined below (sigmoid32) so that it is reproducible bit for bit;
 *  - capacity C = ceil(((cf*T)*k)/E) in IEEE double, tokens served first come
 *    first served in index order, each taking its best-ranked allowed experts
 *    that still have room; slots left empty get index -1 and gate 0; groups
 *    are not re-chosen after overflow; gates are computed on the final set.
 *    Parity unpinned: the pages fix that an expert takes at most C tokens and
 *    that overflow moves to the next-best expert (both pinned), not which
 *    tokens are served first; the index order is checked only against a
 *    brute-force walk written from the same reading;
 *  - drop mode (the same page's serving configuration, section 4.2: the
 *    drop_tokens switch, overflow is dropped rather than sent to a lesser
 *    expert): each token keeps its top-k and the gates of that top-k; in
 *    token order a
 *    (token, expert) assignment is kept while the expert holds fewer than C
 *    tokens, else it is dropped (index -1, gate 0, no other expert instead,
 *    the other gates unchanged);
 *  - sqrt(softplus) scoring (same DeepSeek page, V4 section: softplus, then a
 *    square root, in place of the sigmoid, with the selection bias and no
 *    group limit): selected on the fp32 function sqrtsoftplus32 below, gates
 *    from the unbiased fp64 value renormalised over the chosen experts and
 *    scaled, as for sigmoid scoring;
 *  - hash routing (same section: a fixed token-id -> experts table chooses,
 *    the router only weights): an id outside the table chooses nothing, a
 *    table entry outside [0, E) or repeating an earlier entry of its row
 *    leaves its slot empty, the gates are those of the configured scoring
 *    over the table's experts, and a capacity limit can only drop;
 *  - shared expert s for token t lives at row T*k + s*T + t of the row space.
 *
 * Arithmetic: every dot product, activation, gate and sum is evaluated in
 * double from the exact input values; the router logits are rounded once to
 * fp32 because selection is defined on fp32 logits.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
  int32_t H, E, S, k, G, topk_group, I;
  int32_t scoring;          /* 0 = softmax, 1 = sigmoid, 2 = sqrt(softplus)   */
  int32_t renorm;           /* 1 = renormalise the selected gates             */
  double scale;             /* routed scaling factor                          */
  double capacity_factor;   /* <= 0 : no capacity limit                       */
  int32_t dtype;            /* 0 = fp32 inputs, 1 = bf16 inputs (bit patterns) */
  int32_t drop_tokens;      /* with a capacity: 1 = drop overflow, 0 = re-route */
} oracle_layer;

/* ---- input access --------------------------------------------------------- */

static double bf16_to_double(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* element i of a row-major array of fp32 (dtype 0) or bf16 bits (dtype 1) */
static double elem(const void* base, int dtype, int64_t i) {
  if (dtype == 1) return bf16_to_double(((const uint16_t*)base)[i]);
  return (double)((const float*)base)[i];
}

/* ---- fp32 sigmoid used for selection -------------------------------------- */
/* exp32(z) for z <= 0: Cody-Waite reduction z = n*ln2 + r with n = rint(z*log2e)
 * and ln2 split in a high and a low part, e^r by the degree-7 Taylor polynomial
 * (coefficients 1/j! rounded to fp32) in Horner form with fused multiply-adds,
 * and a final exact scaling by 2^n.  Every step is one correctly rounded IEEE
 * fp32 operation, so the result is fixed bit for bit by this description. */
static const float EXP32_LOG2E = 0x1.715476p+0f;
static const float EXP32_LN2_HI = 0x1.62e4p-1f;
static const float EXP32_LN2_LO = 0x1.7f7d1cp-20f;
static const float EXP32_C[8] = {0x1p+0f,       0x1p+0f,       0x1p-1f,       0x1.555556p-3f,
                                 0x1.555556p-5f, 0x1.111112p-7f, 0x1.6c16c2p-10f, 0x1.a01a02p-13f};

float oracle_exp32(float z) {
  float t = z * EXP32_LOG2E;
  float n = rintf(t);
  float r = fmaf(-n, EXP32_LN2_HI, z);
  r = fmaf(-n, EXP32_LN2_LO, r);
  float p = EXP32_C[7];
  for (int j = 6; j >= 0; --j) p = fmaf(p, r, EXP32_C[j]);
  return ldexpf(p, (int)n);
}

/* sigmoid32(l): clamp l to [-80, 80]; for l >= 0, 1/(1 + exp32(-l)); for
 * l < 0, e/(1 + e) with e = exp32(l).  The clamp keeps every intermediate a
 * normal fp32 number. */
float oracle_sigmoid32(float l) {
  if (l > 80.0f) l = 80.0f;
  if (l < -80.0f) l = -80.0f;
  if (l >= 0.0f) {
    float e = oracle_exp32(-l);
    float d = 1.0f + e;
    return 1.0f / d;
  } else {
    float e = oracle_exp32(l);
    float d = 1.0f + e;
    return e / d;
  }
}

void oracle_sigmoid32_array(int64_t n, const float* in, float* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_sigmoid32(in[i]);
}

void oracle_exp32_array(int64_t n, const float* in, float* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_exp32(in[i]);
}

/* ---- fp32 sqrt(softplus) used for selection ------------------------------- */
/* log(1 + u) for 0 < u <= 1 from log(1+u) = 2 atanh(z), z = u / (2 + u) in
 * (0, 1/3]: atanh(z) = z * sum_j w^j / (2j + 1) with w = z^2 <= 1/9, summed
 * through the w^7 term (the first omitted term is below 2^-26 of the sum).
 * Coefficients 1/(2j+1) rounded to fp32, Horner form with fused multiply-adds,
 * every step one correctly rounded fp32 operation. */
static const float LOG1P32_C[8] = {0x1p+0f,        0x1.555556p-2f, 0x1.99999ap-3f, 0x1.24924ap-3f,
                                   0x1.c71c72p-4f, 0x1.745d18p-4f, 0x1.3b13b2p-4f, 0x1.111112p-4f};

static float log1p32_unit(float u) {
  float d = 2.0f + u;
  float z = u / d;
  float w = z * z;
  float q = LOG1P32_C[7];
  for (int j = 6; j >= 0; --j) q = fmaf(q, w, LOG1P32_C[j]);
  float z2 = z + z;
  return z2 * q;
}

/* sqrtsoftplus32(l) = sqrt(max(l, 0) + log1p32(exp32(-a))), a = min(|l|, 80):
 * softplus(l) = max(l, 0) + log(1 + e^-|l|) keeps every intermediate normal;
 * below l = -80 the value stays at that of -80.  The square root is the
 * correctly rounded fp32 one. */
float oracle_sqrtsoftplus32(float l) {
  float a = fabsf(l);
  if (a > 80.0f) a = 80.0f;
  float u = oracle_exp32(-a);
  float sp = (l > 0.0f ? l : 0.0f) + log1p32_unit(u);
  return sqrtf(sp);
}

void oracle_sqrtsoftplus32_array(int64_t n, const float* in, float* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_sqrtsoftplus32(in[i]);
}

/* ---- router logits -------------------------------------------------------- */
/* logits[t,e] = fl32( sum_h x[t,h] * w_router[e,h] + logit_bias[e] ) */
int oracle_router_logits(const oracle_layer* L, int64_t T, const void* x, const void* w_router,
                         const float* logit_bias, float* logits) {
  const int64_t H = L->H, E = L->E;
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t) {
    for (int64_t e = 0; e < E; ++e) {
      double acc = 0.0;
      for (int64_t h = 0; h < H; ++h) acc += elem(x, L->dtype, t * H + h) * elem(w_router, L->dtype, e * H + h);
      if (logit_bias) acc += (double)logit_bias[e];
      logits[t * E + e] = (float)acc;
    }
  }
  return 0;
}

/* ---- selection ------------------------------------------------------------ */

/* a ranks before b: higher value first, lower index on equal values */
static int ranks_before(float va, int ia, float vb, int ib) { return va > vb || (va == vb && ia < ib); }

/* Sort ids[0..n) by (value desc, index asc).  Plain insertion sort: n <= a few
 * hundred and it keeps the code free of shared state. */
static void rank_sort(int* ids, int n, const float* v) {
  for (int i = 1; i < n; ++i) {
    int cur = ids[i], j = i - 1;
    while (j >= 0 && ranks_before(v[cur], cur, v[ids[j]], ids[j])) {
      ids[j + 1] = ids[j];
      --j;
    }
    ids[j + 1] = cur;
  }
}

static double sigmoid64(double l) { return 1.0 / (1.0 + exp(-l)); }

/* sqrt(softplus(l)) in double, softplus(l) = max(l, 0) + log1p(exp(-|l|)) */
static double sqrtsoftplus64(double l) { return sqrt((l > 0.0 ? l : 0.0) + log1p(exp(-fabs(l)))); }

/* unbiased score of the gates: sigmoid (scoring 1) or sqrt(softplus) (2) */
static double gate_score64(const oracle_layer* L, float l) {
  return L->scoring == 2 ? sqrtsoftplus64((double)l) : sigmoid64((double)l);
}

/* Per token: the selection score of each expert (fp32), the allowed set after
 * group limiting, the allowed experts in rank order, and the selection margin.
 * Returns the number of allowed experts written to `order`. */
static int token_ranking(const oracle_layer* L, const float* logit, const float* sel_bias, float* score,
                         int* order, double* margin) {
  const int E = L->E, G = L->G;
  for (int e = 0; e < E; ++e) {
    if (L->scoring == 1 || L->scoring == 2) {
      float s = L->scoring == 1 ? oracle_sigmoid32(logit[e]) : oracle_sqrtsoftplus32(logit[e]);
      float b = sel_bias ? sel_bias[e] : 0.0f;
      score[e] = s + b; /* fp32 addition */
    } else {
      score[e] = logit[e];
    }
  }
  double m = INFINITY;
  int n_allowed = 0;
  if (G > 1) {
    const int gsz = E / G;
    float gscore[1024];
    int gid[1024];
    for (int g = 0; g < G; ++g) {
      /* best and second best biased score of the group; an equal value at a
       * second index counts as the second best */
      int best = g * gsz;
      for (int e = g * gsz + 1; e < (g + 1) * gsz; ++e)
        if (ranks_before(score[e], e, score[best], best)) best = e;
      int second = -1;
      for (int e = g * gsz; e < (g + 1) * gsz; ++e) {
        if (e == best) continue;
        if (second < 0 || ranks_before(score[e], e, score[second], second)) second = e;
      }
      gscore[g] = score[best] + score[second]; /* fp32 addition */
      gid[g] = g;
    }
    rank_sort(gid, G, gscore);
    if (L->topk_group < G) m = (double)gscore[gid[L->topk_group - 1]] - (double)gscore[gid[L->topk_group]];
    int kept[1024];
    memset(kept, 0, sizeof(int) * (size_t)G);
    for (int i = 0; i < L->topk_group; ++i) kept[gid[i]] = 1;
    for (int e = 0; e < E; ++e)
      if (kept[e / gsz]) order[n_allowed++] = e;
  } else {
    for (int e = 0; e < E; ++e) order[n_allowed++] = e;
  }
  rank_sort(order, n_allowed, score);
  if (n_allowed > L->k) {
    double d = (double)score[order[L->k - 1]] - (double)score[order[L->k]];
    if (d < m) m = d;
  }
  if (margin) *margin = m;
  return n_allowed;
}

/* Gates of one token over its final selection idx[0..k) (-1 = empty slot). */
static void token_gates(const oracle_layer* L, const float* logit, const int32_t* idx, double* w) {
  const int k = L->k, E = L->E;
  if (L->scoring == 1 || L->scoring == 2) {
    double sum = 0.0;
    for (int j = 0; j < k; ++j)
      if (idx[j] >= 0) sum += gate_score64(L, logit[idx[j]]);
    for (int j = 0; j < k; ++j) {
      if (idx[j] < 0) {
        w[j] = 0.0;
        continue;
      }
      double s = gate_score64(L, logit[idx[j]]);
      w[j] = (L->renorm ? s / sum : s) * L->scale;
    }
  } else {
    /* softmax over all E logits; renormalised over the selected experts when
     * asked (equal to a softmax over the selected logits only) */
    double mx = -INFINITY;
    for (int e = 0; e < E; ++e)
      if ((double)logit[e] > mx) mx = (double)logit[e];
    double z_all = 0.0, z_sel = 0.0;
    for (int e = 0; e < E; ++e) z_all += exp((double)logit[e] - mx);
    for (int j = 0; j < k; ++j)
      if (idx[j] >= 0) z_sel += exp((double)logit[idx[j]] - mx);
    for (int j = 0; j < k; ++j) {
      if (idx[j] < 0) {
        w[j] = 0.0;
        continue;
      }
      double p = exp((double)logit[idx[j]] - mx);
      w[j] = (L->renorm ? p / z_sel : p / z_all) * L->scale;
    }
  }
}

/* Capacity of every expert: ceil(((cf*T)*k)/E) in IEEE double, left to right. */
int64_t oracle_capacity(const oracle_layer* L, int64_t T) {
  if (!(L->capacity_factor > 0.0)) return -1;
  double c = ceil(L->capacity_factor * (double)T * (double)L->k / (double)L->E);
  return (int64_t)c;
}

/* Selection of every token: idx[T,k] (rank order, -1 = empty slot), gates w[T,k]
 * (double) and margin[T] (NULL allowed).  With a capacity limit the tokens are
 * processed in index order and every token takes the best-ranked allowed
 * experts whose count is still below C. */
int oracle_select(const oracle_layer* L, int64_t T, const float* logits, const float* sel_bias, int32_t* idx,
                  double* w, double* margin, int32_t* counts_out) {
  const int E = L->E, k = L->k;
  if (E > 4096 || L->G > 1024) return -1;
  const int64_t cap = oracle_capacity(L, T);
  if (cap < 0) {
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
      float score[4096];
      int order[4096];
      int n = token_ranking(L, logits + t * E, sel_bias, score, order, margin ? margin + t : NULL);
      for (int j = 0; j < k; ++j) idx[t * k + j] = j < n ? order[j] : -1;
      token_gates(L, logits + t * E, idx + t * k, w + t * k);
    }
  } else if (L->drop_tokens) {
    /* the top-k and its gates as without a limit, then, token by token, an
     * assignment to an expert that already holds C tokens is dropped */
    int64_t* count = (int64_t*)calloc((size_t)E, sizeof(int64_t));
    float* score = (float*)malloc(sizeof(float) * (size_t)E);
    int* order = (int*)malloc(sizeof(int) * (size_t)E);
    for (int64_t t = 0; t < T; ++t) {
      int n = token_ranking(L, logits + t * E, sel_bias, score, order, margin ? margin + t : NULL);
      for (int j = 0; j < k; ++j) idx[t * k + j] = j < n ? order[j] : -1;
      token_gates(L, logits + t * E, idx + t * k, w + t * k);
      for (int j = 0; j < k; ++j) {
        int e = idx[t * k + j];
        if (e < 0) continue;
        if (count[e] < cap) {
          count[e] += 1;
        } else {
          idx[t * k + j] = -1;
          w[t * k + j] = 0.0;
        }
      }
    }
    free(count);
    free(score);
    free(order);
  } else {
    int64_t* count = (int64_t*)calloc((size_t)E, sizeof(int64_t));
    float* score = (float*)malloc(sizeof(float) * (size_t)E);
    int* order = (int*)malloc(sizeof(int) * (size_t)E);
    for (int64_t t = 0; t < T; ++t) {
      int n = token_ranking(L, logits + t * E, sel_bias, score, order, margin ? margin + t : NULL);
      int got = 0;
      for (int r = 0; r < n && got < k; ++r) {
        int e = order[r];
        if (count[e] < cap) {
          idx[t * k + got++] = e;
          count[e] += 1;
        }
      }
      for (int j = got; j < k; ++j) idx[t * k + j] = -1;
      token_gates(L, logits + t * E, idx + t * k, w + t * k);
    }
    free(count);
    free(score);
    free(order);
  }
  if (counts_out) {
    memset(counts_out, 0, sizeof(int32_t) * (size_t)E);
    for (int64_t i = 0; i < T * k; ++i)
      if (idx[i] >= 0) counts_out[idx[i]] += 1;
  }
  return 0;
}

/* ---- hash routing ----------------------------------------------------------- */
/* Experts of token t read from a fixed table: row token_ids[t] of tid2eid
 * [vocab, k]; the logits only give the gates (token_gates over that set).
 * An id outside [0, vocab) chooses nothing; an entry outside [0, E) or equal
 * to an earlier entry of its row leaves its slot empty (-1, gate 0).  With a
 * capacity limit only drop mode applies (there is no next-best expert): in
 * token order an assignment to an expert that already holds C tokens is
 * dropped.  Returns -2 for a re-route capacity, -1 for a bad shape. */
int oracle_hash_select(const oracle_layer* L, int64_t T, const float* logits, const int32_t* token_ids,
                       const int32_t* tid2eid, int64_t vocab, int32_t* idx, double* w, int32_t* counts_out) {
  const int E = L->E, k = L->k;
  if (E > 4096 || k < 1 || vocab < 0) return -1;
  const int64_t cap = oracle_capacity(L, T);
  if (cap >= 0 && !L->drop_tokens) return -2;
  for (int64_t t = 0; t < T; ++t) {
    const int64_t id = token_ids[t];
    for (int j = 0; j < k; ++j) {
      int e = -1;
      if (id >= 0 && id < vocab) {
        e = tid2eid[id * k + j];
        if (e < 0 || e >= E) e = -1;
        for (int i = 0; i < j && e >= 0; ++i)
          if (tid2eid[id * k + i] == e) e = -1;
      }
      idx[t * k + j] = e;
    }
    token_gates(L, logits + t * E, idx + t * k, w + t * k);
  }
  if (cap >= 0) {
    int64_t* held = (int64_t*)calloc((size_t)E, sizeof(int64_t));
    for (int64_t i = 0; i < T * k; ++i) {
      const int e = idx[i];
      if (e < 0) continue;
      if (held[e] >= cap) {
        idx[i] = -1; /* the expert is full: this assignment is dropped */
        w[i] = 0.0;
      } else {
        held[e] += 1;
      }
    }
    free(held);
  }
  if (counts_out) {
    memset(counts_out, 0, sizeof(int32_t) * (size_t)E);
    for (int64_t i = 0; i < T * k; ++i)
      if (idx[i] >= 0) counts_out[idx[i]] += 1;
  }
  return 0;
}

/* ---- permutation ------------------------------------------------------------ */
/* Rows of the routed experts ordered by (expert asc, token asc):
 * counts[e], offsets[0..E] (exclusive prefix sum), row_token[row] = token,
 * slot_row[t*k+j] = row of (t, slot j) or -1 for an empty slot.  Shared expert
 * s takes rows T*k + s*T + t, so row_token has T*k + S*T entries (entries
 * between offsets[E] and T*k are -1). */
int oracle_permute(const oracle_layer* L, int64_t T, const int32_t* idx, int32_t* counts, int32_t* offsets,
                   int32_t* row_token, int32_t* slot_row) {
  const int E = L->E, k = L->k, S = L->S;
  memset(counts, 0, sizeof(int32_t) * (size_t)E);
  for (int64_t i = 0; i < T * k; ++i) {
    if (idx[i] < -1 || idx[i] >= E) return -1;
    if (idx[i] >= 0) counts[idx[i]] += 1;
  }
  offsets[0] = 0;
  for (int e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
  for (int64_t r = 0; r < T * k + (int64_t)S * T; ++r) row_token[r] = -1;
  int32_t* fill = (int32_t*)calloc((size_t)E, sizeof(int32_t));
  for (int e = 0; e < E; ++e) fill[e] = offsets[e];
  for (int64_t t = 0; t < T; ++t) {
    for (int j = 0; j < k; ++j) {
      int e = idx[t * k + j];
      if (e < 0) {
        slot_row[t * k + j] = -1;
        continue;
      }
      int32_t r = fill[e]++;
      row_token[r] = (int32_t)t;
      slot_row[t * k + j] = r;
    }
  }
  free(fill);
  for (int s = 0; s < S; ++s)
    for (int64_t t = 0; t < T; ++t) row_token[T * k + (int64_t)s * T + t] = (int32_t)t;
  return 0;
}

/* ---- experts ---------------------------------------------------------------- */
/* One SwiGLU expert on one row: y = W_down (silu(W_gate x) * (W_up x)),
 * silu(g) = g * sigmoid(g); w_gate, w_up are [I,H] and w_down is [H,I]. */
static void swiglu_row(const oracle_layer* L, const void* x, int64_t x_off, const void* wg, const void* wu,
                       const void* wd, double* hbuf, double* y) {
  const int64_t H = L->H, I = L->I;
  for (int64_t i = 0; i < I; ++i) {
    double g = 0.0, u = 0.0;
    for (int64_t h = 0; h < H; ++h) {
      double xv = elem(x, L->dtype, x_off + h);
      g += elem(wg, L->dtype, i * H + h) * xv;
      u += elem(wu, L->dtype, i * H + h) * xv;
    }
    hbuf[i] = g * sigmoid64(g) * u;
  }
  for (int64_t n = 0; n < H; ++n) {
    double acc = 0.0;
    for (int64_t i = 0; i < I; ++i) acc += elem(wd, L->dtype, n * I + i) * hbuf[i];
    y[n] = acc;
  }
}

/* y[r,:] = expert(x_rows[r,:]) for n rows of one expert. */
int oracle_expert_rows(const oracle_layer* L, int64_t n, const void* x_rows, const void* wg, const void* wu,
                       const void* wd, double* y) {
  const int64_t H = L->H;
#pragma omp parallel
  {
    double* hbuf = (double*)malloc(sizeof(double) * (size_t)L->I);
#pragma omp for schedule(dynamic, 1)
    for (int64_t r = 0; r < n; ++r) swiglu_row(L, x_rows, r * H, wg, wu, wd, hbuf, y + r * H);
    free(hbuf);
  }
  return 0;
}

/* Layer output of the listed tokens:
 *   out[i,:] = sum_j w[t,j] * expert_{idx[t,j]}(x[t]) + sum_s shared_s(x[t]),
 * t = tokens[i], empty slots skipped.  Expert e's matrices are wg[e], wu[e],
 * wd[e] (pointer arrays of length E+S, shared experts after the routed ones;
 * entries no listed token needs may be NULL). */
int oracle_forward_tokens(const oracle_layer* L, int64_t n_tok, const int64_t* tokens, const void* x,
                          const int32_t* idx, const double* w, const void* const* wg, const void* const* wu,
                          const void* const* wd, double* out) {
  const int64_t H = L->H;
  const int k = L->k, E = L->E, S = L->S;
  int bad = 0;
#pragma omp parallel
  {
    double* hbuf = (double*)malloc(sizeof(double) * (size_t)L->I);
    double* y = (double*)malloc(sizeof(double) * (size_t)H);
#pragma omp for schedule(dynamic, 1)
    for (int64_t i = 0; i < n_tok; ++i) {
      const int64_t t = tokens[i];
      double* o = out + i * H;
      for (int64_t n = 0; n < H; ++n) o[n] = 0.0;
      for (int j = 0; j < k; ++j) {
        const int e = idx[t * k + j];
        if (e < 0) continue;
        if (!wg[e] || !wu[e] || !wd[e]) {
#pragma omp atomic write
          bad = 1;
          continue;
        }
        swiglu_row(L, x, t * H, wg[e], wu[e], wd[e], hbuf, y);
        for (int64_t n = 0; n < H; ++n) o[n] += w[t * k + j] * y[n];
      }
      for (int s = 0; s < S; ++s) {
        const int e = E + s;
        if (!wg[e] || !wu[e] || !wd[e]) {
#pragma omp atomic write
          bad = 1;
          continue;
        }
        swiglu_row(L, x, t * H, wg[e], wu[e], wd[e], hbuf, y);
        for (int64_t n = 0; n < H; ++n) o[n] += y[n];
      }
    }
    free(hbuf);
    free(y);
  }
  return bad ? -1 : 0;
}

/* Combine over the row space: out[t,:] = sum_j w[t,j] * y_rows[slot_row[t,j],:]
 * (empty slots skipped) + sum_s y_rows[T*k + s*T + t,:], in double. */
int oracle_combine(const oracle_layer* L, int64_t T, const double* y_rows, const int32_t* slot_row, const double* w,
                   double* out) {
  const int64_t H = L->H;
  const int k = L->k, S = L->S;
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t) {
    double* o = out + t * H;
    for (int64_t n = 0; n < H; ++n) o[n] = 0.0;
    for (int j = 0; j < k; ++j) {
      const int32_t r = slot_row[t * k + j];
      if (r < 0) continue;
      for (int64_t n = 0; n < H; ++n) o[n] += w[t * k + j] * y_rows[(int64_t)r * H + n];
    }
    for (int s = 0; s < S; ++s) {
      const int64_t r = T * k + (int64_t)s * T + t;
      for (int64_t n = 0; n < H; ++n) o[n] += y_rows[r * H + n];
    }
  }
  return 0;
}

/* ---- load balancing ---------------------------------------------------------- */
/* One step of the auxiliary-loss-free balancing ("15. DeepSeek：MLA、MoE 与 MTP",
 * section "V3 的 MoE：256 个专家怎样选 8 个", the paragraph on the bias): an
 * expert that received more tokens than the mean over the experts has its
 * selection bias lowered by gamma, one that received fewer has it raised, one
 * exactly at the mean keeps it (reading: the page names only overloaded and
 * idle experts).  The bias is fp32 state, so the step is one fp32 rounding:
 * b <- fl32(b - gamma) or fl32(b + gamma).  The mean test is exact integer
 * arithmetic: n_e > N/E  <=>  n_e * E > N.
 * Load telemetry (the same section's monitoring paragraph; the expert-call
 * entropy of "GPT-4稀疏激活原理：2%参数调用背后的MoE工程实践", section 4.4):
 * share[e] = n_e / N, stats = {entropy -sum share*ln(share) in nats (0*ln 0 =
 * 0), largest share, experts above the mean, experts below the mean}.  N == 0:
 * no update, shares 0, entropy 0. */
int oracle_balance_update(int E, const int32_t* counts, float* bias, float gamma, double* share, double* stats) {
  int64_t N = 0;
  for (int e = 0; e < E; ++e) {
    if (counts[e] < 0) return -1;
    N += counts[e];
  }
  double ent = 0.0, mx = 0.0;
  int over = 0, under = 0;
  for (int e = 0; e < E; ++e) {
    const int64_t scaled = (int64_t)counts[e] * E;
    if (N > 0 && scaled > N) {
      bias[e] = bias[e] - gamma;
      over += 1;
    } else if (N > 0 && scaled < N) {
      bias[e] = bias[e] + gamma;
      under += 1;
    }
    const double p = N > 0 ? (double)counts[e] / (double)N : 0.0;
    if (share) share[e] = p;
    if (p > 0.0) ent -= p * log(p);
    if (p > mx) mx = p;
  }
  if (stats) {
    stats[0] = ent;
    stats[1] = mx;
    stats[2] = over;
    stats[3] = under;
  }
  return 0;
}

/* ---- FP8 (e4m3) experts with block scales ------------------------------------ */
/* "15. DeepSeek：MLA、MoE 与 MTP", section "FP8 训练是训练配方，不是架构": matrix
 * multiplication inputs in E4M3, one scale per 1 x 128 tile of activations and
 * per 128 x 128 block of weights; V3.1 stores the scales as UE8M0 (an 8-bit
 * exponent).  Readings: every scale (weights' and activations') is UE8M0,
 * value 2^(b - 127); E4M3 is the format with 4 exponent bits (bias 7), 3
 * mantissa bits, subnormals, maximum 448 and no infinities (S.1111.111 is
 * NaN); an activation tile's scale is the smallest power of two 2^p with
 * amax / 2^p <= 448 (p >= -127; an all-zero or subnormal-only tile takes
 * p = -127), and each element's code is its value / 2^p rounded to the
 * nearest E4M3 value, ties to the even mantissa, the sign kept (also on
 * zero).  The decision is taken on fp32 values: x is bf16 (exact in fp32),
 * the SwiGLU output h is rounded from double to fp32 first. */

double oracle_e4m3_value(int c) {
  c &= 0xFF;
  const int e = (c >> 3) & 15, m = c & 7;
  if (e == 15 && m == 7) return NAN;
  const double v = e == 0 ? ldexp((double)m, -9) : ldexp((double)(8 + m), e - 10);
  return (c & 0x80) ? -v : v;
}

double oracle_e8m0_value(int b) {
  b &= 0xFF;
  return b == 255 ? NAN : ldexp(1.0, b - 127);
}

/* exponent p of the UE8M0 scale of a tile whose largest magnitude is amax */
static int tile_scale_exp(float amax) {
  if (!(amax >= 0x1p-126f)) return -127; /* zero or subnormal */
  int ex;
  const double f = frexp((double)amax, &ex); /* amax = f * 2^ex, f in [0.5, 1) */
  const int E = ex - 1;                      /* amax = M * 2^E, M in [1, 2) */
  const double M = 2.0 * f;
  int p = E - 8 + (M > 1.75 ? 1 : 0);       /* 448 = 1.75 * 2^8 */
  return p < -127 ? -127 : p;
}

/* nearest E4M3 code of v (|v| <= 448), ties to the even mantissa */
static uint8_t e4m3_round(double v) {
  const uint8_t sign = signbit(v) ? 0x80 : 0;
  const double a = fabs(v);
  double spacing;
  if (a < 0x1p-6) {
    spacing = 0x1p-9;
  } else {
    int ex;
    frexp(a, &ex);
    spacing = ldexp(1.0, ex - 1 - 3);
  }
  const double q = nearbyint(a / spacing); /* a / spacing is exact; rounding mode: nearest-even */
  const double r = q * spacing;
  if (r == 0.0) return sign;
  if (r < 0x1p-6) return (uint8_t)(sign | (int)(r / 0x1p-9));
  int ex;
  frexp(r, &ex);
  const int E = ex - 1;
  const int m = (int)((r / ldexp(1.0, E) - 1.0) * 8.0);
  return (uint8_t)(sign | ((E + 7) << 3) | m);
}

/* Quantise rows x K fp32 values (K % 128 == 0) in 1 x 128 tiles: codes
 * [rows, K] and scale bytes at scales[r * scale_stride + K-tile]. */
int oracle_quantize_e4m3(int64_t rows, int64_t K, const float* in, uint8_t* codes, uint8_t* scales,
                         int64_t scale_stride) {
  if (K % 128 != 0 || scale_stride < K / 128) return -1;
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t kb = 0; kb < K / 128; ++kb) {
      const float* v = in + r * K + kb * 128;
      float amax = 0.0f;
      for (int i = 0; i < 128; ++i)
        if (fabsf(v[i]) > amax) amax = fabsf(v[i]);
      const int p = tile_scale_exp(amax);
      scales[r * scale_stride + kb] = (uint8_t)(p + 127);
      for (int i = 0; i < 128; ++i) codes[r * K + kb * 128 + i] = e4m3_round(ldexp((double)v[i], -p));
    }
  return 0;
}

void oracle_e4m3_values(int64_t n, const uint8_t* codes, double* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_e4m3_value(codes[i]);
}

/* value of element (row, col) of a block-scaled FP8 matrix [rows, cols]:
 * code * 2^(scale[row/128, col/128] - 127) */
static double fp8_weight(const uint8_t* codes, const uint8_t* scales, int64_t cols, int64_t row, int64_t col) {
  return oracle_e4m3_value(codes[row * cols + col]) *
         oracle_e8m0_value(scales[(row / 128) * (cols / 128) + col / 128]);
}

/* One expert on one token, FP8: x (bf16 bits [H]) quantised in 1 x 128
 * tiles; g, u = dot products of the dequantised values in double; h =
 * silu(g) * u rounded to fp32 and quantised in 1 x 128 tiles; y = W_down h
 * over the dequantised values in double. */
static void swiglu_row_fp8(const oracle_layer* L, const double* xq, const uint8_t* wg, const uint8_t* sg,
                           const uint8_t* wu, const uint8_t* su, const uint8_t* wd, const uint8_t* sd, float* hbuf,
                           uint8_t* hcodes, uint8_t* hscales, double* y) {
  const int64_t H = L->H, I = L->I;
  for (int64_t i = 0; i < I; ++i) {
    double g = 0.0, u = 0.0;
    for (int64_t h = 0; h < H; ++h) {
      g += fp8_weight(wg, sg, H, i, h) * xq[h];
      u += fp8_weight(wu, su, H, i, h) * xq[h];
    }
    hbuf[i] = (float)(g * sigmoid64(g) * u);
  }
  oracle_quantize_e4m3(1, I, hbuf, hcodes, hscales, I / 128);
  for (int64_t n = 0; n < H; ++n) {
    double acc = 0.0;
    for (int64_t i = 0; i < I; ++i)
      acc += fp8_weight(wd, sd, I, n, i) * oracle_e4m3_value(hcodes[i]) * oracle_e8m0_value(hscales[i / 128]);
    y[n] = acc;
  }
}

/* Layer output of the listed tokens with FP8 experts (as
 * oracle_forward_tokens): x is bf16 bits [T,H]; expert e's matrices are the
 * codes wg[e], wu[e] [I,H], wd[e] [H,I] with scale bytes sg[e], su[e]
 * [I/128, H/128] and sd[e] [H/128, I/128]. */
int oracle_forward_tokens_fp8(const oracle_layer* L, int64_t n_tok, const int64_t* tokens, const uint16_t* x,
                              const int32_t* idx, const double* w, const uint8_t* const* wg, const uint8_t* const* sg,
                              const uint8_t* const* wu, const uint8_t* const* su, const uint8_t* const* wd,
                              const uint8_t* const* sd, double* out) {
  const int64_t H = L->H, I = L->I;
  const int k = L->k, E = L->E, S = L->S;
  if (H % 128 != 0 || I % 128 != 0) return -2;
  int bad = 0;
#pragma omp parallel
  {
    float* xf = (float*)malloc(sizeof(float) * (size_t)H);
    uint8_t* xc = (uint8_t*)malloc((size_t)H);
    uint8_t* xs = (uint8_t*)malloc((size_t)(H / 128));
    double* xq = (double*)malloc(sizeof(double) * (size_t)H);
    float* hbuf = (float*)malloc(sizeof(float) * (size_t)I);
    uint8_t* hc = (uint8_t*)malloc((size_t)I);
    uint8_t* hs = (uint8_t*)malloc((size_t)(I / 128));
    double* y = (double*)malloc(sizeof(double) * (size_t)H);
#pragma omp for schedule(dynamic, 1)
    for (int64_t i = 0; i < n_tok; ++i) {
      const int64_t t = tokens[i];
      for (int64_t h = 0; h < H; ++h) xf[h] = (float)bf16_to_double(x[t * H + h]);
      oracle_quantize_e4m3(1, H, xf, xc, xs, H / 128);
      for (int64_t h = 0; h < H; ++h) xq[h] = oracle_e4m3_value(xc[h]) * oracle_e8m0_value(xs[h / 128]);
      double* o = out + i * H;
      for (int64_t n = 0; n < H; ++n) o[n] = 0.0;
      for (int j = 0; j < k + S; ++j) {
        const int e = j < k ? idx[t * k + j] : E + (j - k);
        if (e < 0) continue;
        if (!wg[e] || !sg[e] || !wu[e] || !su[e] || !wd[e] || !sd[e]) {
#pragma omp atomic write
          bad = 1;
          continue;
        }
        swiglu_row_fp8(L, xq, wg[e], sg[e], wu[e], su[e], wd[e], sd[e], hbuf, hc, hs, y);
        const double gate = j < k ? w[t * k + j] : 1.0;
        for (int64_t n = 0; n < H; ++n) o[n] += gate * y[n];
      }
    }
    free(xf);
    free(xc);
    free(xs);
    free(xq);
    free(hbuf);
    free(hc);
    free(hs);
    free(y);
  }
  return bad ? -1 : 0;
}

/* ---- parameter arithmetic ---------------------------------------------------- */
/* One MoE layer: router E*H plus (E+S) experts of three H x I matrices. */
int64_t oracle_moe_layer_params(int64_t H, int64_t E, int64_t S, int64_t I) { return E * H + (E + S) * 3 * H * I; }

/* Parameters one token passes through in a MoE layer: the router, its k
 * routed experts and the S shared experts. */
int64_t oracle_moe_active_params(int64_t H, int64_t E, int64_t S, int64_t k, int64_t I) {
  return E * H + (k + S) * 3 * H * I;
}
