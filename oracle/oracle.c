/*
 * oracle.c -- plain, slow, scalar fp64 CPU oracle of one quantized
 * Mixture-of-Experts FFN step.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link,
 * load or call this file; only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark do.  It shares no code, header, table or
 * constant with the HIP library: every conversion, unpack and reduction here
 * is written out from the definitions.
 *
 * Sources (page titles and sections; the pages describe the step in words,
 * the shapes, distributions, GELU form and rounding points are the workload
 * definitions this oracle is written against):
 *  [devtrends] "Come eseguire un modello da 26 miliardi di parametri in due
 *      gigabyte di memoria su un Mac normale", section "Qual è il trucco
 *      principale dell'architettura": a router at every layer picks 8
 *      experts; 16-slot LFU expert cache; section "Prestazioni nel mondo
 *      reale": 128-token prefill chunks let one loaded expert serve a group
 *      of rows.
 *  [remio] "TurboFieldfare esegue Mac Gemma 4 26B in 2 GB, ma la velocità
 *      dell'SSD diventa il compromesso", section "Mac Gemma 4 26B entra nello
 *      spazio disponibile…": eight routed experts plus one shared expert;
 *      section "L'affermazione dei 2 GB trasforma la larghezza di banda
 *      dell'SSD nel nuovo vincolo": 4-bit MLX-affine weights, 8-bit router,
 *      the shared branch and the routed branch are combined, 30 layers,
 *      prefill chunks of up to 128 tokens.
 *  [iitog] "TurboFieldfare: движок с открытым кодом запускает Gemma 4 26B на
 *      Mac с 8 ГБ памяти", technical paragraph: MLX affine 4-bit, 8-bit
 *      router, kernels for quantized GEMV, MoE routing, normalisation.
 *  [elsolitario] TurboFieldfare article, section "Detalles técnicos y
 *      rendimiento": MLX affine 4-bit with group size 64; router at 8 bits.
 *
 * Readings of what the pages leave open (each one is listed with its reason
 * in the design notes): codes packed LSB-first along the input axis; one fp16
 * scale and one fp16 bias per row and per 64 inputs, w = s*q + bias; the FFN
 * is down(gelu_tanh(gate h) * (up h)); routing keeps the k largest logits
 * (ties to the lower expert index) and renormalises their softmax; the shared
 * expert enters the combine unweighted; one bf16 round-to-nearest-even per
 * layer output, after the residual add.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_GROUP 64

/* ------------------------------------------------------------------ types */
typedef struct {
  const uint32_t* q; /* codes, [rows][cols*bits/32] */
  const uint16_t* s; /* fp16 bits, [rows][cols/64] */
  const uint16_t* b; /* fp16 bits, [rows][cols/64] */
} orc_qmat;

typedef struct {
  int32_t H, E, K, I, Is;
  orc_qmat router;        /* 8-bit, [E x H] */
  const orc_qmat* gate;   /* E entries, 4-bit [I x H] */
  const orc_qmat* up;     /* E entries, 4-bit [I x H] */
  const orc_qmat* down;   /* E entries, 4-bit [H x I] */
  orc_qmat sh_gate;       /* 4-bit [Is x H] */
  orc_qmat sh_up;         /* 4-bit [Is x H] */
  orc_qmat sh_down;       /* 4-bit [H x Is] */
  const uint16_t* gamma;  /* bf16 [H]: RMSNorm weight, NULL = no norm */
  const float* logit_bias;/* [E] added to router logits, NULL = none */
} orc_layer;

/* ------------------------------------------------------- number formats */
/* IEEE 754 binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
double orc_half_to_double(uint16_t h) {
  int sign = (h >> 15) & 1;
  int e = (h >> 10) & 0x1f;
  int f = h & 0x3ff;
  double v;
  if (e == 0)
    v = ldexp((double)f, -24);
  else if (e == 31)
    v = f ? NAN : INFINITY;
  else
    v = ldexp((double)(1024 + f), e - 25);
  return sign ? -v : v;
}

/* bfloat16: 1 sign, 8 exponent (bias 127), 7 fraction bits. */
double orc_bf16_to_double(uint16_t h) {
  int sign = (h >> 15) & 1;
  int e = (h >> 7) & 0xff;
  int f = h & 0x7f;
  double v;
  if (e == 0)
    v = ldexp((double)f, -133);
  else if (e == 255)
    v = f ? NAN : INFINITY;
  else
    v = ldexp((double)(128 + f), e - 134);
  return sign ? -v : v;
}

/* double -> bf16, round to nearest, ties to even, in one step (no detour
 * through float).  The bf16 quantum for |v| in [2^E, 2^(E+1)) is 2^(E-7);
 * below 2^-126 it is the subnormal quantum 2^-133. */
uint16_t orc_double_to_bf16(double v) {
  if (isnan(v)) return 0x7fc0;
  uint16_t sign = signbit(v) ? 0x8000 : 0;
  double a = fabs(v);
  if (a == 0.0) return sign;
  if (isinf(a)) return sign | 0x7f80;
  int e2;
  frexp(a, &e2); /* a = m * 2^e2, m in [0.5,1) -> a in [2^(e2-1), 2^e2) */
  int E = e2 - 1;
  if (E < -126) E = -126;
  double quantum = ldexp(1.0, E - 7);
  double n = nearbyint(a / quantum); /* default mode: ties to even */
  double r = n * quantum;
  if (r >= ldexp(1.0, 128)) return sign | 0x7f80;
  /* encode r, which is exactly representable in bf16 */
  if (r < ldexp(1.0, -126)) {
    return sign | (uint16_t)(r / ldexp(1.0, -133));
  }
  int re2;
  double m = frexp(r, &re2); /* r = m*2^re2, m in [0.5,1) */
  int be = re2 - 1 + 127;    /* biased exponent */
  int frac = (int)(m * 256.0) - 128; /* 8 significant bits -> 7 fraction */
  return sign | (uint16_t)(be << 7) | (uint16_t)frac;
}

/* ------------------------------------------------------------ codes */
/* Code j of a word occupies bits [j*b, (j+1)*b), least significant first;
 * column c of row r lives in word c/(32/b) of that row. */
static int orc_code(const uint32_t* q, int64_t row, int64_t cols, int bits,
                    int64_t c) {
  int per = 32 / bits;
  int64_t words_per_row = cols / per;
  uint32_t w = q[row * words_per_row + c / per];
  int j = (int)(c % per);
  return (int)((w >> (j * bits)) & ((1u << bits) - 1u));
}

void orc_unpack(const uint32_t* q, int64_t rows, int64_t cols, int bits,
                uint8_t* codes) {
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t c = 0; c < cols; ++c)
      codes[r * cols + c] = (uint8_t)orc_code(q, r, cols, bits, c);
}

/* W[r][c] = s[r][c/64] * q[r][c] + bias[r][c/64].  Exact in double: s and
 * bias are fp16, s*q has at most 19 significant bits and the sum of two
 * fp16-derived values that are multiples of 2^-24 below 2^16 fits 53 bits. */
static double orc_weight(const orc_qmat* m, int64_t rows, int64_t cols,
                         int bits, int64_t r, int64_t c) {
  (void)rows;
  int64_t groups = cols / ORC_GROUP;
  double s = orc_half_to_double(m->s[r * groups + c / ORC_GROUP]);
  double b = orc_half_to_double(m->b[r * groups + c / ORC_GROUP]);
  return s * (double)orc_code(m->q, r, cols, bits, c) + b;
}

void orc_dequant(const uint32_t* q, const uint16_t* s, const uint16_t* b,
                 int64_t rows, int64_t cols, int bits, double* W) {
  orc_qmat m = {q, s, b};
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t c = 0; c < cols; ++c)
      W[r * cols + c] = orc_weight(&m, rows, cols, bits, r, c);
}

/* y[r] = sum_c W[r][c] * x[c], accumulated in double in column order. */
static void orc_qgemv_m(const orc_qmat* m, int64_t rows, int64_t cols,
                        int bits, const double* x, double* y) {
  for (int64_t r = 0; r < rows; ++r) {
    double acc = 0.0;
    for (int64_t c = 0; c < cols; ++c)
      acc += orc_weight(m, rows, cols, bits, r, c) * x[c];
    y[r] = acc;
  }
}

void orc_qgemv(const uint32_t* q, const uint16_t* s, const uint16_t* b,
               int64_t rows, int64_t cols, int bits, const double* x,
               double* y) {
  orc_qmat m = {q, s, b};
  orc_qgemv_m(&m, rows, cols, bits, x, y);
}

/* -------------------------------------------------------------- RMSNorm */
/* h_i = bf16( x_i * gamma_i / sqrt(mean(x^2) + eps) ). */
void orc_rmsnorm(const uint16_t* x, const uint16_t* gamma, int64_t H,
                 double eps, uint16_t* h) {
  double ss = 0.0;
  for (int64_t i = 0; i < H; ++i) {
    double v = orc_bf16_to_double(x[i]);
    ss += v * v;
  }
  double inv = 1.0 / sqrt(ss / (double)H + eps);
  for (int64_t i = 0; i < H; ++i)
    h[i] = orc_double_to_bf16(orc_bf16_to_double(x[i]) * inv *
                              orc_bf16_to_double(gamma[i]));
}

/* --------------------------------------------------------------- GELU */
/* tanh form of GELU: 0.5 z (1 + tanh(sqrt(2/pi) (z + 0.044715 z^3))). */
double orc_gelu_tanh(double z) {
  const double k = sqrt(2.0 / M_PI);
  return 0.5 * z * (1.0 + tanh(k * (z + 0.044715 * z * z * z)));
}

/* ------------------------------------------------------ routing top-k */
/* Keep the k largest logits, ordered by descending logit and, among equal
 * logits, ascending expert index; their weights are the softmax over the
 * kept logits (the same numbers as a softmax over all E followed by
 * renormalisation over the kept k). */
void orc_topk_softmax(const double* logits, int32_t E, int32_t k,
                      int32_t* idx, double* w) {
  char* taken = (char*)calloc((size_t)E, 1);
  for (int32_t j = 0; j < k; ++j) {
    int32_t best = -1;
    for (int32_t e = 0; e < E; ++e) {
      if (taken[e]) continue;
      if (best < 0 || logits[e] > logits[best]) best = e;
    }
    taken[best] = 1;
    idx[j] = best;
  }
  free(taken);
  double top = logits[idx[0]], sum = 0.0;
  for (int32_t j = 0; j < k; ++j) {
    w[j] = exp(logits[idx[j]] - top);
    sum += w[j];
  }
  for (int32_t j = 0; j < k; ++j) w[j] /= sum;
}

static void orc_bf16_vec(const uint16_t* v, int64_t n, double* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_bf16_to_double(v[i]);
}

/* logits_e = sum_c Wr[e][c] h_c (+ bias_e). */
void orc_router_logits(const orc_layer* L, const uint16_t* h, double* logits) {
  double* hd = (double*)malloc(sizeof(double) * L->H);
  orc_bf16_vec(h, L->H, hd);
  orc_qgemv_m(&L->router, L->E, L->H, 8, hd, logits);
  if (L->logit_bias)
    for (int32_t e = 0; e < L->E; ++e) logits[e] += (double)L->logit_bias[e];
  free(hd);
}

/* ---------------------------------------------------------------- FFN */
/* y = W_down (gelu(W_gate h) * (W_up h)), all in double. */
static void orc_ffn(const orc_qmat* g, const orc_qmat* u, const orc_qmat* d,
                    int32_t H, int32_t I, const double* h, double* y) {
  double* gv = (double*)malloc(sizeof(double) * I);
  double* uv = (double*)malloc(sizeof(double) * I);
  orc_qgemv_m(g, I, H, 4, h, gv);
  orc_qgemv_m(u, I, H, 4, h, uv);
  for (int32_t i = 0; i < I; ++i) gv[i] = orc_gelu_tanh(gv[i]) * uv[i];
  orc_qgemv_m(d, H, I, 4, gv, y);
  free(gv);
  free(uv);
}

void orc_expert_ffn(const orc_qmat* g, const orc_qmat* u, const orc_qmat* d,
                    int32_t H, int32_t I, const uint16_t* h, double* y) {
  double* hd = (double*)malloc(sizeof(double) * H);
  orc_bf16_vec(h, H, hd);
  orc_ffn(g, u, d, H, I, hd, y);
  free(hd);
}

/* ------------------------------------------------------ one MoE layer */
/* One token through one layer.
 *   x        bf16 [H]: layer input
 *   residual nonzero: out = bf16(x + y), else out = bf16(y)
 *   force_idx/force_w: if non-NULL, use this routing instead of the router
 * Outputs (each may be NULL): out bf16 [H], y double [H] (pre-rounding),
 * h bf16 [H] (expert input), logits [E], idx [K], w [K].
 * Returns 0. */
int orc_layer_forward(const orc_layer* L, const uint16_t* x, int residual,
                      const int32_t* force_idx, const double* force_w,
                      uint16_t* out, double* y_out, uint16_t* h_out,
                      double* logits_out, int32_t* idx_out, double* w_out) {
  const int32_t H = L->H, E = L->E, K = L->K;
  uint16_t* h = (uint16_t*)malloc(sizeof(uint16_t) * H);
  double* hd = (double*)malloc(sizeof(double) * H);
  double* y = (double*)malloc(sizeof(double) * H);
  double* ye = (double*)malloc(sizeof(double) * H);
  double* logits = (double*)malloc(sizeof(double) * E);
  int32_t* idx = (int32_t*)malloc(sizeof(int32_t) * K);
  double* w = (double*)malloc(sizeof(double) * K);

  if (L->gamma)
    orc_rmsnorm(x, L->gamma, H, 1e-6, h);
  else
    memcpy(h, x, sizeof(uint16_t) * H);
  orc_bf16_vec(h, H, hd);

  orc_router_logits(L, h, logits);
  if (force_idx) {
    memcpy(idx, force_idx, sizeof(int32_t) * K);
    memcpy(w, force_w, sizeof(double) * K);
  } else {
    orc_topk_softmax(logits, E, K, idx, w);
  }

  /* shared expert, then the routed experts in rank order */
  orc_ffn(&L->sh_gate, &L->sh_up, &L->sh_down, H, L->Is, hd, y);
  for (int32_t j = 0; j < K; ++j) {
    int32_t e = idx[j];
    orc_ffn(&L->gate[e], &L->up[e], &L->down[e], H, L->I, hd, ye);
    for (int32_t i = 0; i < H; ++i) y[i] += w[j] * ye[i];
  }
  if (residual)
    for (int32_t i = 0; i < H; ++i) y[i] += orc_bf16_to_double(x[i]);

  if (out)
    for (int32_t i = 0; i < H; ++i) out[i] = orc_double_to_bf16(y[i]);
  if (y_out) memcpy(y_out, y, sizeof(double) * H);
  if (h_out) memcpy(h_out, h, sizeof(uint16_t) * H);
  if (logits_out) memcpy(logits_out, logits, sizeof(double) * E);
  if (idx_out) memcpy(idx_out, idx, sizeof(int32_t) * K);
  if (w_out) memcpy(w_out, w, sizeof(double) * K);
  free(h); free(hd); free(y); free(ye); free(logits); free(idx); free(w);
  return 0;
}

/* ---------------------------------------------- prefill expert dispatch */
/* Group the T*K (token, rank) pairs of a chunk by expert, stably: by
 * expert, then token, then rank.  counts[E], offsets[E+1] (exclusive
 * prefix of counts), perm[T*K] holds flat pair indices t*K + j. */
void orc_dispatch(const int32_t* idx, int32_t T, int32_t K, int32_t E,
                  int32_t* counts, int32_t* offsets, int32_t* perm) {
  for (int32_t e = 0; e < E; ++e) counts[e] = 0;
  for (int32_t p = 0; p < T * K; ++p) counts[idx[p]]++;
  offsets[0] = 0;
  for (int32_t e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
  int32_t n = 0;
  for (int32_t e = 0; e < E; ++e)
    for (int32_t p = 0; p < T * K; ++p)
      if (idx[p] == e) perm[n++] = p;
}

/* -------------------------------------------------------- LFU replay */
/* Per-layer expert cache with `slots` device slots and least-frequently-used
 * replacement ([devtrends] "Qual è il trucco principale dell'architettura";
 * [remio] "Mac Gemma 4 26B entra nello spazio disponibile…").
 * Use counts are kept for every expert and survive eviction.  For each step,
 * with the needed experts `need[step][0..K)` in rank order:
 *   1. count[e] += 1 and last[e] = step for every needed e;
 *   2. a needed expert already resident is a hit;
 *   3. each miss, in rank order, takes the lowest-numbered empty slot, else
 *      evicts the resident expert not needed this step with the smallest
 *      (count, last use, id).
 * Outputs per (step, rank): hit[] 1/0, slot[] the slot that holds the
 * expert after the step, victim[] the evicted expert or -1.
 * Returns the number of hits, or -1 when no victim can be found. */
int64_t orc_lfu_replay(int32_t E, int32_t slots, int32_t K, int32_t steps,
                       const int32_t* need, int32_t* hit, int32_t* slot,
                       int32_t* victim) {
  int64_t* count = (int64_t*)calloc((size_t)E, sizeof(int64_t));
  int64_t* last = (int64_t*)malloc(sizeof(int64_t) * E);
  int32_t* holder = (int32_t*)malloc(sizeof(int32_t) * slots); /* expert or -1 */
  int32_t* where = (int32_t*)malloc(sizeof(int32_t) * E);      /* slot or -1 */
  char* needed = (char*)calloc((size_t)E, 1);
  int64_t hits = 0;
  for (int32_t e = 0; e < E; ++e) { last[e] = -1; where[e] = -1; }
  for (int32_t s = 0; s < slots; ++s) holder[s] = -1;

  for (int32_t t = 0; t < steps; ++t) {
    const int32_t* n = need + (int64_t)t * K;
    for (int32_t j = 0; j < K; ++j) {
      count[n[j]] += 1;
      last[n[j]] = t;
      needed[n[j]] = 1;
    }
    for (int32_t j = 0; j < K; ++j) {
      int32_t e = n[j];
      int64_t o = (int64_t)t * K + j;
      victim[o] = -1;
      if (where[e] >= 0) {
        hit[o] = 1;
        slot[o] = where[e];
        hits++;
        continue;
      }
      hit[o] = 0;
      int32_t s_free = -1;
      for (int32_t s = 0; s < slots; ++s)
        if (holder[s] < 0) { s_free = s; break; }
      if (s_free < 0) {
        int32_t best = -1;
        for (int32_t s = 0; s < slots; ++s) {
          int32_t c = holder[s];
          if (needed[c]) continue;
          if (best < 0) { best = s; continue; }
          int32_t b = holder[best];
          if (count[c] < count[b] ||
              (count[c] == count[b] &&
               (last[c] < last[b] || (last[c] == last[b] && c < b))))
            best = s;
        }
        if (best < 0) {
          hits = -1;
          goto done;
        }
        victim[o] = holder[best];
        where[holder[best]] = -1;
        s_free = best;
      }
      holder[s_free] = e;
      where[e] = s_free;
      slot[o] = s_free;
    }
    for (int32_t j = 0; j < K; ++j) needed[n[j]] = 0;
  }
done:
  free(count); free(last); free(holder); free(where); free(needed);
  return hits;
}

/* ---------------------------------------------------------- sampling */
/* The token choice after the last layer.  [elsolitario] TurboFieldfare
 * article, section "Cómo empezar": temperature 0.2, top-K 64 and top-P 0.95
 * by default, temperature 0 for deterministic output; [pikobit] "Un modello
 * da 26 miliardi di parametri in 2 GB di RAM, su un Mac da 8 GB": default
 * temperature 0.2; [iitog] technical paragraph: sampling is one of the
 * engine's kernels.
 * Readings (the pages give the three parameters only): keep the top_k
 * largest logits (equal logits: lower token id first), in descending order;
 * temperature 0 chooses the first; otherwise p_j = exp((l_j - l_0) / T)
 * over the kept ranks, the top-P cut keeps rank j while the mass of the
 * ranks before it is below top_p of their total, and the draw u in [0, 1)
 * picks the first kept rank whose cumulative mass exceeds u times the kept
 * mass.  Returns the token id.  ranked (top_k ids) and cum (top_k inclusive
 * cumulative masses over the total) may be NULL; *kept (may be NULL) gets
 * the number of kept ranks (1 with temperature 0). */
int32_t orc_sample(const float* logits, int32_t V, double temperature, int32_t top_k,
                   double top_p, double u, int32_t* ranked, double* cum, int32_t* kept) {
  if (top_k < 1 || top_k > V) return -1;
  int32_t* id = (int32_t*)calloc((size_t)top_k, sizeof(int32_t));
  char* taken = (char*)calloc((size_t)V, 1);
  for (int32_t j = 0; j < top_k; ++j) {
    int32_t best = -1;
    for (int32_t t = 0; t < V; ++t) {
      if (taken[t]) continue;
      if (best < 0 || logits[t] > logits[best]) best = t;
    }
    taken[best] = 1;
    id[j] = best;
  }
  free(taken);
  if (ranked)
    for (int32_t j = 0; j < top_k; ++j) ranked[j] = id[j];
  int32_t token;
  if (temperature == 0.0) {
    token = id[0];
    if (kept) *kept = 1;
    if (cum)
      for (int32_t j = 0; j < top_k; ++j) cum[j] = 1.0;  /* all mass on rank 0 */
  } else {
    double* p = (double*)malloc(sizeof(double) * (size_t)top_k);
    double* c = (double*)malloc(sizeof(double) * (size_t)top_k);
    const double l0 = (double)logits[id[0]];
    double total = 0.0;
    for (int32_t j = 0; j < top_k; ++j) {
      p[j] = exp(((double)logits[id[j]] - l0) / temperature);
      total += p[j];
      c[j] = total;
    }
    int32_t m = 0;
    while (m < top_k && (m == 0 ? 0.0 : c[m - 1]) < top_p * total) ++m;
    const double target = u * c[m - 1];
    int32_t r = 0;
    while (r < m - 1 && !(c[r] > target)) ++r;
    token = id[r];
    if (kept) *kept = m;
    if (cum)
      for (int32_t j = 0; j < top_k; ++j) cum[j] = c[j] / total;
    free(p);
    free(c);
  }
  free(id);
  return token;
}

/* ------------------------------------------- decode attention, FP16 KV */
/* double -> IEEE binary16, round to nearest, ties to even, in one step.  The
 * fp16 quantum for |v| in [2^E, 2^(E+1)) is 2^(E-10); below 2^-14 it is the
 * subnormal quantum 2^-24.  Results of 2^16 or more are infinite. */
uint16_t orc_double_to_half(double v) {
  if (isnan(v)) return 0x7e00;
  uint16_t sign = signbit(v) ? 0x8000 : 0;
  double a = fabs(v);
  if (a == 0.0) return sign;
  if (isinf(a)) return sign | 0x7c00;
  int e2;
  frexp(a, &e2);
  int E = e2 - 1;
  if (E < -14) E = -14;
  double quantum = ldexp(1.0, E - 10);
  double r = nearbyint(a / quantum) * quantum;
  if (r >= 65536.0) return sign | 0x7c00;
  if (r < ldexp(1.0, -14)) return sign | (uint16_t)(r / ldexp(1.0, -24));
  int re2;
  double m = frexp(r, &re2);
  int be = re2 - 1 + 15;
  int frac = (int)(m * 2048.0) - 1024; /* 11 significant bits -> 10 fraction */
  return sign | (uint16_t)(be << 10) | (uint16_t)frac;
}

/* Rotary position embedding of one head vector x[D] for the token at time
 * pos ([iitog] technical paragraph and [devtrends] section "Senza
 * dipendenze da llama.cpp e MLX": RoPE is one of the engine's kernels).
 * Reading (the pages name the operation only): element i and element
 * i + D/2 form a plane, i < D/2, rotated by the angle pos * base^(-2i/D)
 * in the positive sense:
 *   out[i]       = x[i] cos(a) - x[i + D/2] sin(a)
 *   out[i + D/2] = x[i + D/2] cos(a) + x[i] sin(a). */
void orc_rope(const double* x, int32_t D, int64_t pos, double base, double* out) {
  const int32_t h = D / 2;
  for (int32_t i = 0; i < h; ++i) {
    const double a = (double)pos * pow(base, -2.0 * (double)i / (double)D);
    const double c = cos(a), s = sin(a);
    const double x0 = x[i], x1 = x[i + h];
    out[i] = x0 * c - x1 * s;
    out[i + h] = x1 * c + x0 * s;
  }
}

/* One decode step of attention for the token at time pos over an FP16 key
 * and value history ([iitog] technical paragraph: the KV cache is FP16, 25
 * layers attend over a sliding window kept in a bounded circular store and
 * 5 layers over the whole context kept in a linear one; [remio] section
 * "Mac Gemma 4 26B entra nello spazio disponibile…" and [pikobit]: a
 * 4,096-token cache).
 *   q [Hq][D], k, v [Hkv][D]: this token's projections (fp32);
 *   khist, vhist [time][Hkv][D] fp16 bits: entries of times before pos are
 *     read; this step writes time pos: fp16 of RoPE(k) and fp16 of v;
 *   out [Hq][D]: the attention output.
 * Readings: head h attends with key/value head h / (Hq / Hkv); the times
 * attended are max(0, pos - window + 1) .. pos, or 0 .. pos with window 0;
 * the query is RoPE(q) unrounded; score(t) = scale * <RoPE(q_h), K[t]>;
 * out_h = sum_t softmax(score)_t V[t].  Returns 0, or -1 on bad shapes. */
int orc_attn_step(int32_t Hq, int32_t Hkv, int32_t D, int64_t window, double scale,
                  double base, int64_t pos, const float* q, const float* k, const float* v,
                  uint16_t* khist, uint16_t* vhist, double* out) {
  if (Hq < 1 || Hkv < 1 || Hq % Hkv || D < 2 || D % 2 || pos < 0 || window < 0) return -1;
  const int32_t G = Hq / Hkv;
  double* x = (double*)malloc(sizeof(double) * (size_t)D);
  double* r = (double*)malloc(sizeof(double) * (size_t)D);
  /* this token's key and value into the history */
  for (int32_t g = 0; g < Hkv; ++g) {
    for (int32_t d = 0; d < D; ++d) x[d] = (double)k[(int64_t)g * D + d];
    orc_rope(x, D, pos, base, r);
    uint16_t* kd = khist + (pos * Hkv + g) * (int64_t)D;
    uint16_t* vd = vhist + (pos * Hkv + g) * (int64_t)D;
    for (int32_t d = 0; d < D; ++d) {
      kd[d] = orc_double_to_half(r[d]);
      vd[d] = orc_double_to_half((double)v[(int64_t)g * D + d]);
    }
  }
  const int64_t t0 = (window > 0 && pos - window + 1 > 0) ? pos - window + 1 : 0;
  const int64_t n = pos - t0 + 1;
  double* sc = (double*)malloc(sizeof(double) * (size_t)n);
  for (int32_t hq = 0; hq < Hq; ++hq) {
    const int32_t g = hq / G;
    for (int32_t d = 0; d < D; ++d) x[d] = (double)q[(int64_t)hq * D + d];
    orc_rope(x, D, pos, base, r);
    double m = -INFINITY;
    for (int64_t j = 0; j < n; ++j) {
      const uint16_t* kt = khist + ((t0 + j) * Hkv + g) * (int64_t)D;
      double s = 0.0;
      for (int32_t d = 0; d < D; ++d) s += r[d] * orc_half_to_double(kt[d]);
      sc[j] = scale * s;
      if (sc[j] > m) m = sc[j];
    }
    double z = 0.0;
    for (int64_t j = 0; j < n; ++j) {
      sc[j] = exp(sc[j] - m);
      z += sc[j];
    }
    double* o = out + (int64_t)hq * D;
    for (int32_t d = 0; d < D; ++d) o[d] = 0.0;
    for (int64_t j = 0; j < n; ++j) {
      const uint16_t* vt = vhist + ((t0 + j) * Hkv + g) * (int64_t)D;
      for (int32_t d = 0; d < D; ++d) o[d] += sc[j] / z * orc_half_to_double(vt[d]);
    }
  }
  free(sc);
  free(x);
  free(r);
  return 0;
}
