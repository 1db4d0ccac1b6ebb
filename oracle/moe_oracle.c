/*
 * fp64 CPU oracle of the routed MoE layer (sqrt-softplus router, top-k or hash
 * routing, one shared expert, SwiGLU experts on MXFP4 weights).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or constant with the HIP implementation.
 *
 * Every result is computed in double precision from the plain definition, each
 * sum taken in ascending index order by one thread, so the output does not
 * depend on the thread count.  Sources of each step:
 * - MXFP4 = E2M1 elements with one E8M0 power-of-two scale per 32 elements:
 *   aimarketly "Deepseek-V4-Flash-Dspark-FST" model card, Preprocessing
 *   (17-byte blocks: one e8m0 scale + 16 bytes of FP4) and TensorSharp
 *   "DeepSeek V4 Flash", Getting a drafter (per-32 E8M0 scales).  Element
 *   values follow the OCP Microscaling specification (the pages do not print
 *   them).
 * - router score sqrt(softplus(x W^T)), top-6 of 256 plus one shared expert,
 *   hash routing: TensorSharp "How TensorSharp runs it" (sqrt-softplus MoE
 *   routing with hash layers) and the model card "Model Architecture and
 *   Objective" (top-k = 6, hash-routed layers, route_scale, swiglu_limit).
 * - gates = selected scores normalised to sum 1.
 * - expert FFN: down(silu(gate x) * up x) with the swiglu limit clamp
 *   (TensorSharp Ops.SiLUMulClamp; model card swiglu_limit = 10), combined as a
 *   weighted sum of the routed experts plus the shared expert (TensorSharp
 *   "Fitting the model": weighted-sum epilogue; pypto "MoE and output stages":
 *   shared and routed FFN paths).
 * - the shared expert optionally in bf16 instead of MXFP4 (model card,
 *   Preprocessing and "Model Architecture and Objective": shared tensors in
 *   Q8_0/BF16, expert blocks in MXFP4).
 * - the routed experts optionally as Q2_K blocks (TensorSharp "Getting a
 *   drafter": --expert-type q2_k for the drafter's routed experts; the
 *   layout is GGUF's Q2_K, see orc_decode_q2k_row).  The pages do not define
 *   the format, so its byte-level reading is parity unpinned against a GGUF
 *   implementation: the pins check the decode against the format's published
 *   description (positions, scales, mins, fp16 factors), not against a file.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ decoding */

/* E2M1 (OCP): bit 3 sign, bits 2..1 exponent E (bias 1), bit 0 mantissa M.
 * E == 0: subnormal 0.5*M; otherwise 2^(E-1) * (1 + M/2). */
double orc_e2m1(int code) {
  int sign = (code >> 3) & 1, E = (code >> 1) & 3, M = code & 1;
  double mag = (E == 0) ? 0.5 * M : ldexp(1.0 + 0.5 * M, E - 1);
  return sign ? -mag : mag;
}

/* E8M0 (OCP): 2^(e - 127); 0xFF encodes NaN. */
double orc_e8m0(int e) {
  if (e == 0xFF) return NAN;
  return ldexp(1.0, e - 127);
}

/* bf16 bit pattern -> value (the upper half of an fp32). */
double orc_bf16(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* fp32 -> bf16 bit pattern, round to nearest even (NaN stays a quiet NaN). */
uint16_t orc_f32_to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

/* RMSNorm in front of the layer (the FFN input norm, ffn_norm in the ds4
 * issue's loader spec; RMSNorm kernels in the FaStar README, Features; "hc_pre
 * -> rmsnorm" in the pypto DSpark point pipeline).  The pages fix neither the
 * precision nor eps; the layer's activations are bf16, so the normalised row is
 * computed in fp32, the precision of the kernel that takes the same rounding
 * decision, and rounded once to bf16:
 *   ms = (sum_i x_i^2) / d  (fp32, i ascending),  r = 1 / sqrt(ms + eps),
 *   xn_i = bf16((x_i * r) * g_i). */
void orc_rmsnorm_bf16(const uint16_t* x, int N, int d, const uint16_t* g, float eps, uint16_t* xn) {
  for (long r = 0; r < N; ++r) {
    const uint16_t* xr = x + (size_t)r * d;
    float ss = 0.0f;
    for (int i = 0; i < d; ++i) {
      const float v = (float)orc_bf16(xr[i]);
      ss = ss + v * v;
    }
    const float inv = 1.0f / sqrtf(ss / (float)d + eps);
    for (int i = 0; i < d; ++i) {
      const float v = (float)orc_bf16(xr[i]);
      const float t = v * inv;
      xn[(size_t)r * d + i] = orc_f32_to_bf16(t * (float)orc_bf16(g[i]));
    }
  }
}

/* One row of an MXFP4 matrix: K values, element t in byte t/2 (low nibble when
 * t is even), scale byte t/32. */
void orc_decode_mxfp4_row(const uint8_t* q, const uint8_t* s, int K, double* out) {
  for (int b = 0; b < K / 32; ++b) {
    const double scale = orc_e8m0(s[b]);
    for (int t = 32 * b; t < 32 * b + 32; ++t) {
      int byte = q[t / 2];
      int code = (t & 1) ? (byte >> 4) : (byte & 15);
      out[t] = orc_e2m1(code) * scale;
    }
  }
}

/* IEEE half-precision bits -> value (sign, 5 exponent bits with bias 15, 10
 * fraction bits; exponent 0 = subnormal f * 2^-24; exponent 31 = inf / NaN). */
double orc_half(uint16_t h) {
  const int sign = h >> 15, ex = (h >> 10) & 31, f = h & 1023;
  double mag;
  if (ex == 0) mag = ldexp((double)f, -24);
  else if (ex == 31) mag = f ? NAN : INFINITY;
  else mag = ldexp(1.0 + f / 1024.0, ex - 15);
  return sign ? -mag : mag;
}

/* One row of a Q2_K matrix (the GGUF Q2_K format; the pages name the format,
 * TensorSharp "Getting a drafter", --expert-type q2_k, without defining it):
 * K values in K/256 super-blocks of 84 bytes.  A super-block holds 16
 * sub-blocks of 16 consecutive values; byte n (0..15) carries sub-block n's
 * 4-bit scale (low nibble) and 4-bit min (high nibble); bytes 16..79 carry the
 * 2-bit quants, four to a byte: the block's two halves of 128 values use 32
 * bytes each, and inside a half, byte i (0..31) holds in bits 2j..2j+1 the
 * quant of value 32j + i; bytes 80..81 and 82..83 are the half-precision
 * factors d and dmin.  A value decodes to d * scale * q - dmin * min. */
void orc_decode_q2k_row(const uint8_t* row, int K, double* out) {
  for (int b = 0; b < K / 256; ++b) {
    const uint8_t* blk = row + (size_t)b * 84;
    const double d = orc_half((uint16_t)(blk[80] | (blk[81] << 8)));
    const double dmin = orc_half((uint16_t)(blk[82] | (blk[83] << 8)));
    double* o = out + 256 * b;
    for (int half = 0; half < 2; ++half)
      for (int j = 0; j < 4; ++j)
        for (int i = 0; i < 32; ++i) {
          const int t = 128 * half + 32 * j + i;
          const int q = (blk[16 + 32 * half + i] >> (2 * j)) & 3;
          const int sb = blk[t / 16];
          o[t] = d * (double)(sb & 15) * q - dmin * (double)(sb >> 4);
        }
  }
}

/* -------------------------------------------------------------- thread helper */

typedef void (*item_fn)(void* ctx, long item);
typedef struct { item_fn fn; void* ctx; long n; int t, nt; } orc_job;

static void* orc_job_main(void* p) {
  orc_job* j = (orc_job*)p;
  for (long i = j->t; i < j->n; i += j->nt) j->fn(j->ctx, i);
  return NULL;
}

/* Runs fn(ctx, i) for i in [0, n); each item is done entirely by one thread. */
static void orc_parallel(item_fn fn, void* ctx, long n, int nthreads) {
  if (nthreads > 256) nthreads = 256;
  if (nthreads <= 1 || n < 2) {
    for (long i = 0; i < n; ++i) fn(ctx, i);
    return;
  }
  pthread_t th[256];
  orc_job jobs[256];
  int ok[256];
  for (int t = 0; t < nthreads; ++t) {
    jobs[t] = (orc_job){fn, ctx, n, t, nthreads};
    ok[t] = pthread_create(&th[t], NULL, orc_job_main, &jobs[t]) == 0;
    if (!ok[t]) orc_job_main(&jobs[t]);
  }
  for (int t = 0; t < nthreads; ++t)
    if (ok[t]) pthread_join(th[t], NULL);
}

/* -------------------------------------------------------------------- router */

typedef struct {
  const uint16_t* x; int d; const float* w; int E; const float* bias; double* z;
} logit_ctx;

static void logit_row(void* p, long r) {
  logit_ctx* c = (logit_ctx*)p;
  double* xr = (double*)malloc(sizeof(double) * (size_t)c->d);
  for (int i = 0; i < c->d; ++i) xr[i] = orc_bf16(c->x[(size_t)r * c->d + i]);
  for (int e = 0; e < c->E; ++e) {
    const float* we = c->w + (size_t)e * c->d;
    double acc = 0.0;
    for (int i = 0; i < c->d; ++i) acc += xr[i] * (double)we[i];
    if (c->bias) acc += (double)c->bias[e];
    c->z[(size_t)r * c->E + e] = acc;
  }
  free(xr);
}

/* z[r][e] = sum_i x[r][i] * W[e][i]  (+ bias[e] when bias != NULL). */
void orc_router_logits(const uint16_t* x, int N, int d, const float* w, int E, const float* bias, double* z,
                       int nthreads) {
  logit_ctx c = {x, d, w, E, bias, z};
  orc_parallel(logit_row, &c, N, nthreads);
}

/* softplus(z) = ln(1 + e^z), written as max(z,0) + ln(1 + e^-|z|) so that
 * neither branch overflows. */
double orc_softplus(double z) { return fmax(z, 0.0) + log1p(exp(-fabs(z))); }

/* Router score: sqrt(softplus(z)). */
double orc_score(double z) { return sqrt(orc_softplus(z)); }

/* Indices of the k largest s[0..E) (a tie goes to the lower index), written in
 * ascending index order.  Returns the score gap between the k-th and the
 * (k+1)-th largest (+inf when k == E). */
double orc_topk(const double* s, int E, int k, int* idx) {
  char taken[1024];
  memset(taken, 0, sizeof(taken));
  double kth = 0.0;
  for (int j = 0; j < k; ++j) {
    int best = -1;
    for (int e = 0; e < E; ++e)
      if (!taken[e] && (best < 0 || s[e] > s[best])) best = e;
    taken[best] = 1;
    idx[j] = best;
    kth = s[best];
  }
  double next = -INFINITY;
  for (int e = 0; e < E; ++e)
    if (!taken[e] && s[e] > next) next = s[e];
  /* ascending expert id */
  for (int a = 1; a < k; ++a)
    for (int b = a; b > 0 && idx[b - 1] > idx[b]; --b) {
      int t = idx[b];
      idx[b] = idx[b - 1];
      idx[b - 1] = t;
    }
  return (k < E) ? kth - next : INFINITY;
}

/* Routing of N rows from logits z [N][E].
 * routing 0: the k highest scores, or with sel_bias (the selection-only bias
 * reading of the router bias, gate.bias in the ds4 loader spec) the k highest
 * s + sel_bias.  routing 1 (hash): the k experts listed in
 * tid2eid[token_ids[r]] (distinct, in range; returns -1 otherwise).
 * idx [N][k] ascending expert id; gates [N][k] = s at idx (never biased),
 * normalised to sum 1; margin [N] (may be NULL): gap between the k-th and the
 * (k+1)-th selection value (routing 0) or +inf (routing 1). */
int orc_route(const double* z, int N, int E, int k, int routing, const int32_t* token_ids,
              const int32_t* tid2eid, long vocab, const float* sel_bias, int32_t* idx, double* gates,
              double* margin) {
  double* s = (double*)malloc(sizeof(double) * (size_t)E);
  double* t = (double*)malloc(sizeof(double) * (size_t)E);
  int sel[1024];
  int rc = 0;
  for (int r = 0; r < N && rc == 0; ++r) {
    for (int e = 0; e < E; ++e) s[e] = orc_score(z[(size_t)r * E + e]);
    double m = INFINITY;
    if (routing == 0) {
      for (int e = 0; e < E; ++e) t[e] = sel_bias ? s[e] + (double)sel_bias[e] : s[e];
      m = orc_topk(t, E, k, sel);
    } else {
      long t = token_ids[r];
      if (t < 0 || t >= vocab) { rc = -1; break; }
      for (int j = 0; j < k; ++j) {
        sel[j] = tid2eid[t * k + j];
        if (sel[j] < 0 || sel[j] >= E) rc = -1;
        for (int i = 0; i < j; ++i)
          if (sel[i] == sel[j]) rc = -1;
      }
      for (int a = 1; a < k; ++a)
        for (int b = a; b > 0 && sel[b - 1] > sel[b]; --b) {
          int tt = sel[b];
          sel[b] = sel[b - 1];
          sel[b - 1] = tt;
        }
    }
    if (rc) break;
    double sum = 0.0;
    for (int j = 0; j < k; ++j) sum += s[sel[j]];
    for (int j = 0; j < k; ++j) {
      idx[(size_t)r * k + j] = sel[j];
      gates[(size_t)r * k + j] = s[sel[j]] / sum;
    }
    if (margin) margin[r] = m;
  }
  free(s);
  free(t);
  return rc;
}

/* Expert-major bookkeeping of the N*k (row, slot) pairs:
 * counts[e] = number of pairs routed to e; offsets = exclusive prefix sum
 * (E+1 entries); pairs of one expert are ordered by row; perm[p] = r*k + j for
 * the pair at position p; inv[r*k + j] = p. */
void orc_bookkeeping(const int32_t* idx, int N, int k, int E, int32_t* counts, int32_t* offsets, int32_t* perm,
                     int32_t* inv) {
  for (int e = 0; e < E; ++e) counts[e] = 0;
  for (long q = 0; q < (long)N * k; ++q) counts[idx[q]]++;
  offsets[0] = 0;
  for (int e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
  long p = 0;
  for (int e = 0; e < E; ++e)
    for (int r = 0; r < N; ++r)
      for (int j = 0; j < k; ++j)
        if (idx[(long)r * k + j] == e) {
          perm[p] = r * k + j;
          inv[r * k + j] = (int32_t)p;
          ++p;
        }
}

/* ------------------------------------------------------------------- experts */

typedef struct {
  const uint8_t* q; /* [rows][K/2] */
  const uint8_t* s; /* [rows][K/32] */
} orc_mat;

typedef struct {
  int d, I;
  int q2k;  /* routed experts in Q2_K blocks (gq/uq/dq), else MXFP4 */
  double limit;
  /* per expert e in [0, E]: gate/up [I][d], down [d][I]; E = shared */
  const uint8_t *gq, *gs, *uq, *us, *dq, *ds;       /* routed, [E][...] */
  const uint8_t *sgq, *sgs, *suq, *sus, *sdq, *sds; /* shared, MXFP4 */
  const uint16_t *sgw, *suw, *sdw;                  /* shared, bf16 (used when sgw != NULL) */
  int E;
  /* work list: pairs grouped by expert */
  const int* pair_row;   /* [n_pairs] index into xd */
  const int* exp_start;  /* [E+2] pairs of expert e are [exp_start[e], exp_start[e+1]) */
  const double* xd;      /* [n_rows_used][d] */
  double* h;             /* [n_pairs][I] */
  double* y;             /* [n_pairs][d] */
} ffn_ctx;

static orc_mat mat_of(const ffn_ctx* c, int e, int which) {
  size_t gsz_q = (size_t)c->I * (c->d / 2), gsz_s = (size_t)c->I * (c->d / 32);
  size_t dsz_q = (size_t)c->d * (c->I / 2), dsz_s = (size_t)c->d * (c->I / 32);
  orc_mat m;
  if (e == c->E) {
    if (which == 0) { m.q = c->sgq; m.s = c->sgs; }
    else if (which == 1) { m.q = c->suq; m.s = c->sus; }
    else { m.q = c->sdq; m.s = c->sds; }
  } else {
    if (which == 0) { m.q = c->gq + e * gsz_q; m.s = c->gs + e * gsz_s; }
    else if (which == 1) { m.q = c->uq + e * gsz_q; m.s = c->us + e * gsz_s; }
    else { m.q = c->dq + e * dsz_q; m.s = c->ds + e * dsz_s; }
  }
  return m;
}

/* Row `row` of matrix `which` (0 gate, 1 up: K = d; 2 down: K = I) of expert e
 * in fp64: the shared expert (e == E) from its bf16 weights when given, else
 * from MXFP4. */
static void weight_row(const ffn_ctx* c, int e, int which, int row, int K, double* out) {
  if (e < c->E && c->q2k) {
    const uint8_t* base = which == 0 ? c->gq : which == 1 ? c->uq : c->dq;
    const size_t rows = which == 2 ? (size_t)c->d : (size_t)c->I, row_bytes = (size_t)(K / 256) * 84;
    orc_decode_q2k_row(base + ((size_t)e * rows + row) * row_bytes, K, out);
    return;
  }
  if (e == c->E && c->sgw) {
    const uint16_t* w = which == 0 ? c->sgw : which == 1 ? c->suw : c->sdw;
    for (int i = 0; i < K; ++i) out[i] = orc_bf16(w[(size_t)row * K + i]);
    return;
  }
  orc_mat m = mat_of(c, e, which);
  orc_decode_mxfp4_row(m.q + (size_t)row * (K / 2), m.s + (size_t)row * (K / 32), K, out);
}

/* Item = (expert e, intermediate unit n): h[p][n] for every pair p of e. */
static void ffn_gateup_item(void* p, long item) {
  ffn_ctx* c = (ffn_ctx*)p;
  int e = (int)(item / c->I), n = (int)(item % c->I);
  int p0 = c->exp_start[e], p1 = c->exp_start[e + 1];
  if (p0 == p1) return; /* an expert with no rows reads no weights */
  double* wg = (double*)malloc(sizeof(double) * (size_t)c->d * 2);
  double* wu = wg + c->d;
  weight_row(c, e, 0, n, c->d, wg);
  weight_row(c, e, 1, n, c->d, wu);
  for (int pp = p0; pp < p1; ++pp) {
    const double* xr = c->xd + (size_t)c->pair_row[pp] * c->d;
    double a = 0.0, b = 0.0;
    for (int i = 0; i < c->d; ++i) a += wg[i] * xr[i];
    for (int i = 0; i < c->d; ++i) b += wu[i] * xr[i];
    if (c->limit > 0.0) {
      a = fmin(a, c->limit);
      b = fmin(fmax(b, -c->limit), c->limit);
    }
    c->h[(size_t)pp * c->I + n] = a / (1.0 + exp(-a)) * b;
  }
  free(wg);
}

/* Item = (expert e, output unit m): y[p][m] for every pair p of e. */
static void ffn_down_item(void* p, long item) {
  ffn_ctx* c = (ffn_ctx*)p;
  int e = (int)(item / c->d), m = (int)(item % c->d);
  int p0 = c->exp_start[e], p1 = c->exp_start[e + 1];
  if (p0 == p1) return;
  double* wd = (double*)malloc(sizeof(double) * (size_t)c->I);
  weight_row(c, e, 2, m, c->I, wd);
  for (int pp = p0; pp < p1; ++pp) {
    const double* hr = c->h + (size_t)pp * c->I;
    double acc = 0.0;
    for (int n = 0; n < c->I; ++n) acc += wd[n] * hr[n];
    c->y[(size_t)pp * c->d + m] = acc;
  }
  free(wd);
}

typedef struct {
  int N, d, E, k, I;
  int routing;          /* 0 = sqrt-softplus top-k, 1 = hash */
  double route_scale;   /* multiplies the routed sum only */
  double swiglu_limit;  /* <= 0 disables the clamp */
  float norm_eps;       /* RMSNorm eps (used when norm_w != NULL) */
  int bias_mode;        /* router_bias: 0 added to the logits; 1 added to the scores for the selection only */
  int expert_format;    /* routed experts: 0 MXFP4 (gate_q/gate_s ...), 1 Q2_K blocks (gate_q, up_q, down_q) */
} orc_cfg;

typedef struct {
  const uint16_t* x;        /* bf16 [N][d] */
  const float* router_w;    /* [E][d] */
  const float* router_bias; /* [E] or NULL */
  const int32_t* token_ids; /* [N] (hash) */
  const int32_t* tid2eid;   /* [vocab][k] (hash) */
  long vocab;
  /* routed experts, natural layout: gate/up q [E][I][d/2] s [E][I][d/32], down q [E][d][I/2] s [E][d][I/32];
   * with expert_format 1, gate_q/up_q [E][I][d/256 * 84] and down_q [E][d][I/256 * 84] Q2_K blocks */
  const uint8_t *gate_q, *gate_s, *up_q, *up_s, *down_q, *down_s;
  /* shared expert, same layout with one matrix; gate_q == NULL means no shared expert */
  const uint8_t *sh_gate_q, *sh_gate_s, *sh_up_q, *sh_up_s, *sh_down_q, *sh_down_s;
  const uint16_t* norm_w;   /* bf16 [d]: the layer runs on RMSNorm(x) (orc_rmsnorm_bf16); NULL: on x */
  const uint16_t* residual; /* bf16 [N][d] added to the output, or NULL */
  /* shared expert with bf16 weights (gate/up [I][d], down [d][I]) instead of
   * MXFP4, or NULL.  The model card ("Preprocessing"; "Model Architecture and
   * Objective") stores expert blocks in MXFP4 and shared tensors in Q8_0/BF16
   * without placing the shared expert; both readings are covered. */
  const uint16_t *sh_gate_w, *sh_up_w, *sh_down_w;
} orc_inputs;

/*
 * The whole layer: out[r] = residual[r] + MoE(x'[r]) with x' = RMSNorm(x) when
 * norm_w is given, else x; the residual term only when residual is given.
 * rows (may be NULL = all N rows, in order) lists the rows
 * whose outputs are computed; routing and bookkeeping always cover all N rows.
 * out: [n_out][d] fp64 for the listed rows.  z, idx, gates, margin, counts,
 * offsets, perm, inv: optional (NULL to skip) full-size outputs.
 * Returns 0, or -1 on an invalid hash table entry.
 */
int orc_forward(const orc_cfg* cfg, const orc_inputs* in, const int32_t* rows, int n_out, double* out,
                double* z_out, int32_t* idx_out, double* gates_out, double* margin_out, int32_t* counts,
                int32_t* offsets, int32_t* perm, int32_t* inv, int nthreads) {
  const int N = cfg->N, d = cfg->d, E = cfg->E, k = cfg->k, I = cfg->I;
  if (N == 0) return 0;
  uint16_t* xn = NULL;
  const uint16_t* x = in->x;
  if (in->norm_w) {
    xn = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)N * d);
    orc_rmsnorm_bf16(in->x, N, d, in->norm_w, cfg->norm_eps, xn);
    x = xn;
  }
  double* z = (double*)malloc(sizeof(double) * (size_t)N * E);
  int32_t* idx = (int32_t*)malloc(sizeof(int32_t) * (size_t)N * k);
  double* gates = (double*)malloc(sizeof(double) * (size_t)N * k);
  const int sel_only = cfg->bias_mode == 1;
  orc_router_logits(x, N, d, in->router_w, E, sel_only ? NULL : in->router_bias, z, nthreads);
  int rc = orc_route(z, N, E, k, cfg->routing, in->token_ids, in->tid2eid, in->vocab,
                     sel_only ? in->router_bias : NULL, idx, gates, margin_out);
  if (rc != 0) {
    free(z); free(idx); free(gates); free(xn);
    return rc;
  }
  if (counts || offsets || perm || inv) {
    int32_t* c_ = (int32_t*)malloc(sizeof(int32_t) * (size_t)E);
    int32_t* o_ = (int32_t*)malloc(sizeof(int32_t) * (size_t)(E + 1));
    int32_t* p_ = (int32_t*)malloc(sizeof(int32_t) * (size_t)N * k);
    int32_t* i_ = (int32_t*)malloc(sizeof(int32_t) * (size_t)N * k);
    orc_bookkeeping(idx, N, k, E, c_, o_, p_, i_);
    if (counts) memcpy(counts, c_, sizeof(int32_t) * (size_t)E);
    if (offsets) memcpy(offsets, o_, sizeof(int32_t) * (size_t)(E + 1));
    if (perm) memcpy(perm, p_, sizeof(int32_t) * (size_t)N * k);
    if (inv) memcpy(inv, i_, sizeof(int32_t) * (size_t)N * k);
    free(c_); free(o_); free(p_); free(i_);
  }
  if (z_out) memcpy(z_out, z, sizeof(double) * (size_t)N * E);
  if (idx_out) memcpy(idx_out, idx, sizeof(int32_t) * (size_t)N * k);
  if (gates_out) memcpy(gates_out, gates, sizeof(double) * (size_t)N * k);

  if (out && n_out > 0) {
    const int has_shared = in->sh_gate_q != NULL || in->sh_gate_w != NULL;
    const int slots = k + has_shared;
    /* pairs of the listed rows, grouped by expert (E = shared), row order inside */
    const long n_pairs = (long)n_out * slots;
    int* exp_start = (int*)calloc((size_t)E + 2, sizeof(int));
    int* pair_row = (int*)malloc(sizeof(int) * (size_t)n_pairs);
    int* pair_of = (int*)malloc(sizeof(int) * (size_t)n_pairs); /* (out row, slot) -> pair */
    for (int o = 0; o < n_out; ++o) {
      int r = rows ? rows[o] : o;
      for (int j = 0; j < k; ++j) exp_start[idx[(size_t)r * k + j] + 1]++;
      if (has_shared) exp_start[E + 1]++;
    }
    for (int e = 0; e <= E; ++e) exp_start[e + 1] += exp_start[e];
    int* fill = (int*)malloc(sizeof(int) * (size_t)(E + 1));
    memcpy(fill, exp_start, sizeof(int) * (size_t)(E + 1));
    for (int o = 0; o < n_out; ++o) {
      int r = rows ? rows[o] : o;
      for (int j = 0; j < slots; ++j) {
        int e = (j < k) ? idx[(size_t)r * k + j] : E;
        int pp = fill[e]++;
        pair_row[pp] = o;
        pair_of[(size_t)o * slots + j] = pp;
      }
    }
    double* xd = (double*)malloc(sizeof(double) * (size_t)n_out * d);
    for (int o = 0; o < n_out; ++o) {
      int r = rows ? rows[o] : o;
      for (int i = 0; i < d; ++i) xd[(size_t)o * d + i] = orc_bf16(x[(size_t)r * d + i]);
    }
    double* h = (double*)malloc(sizeof(double) * (size_t)n_pairs * I);
    double* y = (double*)malloc(sizeof(double) * (size_t)n_pairs * d);
    ffn_ctx fc = {d, I, cfg->expert_format == 1, cfg->swiglu_limit,
                  in->gate_q, in->gate_s, in->up_q, in->up_s, in->down_q, in->down_s,
                  in->sh_gate_q, in->sh_gate_s, in->sh_up_q, in->sh_up_s, in->sh_down_q, in->sh_down_s,
                  in->sh_gate_w, in->sh_up_w, in->sh_down_w,
                  E, pair_row, exp_start, xd, h, y};
    orc_parallel(ffn_gateup_item, &fc, (long)(E + 1) * I, nthreads);
    orc_parallel(ffn_down_item, &fc, (long)(E + 1) * d, nthreads);
    /* out = y_shared + route_scale * sum_j g_j y_j (+ residual), slots in ascending order */
    for (int o = 0; o < n_out; ++o) {
      int r = rows ? rows[o] : o;
      for (int m = 0; m < d; ++m) {
        double acc = 0.0;
        for (int j = 0; j < k; ++j)
          acc += gates[(size_t)r * k + j] * y[(size_t)pair_of[(size_t)o * slots + j] * d + m];
        double sh = has_shared ? y[(size_t)pair_of[(size_t)o * slots + k] * d + m] : 0.0;
        double res = in->residual ? orc_bf16(in->residual[(size_t)r * d + m]) : 0.0;
        out[(size_t)o * d + m] = res + (sh + cfg->route_scale * acc);
      }
    }
    free(exp_start); free(pair_row); free(pair_of); free(fill); free(xd); free(h); free(y);
  }
  free(z); free(idx); free(gates); free(xn);
  return 0;
}
