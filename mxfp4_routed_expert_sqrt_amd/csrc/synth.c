/*
 * Seeded synthetic inputs for the routed MoE layer.
 *
 * This module only draws random numbers and encodes them into the storage
 * formats the layer consumes (bf16 activations, fp32 router weights, MXFP4
 * expert matrices, a hash-routing table).  It contains none of the layer's
 * own arithmetic (no router, no selection, no FFN): both the HIP path and the
 * fp64 oracle receive the bytes produced here.
 *
 * Random source: SplitMix64 (Steele, Lea & Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014) used as a counter-based
 * generator: the i-th draw of a stream is mix(key + (i+1)*gamma).  Every row of
 * every tensor has its own stream key derived from (seed, tags, indices), so
 * the bytes do not depend on the thread count.  Normals come from the
 * Marsaglia-Bray polar method (1964) on consecutive uniform pairs.
 *
 * Q2_K encoding: the GGUF Q2_K super-block layout (see encode_q2k_block).
 *
 * MXFP4 encoding (OCP Microscaling Formats v1.0, section 6.3 conversion):
 * per 32-element block the shared exponent is floor(log2(amax)) - 2 (2 is the
 * largest E2M1 exponent), stored as E8M0 = exponent + 127; every element is
 * divided by 2^exponent, rounded to the nearest E2M1 value with ties to the
 * even code, and saturated at +-6.  Element 2i sits in the low nibble of byte
 * i (one of the readings documented for the MoE weight format).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

/* Stream key for a tuple of up to five 64-bit tags. */
static uint64_t stream_key(uint64_t seed, uint64_t a, uint64_t b, uint64_t c, uint64_t d) {
  uint64_t k = mix64(seed + GAMMA);
  k = mix64(k ^ mix64(a + 2 * GAMMA));
  k = mix64(k ^ mix64(b + 3 * GAMMA));
  k = mix64(k ^ mix64(c + 4 * GAMMA));
  k = mix64(k ^ mix64(d + 5 * GAMMA));
  return k;
}

static inline uint64_t draw64(uint64_t key, uint64_t i) { return mix64(key + (i + 1) * GAMMA); }

/* Uniform in the open interval (0, 1). */
static inline double draw_unif(uint64_t key, uint64_t i) {
  return ((double)(draw64(key, i) >> 11) + 0.5) * 0x1.0p-53;
}

/* Fill out[0..n) with N(0, std) from one stream: Marsaglia-Bray polar method
 * (a pair (v1, v2) uniform on the unit disc gives two independent normals
 * v*sqrt(-2 ln s / s), s = v1^2 + v2^2; pairs outside the disc are skipped). */
static void fill_normal(uint64_t key, double std, long n, double* out) {
  uint64_t i = 0;
  long c = 0;
  while (c < n) {
    double v1 = 2.0 * draw_unif(key, i++) - 1.0;
    double v2 = 2.0 * draw_unif(key, i++) - 1.0;
    double s = v1 * v1 + v2 * v2;
    if (s >= 1.0 || s == 0.0) continue;
    double m = std * sqrt(-2.0 * log(s) / s);
    out[c++] = v1 * m;
    if (c < n) out[c++] = v2 * m;
  }
}

static inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  uint32_t rounding = 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)((u + rounding) >> 16);
}

/* ---- tiny static-partition thread pool ------------------------------------------ */

typedef void (*row_fn)(void* ctx, long row);
typedef struct { row_fn fn; void* ctx; long n; int t, nt; } job_t;

static void* job_main(void* p) {
  job_t* j = (job_t*)p;
  for (long r = j->t; r < j->n; r += j->nt) j->fn(j->ctx, r);
  return NULL;
}

static void parallel_rows(row_fn fn, void* ctx, long n, int nthreads) {
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  if (nthreads == 1 || n < 2) {
    for (long r = 0; r < n; ++r) fn(ctx, r);
    return;
  }
  pthread_t th[256];
  job_t jobs[256];
  int started = 0;
  for (int t = 0; t < nthreads; ++t) {
    jobs[t] = (job_t){fn, ctx, n, t, nthreads};
    if (pthread_create(&th[t], NULL, job_main, &jobs[t]) == 0) {
      ++started;
    } else {
      job_main(&jobs[t]);
      th[t] = 0;
    }
  }
  for (int t = 0; t < nthreads; ++t)
    if (th[t]) pthread_join(th[t], NULL);
  (void)started;
}

/* ---- activations ----------------------------------------------------------------- */

typedef struct { uint64_t seed, cfg_tag; long d; const int32_t* attempts; uint16_t* out; } x_ctx;

static void x_row(void* p, long r) {
  x_ctx* c = (x_ctx*)p;
  uint64_t attempt = c->attempts ? (uint64_t)c->attempts[r] : 0;
  uint64_t key = stream_key(c->seed, c->cfg_tag, 0x78 /* 'x' */, (uint64_t)r, attempt);
  double* buf = (double*)malloc(sizeof(double) * (size_t)(c->d + 1));
  fill_normal(key, 1.0, c->d, buf);
  for (long i = 0; i < c->d; ++i) c->out[r * c->d + i] = f32_to_bf16_rne((float)buf[i]);
  free(buf);
}

/* x[r][i] ~ N(0,1), rounded to fp32 then to bf16 (both round-to-nearest-even).
 * attempts[r] (may be NULL = all 0) selects the redraw of row r. */
void synth_x_bf16(uint64_t seed, uint64_t cfg_tag, long n_rows, long d, const int32_t* attempts,
                  uint16_t* out, int nthreads) {
  x_ctx c = {seed, cfg_tag, d, attempts, out};
  parallel_rows(x_row, &c, n_rows, nthreads);
}

/* ---- router weight ---------------------------------------------------------------- */

typedef struct { uint64_t seed, set_tag; long d; double std; float* out; } w_ctx;

static void wr_row(void* p, long e) {
  w_ctx* c = (w_ctx*)p;
  uint64_t key = stream_key(c->seed, c->set_tag, 0x72 /* 'r' */, (uint64_t)e, 0);
  double* buf = (double*)malloc(sizeof(double) * (size_t)(c->d + 1));
  fill_normal(key, c->std, c->d, buf);
  for (long i = 0; i < c->d; ++i) c->out[e * c->d + i] = (float)buf[i];
  free(buf);
}

void synth_router_f32(uint64_t seed, uint64_t set_tag, long n_experts, long d, double std, float* out,
                      int nthreads) {
  w_ctx c = {seed, set_tag, d, std, out};
  parallel_rows(wr_row, &c, n_experts, nthreads);
}

/* ---- MXFP4 encoding ---------------------------------------------------------------- */

/* Nearest E2M1 magnitude code (0..7) to a >= 0, ties to the even code, saturating
 * at 6.  The E2M1 magnitudes (OCP format: 1 sign, 2 exponent bits with bias 1,
 * 1 mantissa bit) are 0, 0.5, 1, 1.5, 2, 3, 4, 6; the thresholds below are the
 * midpoints between neighbours, and a midpoint goes to whichever neighbour has
 * the even code. */
static int e2m1_round(double a) {
  if (a <= 0.25) return 0;
  if (a < 0.75) return 1;
  if (a <= 1.25) return 2;
  if (a < 1.75) return 3;
  if (a <= 2.5) return 4;
  if (a < 3.5) return 5;
  if (a <= 5.0) return 6;
  return 7;
}

/* Encode 32 fp32 values into 16 packed bytes and one E8M0 byte. */
static void encode_block32(const float* v, uint8_t* q16, uint8_t* s1) {
  double amax = 0.0;
  for (int i = 0; i < 32; ++i) {
    double a = fabs((double)v[i]);
    if (a > amax) amax = a;
  }
  int x = 0;
  if (amax > 0.0) {
    int ex;
    frexp(amax, &ex); /* amax = m * 2^ex, m in [0.5, 1) -> floor(log2 amax) = ex - 1 */
    x = (ex - 1) - 2;
    if (x < -127) x = -127;
    if (x > 127) x = 127;
  }
  *s1 = (uint8_t)(x + 127);
  const double inv = ldexp(1.0, -x); /* exact power of two */
  for (int i = 0; i < 32; i += 2) {
    uint8_t nib[2];
    for (int h = 0; h < 2; ++h) {
      double t = (double)v[i + h] * inv;
      int code = e2m1_round(fabs(t));
      if (signbit(t)) code |= 8;
      nib[h] = (uint8_t)code;
    }
    q16[i / 2] = (uint8_t)(nib[0] | (nib[1] << 4));
  }
}

typedef struct {
  uint64_t seed, set_tag, mat_tag;
  long first_mat, rows, K;
  double std;
  uint8_t *q, *s;
} mx_ctx;

static void mx_row(void* p, long flat) {
  mx_ctx* c = (mx_ctx*)p;
  long m = flat / c->rows, n = flat % c->rows;
  uint64_t key = stream_key(c->seed, c->set_tag, c->mat_tag, (uint64_t)(c->first_mat + m), (uint64_t)n);
  double* buf = (double*)malloc(sizeof(double) * (size_t)(c->K + 1));
  float* f = (float*)malloc(sizeof(float) * (size_t)c->K);
  fill_normal(key, c->std, c->K, buf);
  for (long i = 0; i < c->K; ++i) f[i] = (float)buf[i];
  uint8_t* qrow = c->q + (size_t)flat * (size_t)(c->K / 2);
  uint8_t* srow = c->s + (size_t)flat * (size_t)(c->K / 32);
  for (long b = 0; b < c->K / 32; ++b) encode_block32(f + 32 * b, qrow + 16 * b, srow + b);
  free(f);
  free(buf);
}

/* n_mat matrices [rows][K] with entries ~N(0, std) as fp32, encoded to MXFP4.
 * Matrix m of the call is matrix (first_mat + m) of the stream family mat_tag.
 * q: [n_mat][rows][K/2], s: [n_mat][rows][K/32].  K must be a multiple of 32. */
int synth_mxfp4(uint64_t seed, uint64_t set_tag, uint64_t mat_tag, long first_mat, long n_mat, long rows,
                long K, double std, uint8_t* q, uint8_t* s, int nthreads) {
  if (K % 32 != 0 || rows <= 0 || n_mat < 0) return -1;
  mx_ctx c = {seed, set_tag, mat_tag, first_mat, rows, K, std, q, s};
  parallel_rows(mx_row, &c, n_mat * rows, nthreads);
  return 0;
}

/* Encode caller-given fp32 rows (used by hand-built test weights). */
void synth_encode_mxfp4(const float* v, long rows, long K, uint8_t* q, uint8_t* s) {
  for (long r = 0; r < rows; ++r)
    for (long b = 0; b < K / 32; ++b)
      encode_block32(v + r * K + 32 * b, q + r * (K / 2) + 16 * b, s + r * (K / 32) + b);
}

/* ---- Q2_K encoding -------------------------------------------------------------------- */

/* fp32 -> IEEE half bits, round to nearest even (overflow to infinity,
 * gradual underflow to subnormals). */
static uint16_t f32_to_f16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  const uint32_t sign = (u >> 16) & 0x8000u;
  const int32_t ex = (int32_t)((u >> 23) & 0xFF) - 127;
  uint32_t man = u & 0x7FFFFFu;
  if (ex == 128) return (uint16_t)(sign | 0x7C00u | (man ? 0x200u : 0u));
  if (ex > 15) return (uint16_t)(sign | 0x7C00u);
  if (ex >= -14) { /* normal half: 10 mantissa bits kept of 23 */
    uint32_t h = ((uint32_t)(ex + 15) << 10) | (man >> 13);
    const uint32_t rest = man & 0x1FFFu;
    if (rest > 0x1000u || (rest == 0x1000u && (h & 1u))) ++h; /* may carry into the exponent: still exact RNE */
    return (uint16_t)(sign | h);
  }
  if (ex < -25) return (uint16_t)sign;
  /* subnormal half: value = m * 2^-24 with m = (1.man) * 2^(ex + 24) */
  man |= 0x800000u;
  const int shift = -ex - 1; /* 14 .. 24: bits dropped from the 24-bit significand to units of 2^-24 */
  uint32_t h = man >> shift;
  const uint32_t rest = man & ((1u << shift) - 1u), half = 1u << (shift - 1);
  if (rest > half || (rest == half && (h & 1u))) ++h;
  return (uint16_t)(sign | h);
}

static double f16_bits_to_double(uint16_t h) {
  const int ex = (h >> 10) & 0x1F, man = h & 0x3FF;
  double v = ex == 0 ? ldexp((double)man, -24) : ldexp((double)(man | 0x400), ex - 25);
  return (h & 0x8000) ? -v : v;
}

/* One Q2_K super-block: 256 values into 84 bytes, the GGUF Q2_K block layout:
 * bytes 0-15 one byte per 16-value sub-block (low nibble its scale, high
 * nibble its min), bytes 16-79 the 2-bit quants (value t of the block in
 * byte 16 + 32*(t/128) + (t%32), bits 2*((t%128)/32)), then d and dmin as
 * half floats.  Value t decodes to d*scale*q - dmin*min of its sub-block t/16.
 * Quantiser (for synthetic inputs only): per sub-block the range [lo, hi]
 * with lo = min(0, smallest value) is cut in 3 steps, s = (hi - lo)/3 and
 * m = -lo; d = max s / 15 and dmin = max m / 15 (rounded to half), the 4-bit
 * scale and min round s/d and m/dmin, and each q rounds (v + dmin*min) /
 * (d*scale) into 0..3. */
static void encode_q2k_block(const float* v, uint8_t* blk) {
  double s[16], m[16], smax = 0.0, mmax = 0.0;
  for (int sb = 0; sb < 16; ++sb) {
    double lo = 0.0, hi = -INFINITY;
    for (int i = 0; i < 16; ++i) {
      const double x = v[16 * sb + i];
      if (x < lo) lo = x;
      if (x > hi) hi = x;
    }
    if (hi < lo) hi = lo;
    s[sb] = (hi - lo) / 3.0;
    m[sb] = -lo;
    if (s[sb] > smax) smax = s[sb];
    if (m[sb] > mmax) mmax = m[sb];
  }
  const uint16_t dh = f32_to_f16_rne((float)(smax / 15.0)), mh = f32_to_f16_rne((float)(mmax / 15.0));
  const double d = f16_bits_to_double(dh), dmin = f16_bits_to_double(mh);
  memset(blk, 0, 84);
  for (int sb = 0; sb < 16; ++sb) {
    int sc = d > 0.0 ? (int)lrint(s[sb] / d) : 0, mn = dmin > 0.0 ? (int)lrint(m[sb] / dmin) : 0;
    sc = sc < 0 ? 0 : (sc > 15 ? 15 : sc);
    mn = mn < 0 ? 0 : (mn > 15 ? 15 : mn);
    blk[sb] = (uint8_t)(sc | (mn << 4));
    const double step = d * sc, off = dmin * mn;
    for (int i = 0; i < 16; ++i) {
      const int t = 16 * sb + i;
      int q = step > 0.0 ? (int)lrint(((double)v[t] + off) / step) : 0;
      q = q < 0 ? 0 : (q > 3 ? 3 : q);
      blk[16 + 32 * (t / 128) + (t % 32)] |= (uint8_t)(q << (2 * ((t % 128) / 32)));
    }
  }
  blk[80] = (uint8_t)(dh & 0xFF);
  blk[81] = (uint8_t)(dh >> 8);
  blk[82] = (uint8_t)(mh & 0xFF);
  blk[83] = (uint8_t)(mh >> 8);
}

typedef struct {
  uint64_t seed, set_tag, mat_tag;
  long first_mat, rows, K;
  double std;
  uint8_t* out;
} q2k_ctx;

static void q2k_row(void* p, long flat) {
  q2k_ctx* c = (q2k_ctx*)p;
  long m = flat / c->rows, n = flat % c->rows;
  uint64_t key = stream_key(c->seed, c->set_tag, c->mat_tag, (uint64_t)(c->first_mat + m), (uint64_t)n);
  double* buf = (double*)malloc(sizeof(double) * (size_t)(c->K + 1));
  float* f = (float*)malloc(sizeof(float) * (size_t)c->K);
  fill_normal(key, c->std, c->K, buf);
  for (long i = 0; i < c->K; ++i) f[i] = (float)buf[i];
  uint8_t* row = c->out + (size_t)flat * (size_t)(c->K / 256) * 84;
  for (long b = 0; b < c->K / 256; ++b) encode_q2k_block(f + 256 * b, row + 84 * b);
  free(f);
  free(buf);
}

/* n_mat matrices [rows][K] with entries ~N(0, std), encoded to Q2_K blocks:
 * out [n_mat][rows][K/256][84].  K must be a multiple of 256. */
int synth_q2k(uint64_t seed, uint64_t set_tag, uint64_t mat_tag, long first_mat, long n_mat, long rows, long K,
              double std, uint8_t* out, int nthreads) {
  if (K % 256 != 0 || rows <= 0 || n_mat < 0) return -1;
  q2k_ctx c = {seed, set_tag, mat_tag, first_mat, rows, K, std, out};
  parallel_rows(q2k_row, &c, n_mat * rows, nthreads);
  return 0;
}

/* Encode caller-given fp32 rows [rows][K] to Q2_K blocks (hand-built test weights). */
void synth_encode_q2k(const float* v, long rows, long K, uint8_t* out) {
  for (long r = 0; r < rows; ++r)
    for (long b = 0; b < K / 256; ++b) encode_q2k_block(v + r * K + 256 * b, out + (r * (K / 256) + b) * 84);
}

/* ---- hash routing tables ------------------------------------------------------------ */

typedef struct { uint64_t seed, set_tag; int E, k; int32_t* out; } t_ctx;

/* Uniform integer in [0, n) by Lemire's multiply-shift on the top 32 bits. */
static inline uint32_t draw_below(uint64_t key, uint64_t i, uint32_t n) {
  return (uint32_t)(((draw64(key, i) >> 32) * (uint64_t)n) >> 32);
}

static void tid_row(void* p, long v) {
  t_ctx* c = (t_ctx*)p;
  uint64_t key = stream_key(c->seed, c->set_tag, 0x74 /* 't' */, (uint64_t)v, 0);
  int pool[1024];
  for (int e = 0; e < c->E; ++e) pool[e] = e;
  /* first k steps of a Fisher-Yates shuffle: k distinct ids, uniform without replacement */
  for (int j = 0; j < c->k; ++j) {
    uint32_t pick = (uint32_t)j + draw_below(key, (uint64_t)j, (uint32_t)(c->E - j));
    int t = pool[j];
    pool[j] = pool[pick];
    pool[pick] = t;
    c->out[v * c->k + j] = pool[j];
  }
}

/* tid2eid[vocab][k]: k distinct expert ids in [0, E) per token id, in draw order. */
int synth_tid2eid(uint64_t seed, uint64_t set_tag, long vocab, int E, int k, int32_t* out, int nthreads) {
  if (E < 1 || E > 1024 || k < 1 || k > E) return -1;
  t_ctx c = {seed, set_tag, E, k, out};
  parallel_rows(tid_row, &c, vocab, nthreads);
  return 0;
}

/* Token ids uniform over [0, vocab). */
void synth_token_ids(uint64_t seed, uint64_t cfg_tag, long n, long vocab, int32_t* out) {
  uint64_t key = stream_key(seed, cfg_tag, 0x69 /* 'i' */, 0, 0);
  for (long r = 0; r < n; ++r) out[r] = (int32_t)draw_below(key, (uint64_t)r, (uint32_t)vocab);
}

/* A uniformly random permutation of [0, n) (Fisher-Yates). */
void synth_permutation(uint64_t seed, uint64_t tag, long n, int32_t* out) {
  uint64_t key = stream_key(seed, tag, 0x70 /* 'p' */, 0, 0);
  for (long i = 0; i < n; ++i) out[i] = (int32_t)i;
  for (long i = n - 1; i > 0; --i) {
    long j = (long)draw_below(key, (uint64_t)i, (uint32_t)(i + 1));
    int32_t t = out[i];
    out[i] = out[j];
    out[j] = t;
  }
}
