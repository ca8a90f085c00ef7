/*
 * TAH-Quant reference oracle — TEST INFRASTRUCTURE ONLY (see tah_ref.h).
 *
 * Source of every step: "TAH-Quant: Effective Activation Quantization in
 * Pipeline Parallelism over Slow Network" (arXiv 2506.01352v2):
 *   §3.1  tile-wise group quantization (tile of G contiguous channels per token,
 *         own scale and zero-point per tile);
 *   §3.2  allocation tiles, Eq. (1) normalized magnitudes, Eq. (2) entropy,
 *         top-p% selection per sample, 1-bit width map;
 *   §3.3  Eq. (3) outlier ratio vs tau, pivot swap P_d, Eq. (4) tile-local
 *         Hadamard, asymmetric uniform quantizer, inverse by H^T;
 *   §3.4  mixed precisions + metadata packed into one fixed-size uint8 stream;
 *   Algorithm 1: the sender quantizes, the receiver dequantizes;
 *   Appendix F: tau = 0 always transforms, tau = inf never does.
 * The Sylvester ordering of H_G follows the Hadamard quantizer section of
 * "Training Transformers with 4-bit Integers" (arXiv 2306.11987), and the
 * low-nibble-first code order follows that paper's INT4 packing appendix.
 *
 * Where the pages leave a step open, the reading taken is stated next to the
 * code that implements it below.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fPIC -shared (no fast-math), so
 * every fp32 operation rounds exactly once, in the order written.
 */
#include "tah_ref.h"

#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

/* ϱ (Eq. 3): a "small positive constant". Reading: 2^-40. (The ε of Eq. 1 and
 * the ς of Eq. 2 only guard zeros; see tahref_entropy.) */
static const float kRho = 0x1p-40f;

/* ------------------------------------------------------------------ */
/* small helpers                                                      */
/* ------------------------------------------------------------------ */

static uint32_t f2u(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static float u2f(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

static float bf16_to_f32(uint16_t h) { return u2f((uint32_t)h << 16); }

/* fp32 -> bf16, round to nearest, ties to even (finite inputs). */
static uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = f2u(f);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) return (uint16_t)((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

/* Smallest bf16 value >= f, for f >= 0 finite. */
static uint16_t f32_to_bf16_up(float f) {
  uint32_t u = f2u(f);
  if (u & 0xffffu) u = (u & 0xffff0000u) + 0x10000u;
  return (uint16_t)(u >> 16);
}

static int64_t align256(int64_t v) { return (v + 255) & ~(int64_t)255; }

static void put_u8(uint8_t* p, int64_t off, uint32_t v) { p[off] = (uint8_t)v; }
static void put_u16(uint8_t* p, int64_t off, uint32_t v) {
  p[off] = (uint8_t)v;
  p[off + 1] = (uint8_t)(v >> 8);
}
static void put_u32(uint8_t* p, int64_t off, uint32_t v) {
  for (int i = 0; i < 4; ++i) p[off + i] = (uint8_t)(v >> (8 * i));
}
static void put_u64(uint8_t* p, int64_t off, uint64_t v) {
  for (int i = 0; i < 8; ++i) p[off + i] = (uint8_t)(v >> (8 * i));
}
static uint32_t get_u16(const uint8_t* p, int64_t off) { return (uint32_t)p[off] | ((uint32_t)p[off + 1] << 8); }
static uint32_t get_u32(const uint8_t* p, int64_t off) {
  uint32_t v = 0;
  for (int i = 0; i < 4; ++i) v |= (uint32_t)p[off + i] << (8 * i);
  return v;
}

static int ilog2(int v) {
  int l = 0;
  while ((1 << l) < v) ++l;
  return l;
}

/*
 * The budget as the decimal it stands for. The pages state the split as a
 * percentage (80% INT4 / 20% INT3, §3.2 and §5.1), i.e. a budget of 3.8 bits,
 * which fp32 cannot hold: 3.8f is 3.7999999523..., and floor(0.79999995 N)
 * would give 0.8 N - 1 whenever 0.8 N is an integer. Reading: the budget is
 * the shortest decimal that rounds to the given fp32 value (fewest fractional
 * digits, the nearest such decimal), B = num / den with den = 10^digits.
 * Only budgets below 8 (the widest candidate) ever need it, so at most eight
 * fractional digits and num, den < 2^30.
 */
static void budget_decimal(float B, int64_t* num, int64_t* den) {
  char buf[64];
  for (int digits = 0; digits <= 9; ++digits) {
    snprintf(buf, sizeof buf, "%.*f", digits, (double)B); /* correctly rounded to `digits` places */
    if (strtof(buf, NULL) != B) continue;
    int64_t n = 0, d = 1;
    int frac = 0;
    for (const char* c = buf; *c; ++c) {
      if (*c == '.') {
        frac = 1;
        continue;
      }
      n = n * 10 + (*c - '0');
      if (frac) d *= 10;
    }
    *num = n;
    *den = d;
    return;
  }
  /* unreachable for finite B in [1, 8]: nine digits always round-trip */
  *num = (int64_t)floor((double)B * 1e9);
  *den = 1000000000;
}

/* floor((B - base) * N / step) for the decimal budget B, base <= B, exactly. */
static int64_t budget_floor(float B, int base, int64_t N, int step) {
  int64_t num, den;
  budget_decimal(B, &num, &den);
  const __int128 excess = (__int128)num - (__int128)base * den; /* (B - base) * den >= 0 */
  return (int64_t)((excess * N) / ((__int128)step * den));
}

/* ------------------------------------------------------------------ */
/* parameters and payload layout                                      */
/* ------------------------------------------------------------------ */

/*
 * Width pair and k (§3.2 "Top-p% tile selection"): the paper gives two widths,
 * INT4 for the top p% of a sample's allocation tiles by entropy and INT3 for
 * the rest. Reading for a budget B over a candidate list: b_lo = largest
 * candidate <= B, b_hi = smallest candidate > B (b_lo if none), and
 * p = (B - b_lo)/(b_hi - b_lo), so k = floor(p * SM) of the SM allocation tiles
 * of a sample get b_hi and the average code width never exceeds B. The budget
 * counts code bits only; the paper quotes its metadata bits separately (§3.4).
 *
 * Allocation tile (§3.2 "Tile decomposition"): A channels, aligned with the
 * quantization tiles, so A = kA * G; it must divide hidden. A = G is the
 * paper's default, A = hidden its token-level special case. Every quantization
 * tile takes the width of the allocation tile that holds it.
 */
int tahref_plan_make(int64_t tokens, int64_t hidden, const tahref_params* p, tahref_plan* o) {
  if (!p || !o) return TAHREF_ERR_INVALID_ARG;
  memset(o, 0, sizeof(*o));
  if (tokens < 0 || hidden <= 0) return TAHREF_ERR_INVALID_ARG;
  int G = p->tile;
  if (G < 8 || G > 128 || (G & (G - 1))) return TAHREF_ERR_INVALID_ARG;
  if (hidden % G) return TAHREF_ERR_INVALID_ARG;
  if (p->n_candidates < 1 || p->n_candidates > 4) return TAHREF_ERR_INVALID_ARG;
  for (int i = 0; i < p->n_candidates; ++i) {
    if (p->candidates[i] < 1 || p->candidates[i] > 8) return TAHREF_ERR_INVALID_ARG;
    if (i > 0 && p->candidates[i] <= p->candidates[i - 1]) return TAHREF_ERR_INVALID_ARG;
  }
  if (!isfinite(p->bit_budget)) return TAHREF_ERR_INVALID_ARG;
  if (isnan(p->tau) || p->tau < 0.0f) return TAHREF_ERR_INVALID_ARG;
  if (p->tokens_per_sample < 0) return TAHREF_ERR_INVALID_ARG;
  int64_t S = p->tokens_per_sample == 0 ? tokens : p->tokens_per_sample;
  if (S > 0 && tokens % S) return TAHREF_ERR_INVALID_ARG;
  int64_t A = p->alloc_tile == 0 ? G : p->alloc_tile;
  if (A < G || A % G || hidden % A) return TAHREF_ERR_INVALID_ARG;
  if (p->allocator != 0 && p->allocator != 1) return TAHREF_ERR_INVALID_ARG;
  if ((float)p->candidates[0] > p->bit_budget) return TAHREF_ERR_BUDGET_INFEASIBLE;

  int b_lo = p->candidates[0], b_hi = -1;
  for (int i = 0; i < p->n_candidates; ++i) {
    if ((float)p->candidates[i] <= p->bit_budget) b_lo = p->candidates[i];
    else if (b_hi < 0) b_hi = p->candidates[i];
  }
  if (b_hi < 0) b_hi = b_lo;

  o->tokens = tokens;
  o->hidden = hidden;
  o->S = S;
  o->nsamples = S > 0 ? tokens / S : 0;
  o->G = G;
  o->log2G = ilog2(G);
  o->M = hidden / G;
  o->tiles = tokens * o->M;
  o->tiles_per_sample = S * o->M;
  o->A = A;
  o->kA = A / G;
  o->MA = hidden / A;
  o->atiles = tokens * o->MA;
  o->atiles_per_sample = S * o->MA;
  o->allocator = p->allocator;
  o->nblocks = (o->tiles + 63) / 64;
  if (p->allocator == 0) {
    o->b_lo = b_lo;
    o->b_hi = b_hi;
    /* k = floor(p N) with p = (B - b_lo) / (b_hi - b_lo) and B the decimal budget */
    if (b_hi == b_lo || o->atiles_per_sample == 0)
      o->k = 0;
    else
      o->k = budget_floor(p->bit_budget, b_lo, o->atiles_per_sample, b_hi - b_lo);
  } else {
    /* greedy (tahref_allocate_greedy): every candidate may occur; b_lo and b_hi
     * record the narrowest and the widest, and a sample may spend R bits above
     * c_1 over its allocation tiles, R = floor((B - c_1) N), at most what
     * every tile at the widest candidate would take */
    const int c1 = p->candidates[0], cn = p->candidates[p->n_candidates - 1];
    o->b_lo = c1;
    o->b_hi = cn;
    o->k = 0;
    const int64_t N = o->atiles_per_sample;
    const int64_t cap = (int64_t)(cn - c1) * N;
    /* R = floor((B - c_1) N) with B the decimal budget; from B = c_n on, everything fits */
    o->R = p->bit_budget >= (float)cn ? cap : budget_floor(p->bit_budget, c1, N, 1);
    if (o->R > cap) o->R = cap;
    /* the block table holds the running sum of code widths in 32 bits */
    if ((uint64_t)o->tiles * (uint64_t)cn > 0xffffffffull) return TAHREF_ERR_INVALID_ARG;
  }
  o->off_table = 256;
  o->off_bitmap = align256(o->off_table + 4 * o->nblocks);
  /* width map: 1 bit per tile (allocator 0) or 2 bits (allocator 1) */
  o->off_side = align256(o->off_bitmap + (p->allocator == 0 ? 8 : 16) * o->nblocks);
  o->off_scale = align256(o->off_side + o->tiles);
  o->off_zero = align256(o->off_scale + 2 * o->tiles);
  o->off_codes = align256(o->off_zero + 4 * o->tiles);
  if (p->allocator == 0) {
    int64_t nhi = o->k * o->kA * o->nsamples; /* quantization tiles at b_hi */
    o->code_bytes = (o->tiles * G * o->b_lo + nhi * G * (o->b_hi - o->b_lo)) / 8;
  } else {
    /* the most a sample's code blocks can take: (A/8) bytes per unit of width
     * per allocation tile, c_1 N + R units (A is a multiple of 8) */
    o->code_bytes = o->nsamples * (o->A / 8) * ((int64_t)o->b_lo * o->atiles_per_sample + o->R);
  }
  o->total = align256(o->off_codes + o->code_bytes);
  return TAHREF_OK;
}

/* 128-byte header; bytes 128..255 of the first section are zero. */
static void write_header(uint8_t* P, const tahref_plan* pl, const tahref_params* p, int x_dtype) {
  memset(P, 0, 256);
  put_u32(P, 0, 0x51484154u); /* "TAHQ" */
  put_u16(P, 4, 2);
  put_u8(P, 6, (uint32_t)x_dtype);
  put_u8(P, 7, (uint32_t)pl->log2G);
  put_u64(P, 8, (uint64_t)pl->tokens);
  put_u64(P, 16, (uint64_t)pl->hidden);
  put_u64(P, 24, (uint64_t)pl->S);
  put_u32(P, 32, f2u(p->bit_budget));
  put_u32(P, 36, f2u(p->tau));
  put_u8(P, 40, (uint32_t)p->n_candidates);
  for (int i = 0; i < p->n_candidates; ++i) put_u8(P, 41 + i, p->candidates[i]);
  put_u8(P, 45, (uint32_t)pl->b_lo);
  put_u8(P, 46, (uint32_t)pl->b_hi);
  put_u64(P, 48, (uint64_t)(pl->allocator == 0 ? pl->k : pl->R));
  put_u64(P, 56, (uint64_t)pl->tiles);
  put_u64(P, 64, (uint64_t)pl->off_table);
  put_u64(P, 72, (uint64_t)pl->off_bitmap);
  put_u64(P, 80, (uint64_t)pl->off_side);
  put_u64(P, 88, (uint64_t)pl->off_scale);
  put_u64(P, 96, (uint64_t)pl->off_zero);
  put_u64(P, 104, (uint64_t)pl->off_codes);
  put_u64(P, 112, (uint64_t)pl->total);
  put_u32(P, 120, (uint32_t)pl->A);
  put_u8(P, 124, (uint32_t)pl->allocator);
}

/* ------------------------------------------------------------------ */
/* per-tile building blocks                                           */
/* ------------------------------------------------------------------ */

/*
 * log2 used by the entropy of Eq. (2) (the page writes "log"; any base ranks
 * tiles the same way). For finite u >= 0 with fp32 bits b:
 *   E = the frexp exponent (u = m * 2^E, m in [0.5, 1); E = 0 for u = 0),
 *   j = bits 16..22 of b (the top 7 stored mantissa bits), w = bits 0..15,
 *   T[j] = fp32(log2(1 + j/128) - 1),
 *   D[j] = fp32((log2(1 + (j+1)/128) - log2(1 + j/128)) / 2^16),
 *   log2s(u) = fmaf((float)w, D[j], (float)E + T[j]).
 * For u of the form (1 + j/128) * 2^e (every bf16 value) w = 0 and the result
 * is log2(u) rounded twice (T, then the sum); otherwise the mantissa is
 * interpolated linearly between the two neighbouring 7-bit points, with an
 * error below 1.15e-5. T and D are computed here in double precision from
 * the C library's log2 and rounded once to fp32. log2s(0) = -1 (it is only
 * ever multiplied by 0).
 */
static float g_T[128], g_D[128];
static int g_tab_ready = 0;

static void log2_tables(void) {
  if (g_tab_ready) return;
  for (int j = 0; j < 128; ++j) {
    const double a = log2(1.0 + j / 128.0), b = log2(1.0 + (j + 1) / 128.0);
    g_T[j] = (float)(a - 1.0);
    g_D[j] = (float)((b - a) / 65536.0);
  }
  g_tab_ready = 1;
}

float tahref_log2s(float u) {
  log2_tables();
  uint32_t b;
  memcpy(&b, &u, 4);
  int e;
  (void)frexpf(u, &e);
  const int j = (int)((b >> 16) & 127u);
  const float w = (float)(b & 0xffffu);
  return fmaf(w, g_D[j], (float)e + g_T[j]);
}

/*
 * Unnormalized Sylvester-ordered fast Walsh-Hadamard transform, v <- H_G v,
 * with H_G[i][j] = (-1)^popcount(i & j) (H_1 = [1], H_2k = [[H, H], [H, -H]]).
 * Stage order h = 1, 2, ..., G/2; each butterfly maps (a, b) to (a + b, a - b).
 * The 1/sqrt(G) of Eq. (4) is not applied: min/max asymmetric quantization is
 * scale invariant, so the codes are those of the normalized transform, and the
 * inverse applies the whole 1/G at the receiver (H_G is symmetric, H_G^2 = G I).
 */
void tahref_fwht(float* v, int G) {
  for (int h = 1; h < G; h <<= 1)
    for (int j = 0; j < G; ++j)
      if ((j & h) == 0) {
        float a = v[j], b = v[j + h];
        v[j] = a + b;
        v[j + h] = a - b;
      }
}

/*
 * Entropy of a tile of G channels, Eq. (1)-(2):
 *   p_k = |a_k| / ||a||_1,   H = -sum_k p_k log2 p_k.
 * Reading: Eq. (2) as printed has no minus sign, but the text says H is high
 * for evenly spread energy and low for a sharp outlier, which is Shannon's
 * entropy; the minus sign is restored. The ε of Eq. (1) and the ς inside the
 * log only keep zeros finite; here they are taken as 0, a zero |a_k| adds
 * nothing (0 log 0 = 0) and an all-zero tile has H = 0.
 * Since sum_k p_k = 1, H = log2 L - (1/L) sum_k |a_k| log2 |a_k| with
 * L = ||a||_1, and that is the form evaluated (one log per element, of the
 * input value itself):
 *   L = sum |a_k| left to right; S = sum fmaf(|a_k|, log2s(|a_k|), S) left to
 *   right from 0; H = log2s(L) - S / L (L > 0), H = 0 (L = 0).
 */
static void entropy_sums(const float* alpha, int n, float* L, float* S) {
  float l1 = 0.0f;
  for (int k = 0; k < n; ++k) l1 = l1 + fabsf(alpha[k]);
  float s = 0.0f;
  for (int k = 0; k < n; ++k) {
    const float a = fabsf(alpha[k]);
    s = fmaf(a, tahref_log2s(a), s);
  }
  *L = l1;
  *S = s;
}

static float entropy_from_sums(float L, float S) {
  if (!(L > 0.0f)) return 0.0f;
  return tahref_log2s(L) - S / L;
}

float tahref_entropy(const float* alpha, int G) {
  float L, S;
  entropy_sums(alpha, G, &L, &S);
  return entropy_from_sums(L, S);
}

/*
 * Entropy of an allocation tile of A = kA * G channels (§3.2: the distribution
 * of Eq. (1) is formed over all A channels). Same identity as above; the
 * summation order is a reading (the pages fix none): L and S are first summed
 * inside each of the kA quantization tiles as in tahref_entropy, then those
 * partial sums are added left to right from 0. For A = G this is exactly
 * tahref_entropy.
 */
float tahref_alloc_entropy(const float* alpha, int A, int G) {
  float L = 0.0f, S = 0.0f;
  for (int g = 0; g < A / G; ++g) {
    float l, s;
    entropy_sums(alpha + (int64_t)g * G, G, &l, &s);
    L = L + l;
    S = S + s;
  }
  return entropy_from_sums(L, S);
}

/*
 * Outlier heuristic, Eq. (3): r = |a^(1)| / (|a^(2)| + ϱ), transform iff r > tau.
 * m1 = largest |a_k|; d = the smallest index holding it (pivot, §3.3);
 * m2 = largest |a_k| over k != d, so tied maxima give r ~ 1 and no transform.
 * The ratio test is evaluated without a division as m1 > tau * (m2 + ϱ).
 * tau = +inf never flags; tau = 0 flags every tile that is not all zero.
 */
int tahref_outlier(const float* alpha, int G, float tau, int* d_out, float* m1_out, float* m2_out) {
  float m1 = fabsf(alpha[0]);
  int d = 0;
  for (int k = 1; k < G; ++k)
    if (fabsf(alpha[k]) > m1) {
      m1 = fabsf(alpha[k]);
      d = k;
    }
  float m2 = 0.0f;
  for (int k = 0; k < G; ++k)
    if (k != d && fabsf(alpha[k]) > m2) m2 = fabsf(alpha[k]);
  float thr = tau * (m2 + kRho);
  if (d_out) *d_out = d;
  if (m1_out) *m1_out = m1;
  if (m2_out) *m2_out = m2;
  return m1 > thr;
}

/*
 * Asymmetric uniform quantizer at width b (§3.1, §3.3): per-tile zero-point
 * lo = min y and step s from the range, codes q_k in [0, 2^b - 1].
 *   lo = min y, hi = max y (both + 0 so a -0 becomes +0);
 *   s32 = (hi - lo) / (2^b - 1);  s = smallest bf16 >= s32 (the stored scale);
 *   s = 0 when it is below 2^-126 (a range that underflows is stored as constant);
 *   inv = s > 0 ? 1/s : 0;
 *   q_k = round-half-even of the exact product (y_k - lo) * inv, clamped to [0, 2^b - 1].
 * The clamp never binds for finite input (the step is rounded up), but it is
 * written out so the definition is total.
 */
void tahref_quantize(const float* y, int G, int b, float* lo_out, float* s_out, uint32_t* q) {
  float lo = y[0], hi = y[0];
  for (int k = 1; k < G; ++k) {
    if (y[k] < lo) lo = y[k];
    if (y[k] > hi) hi = y[k];
  }
  lo = lo + 0.0f;
  hi = hi + 0.0f;
  const uint32_t L = (1u << b) - 1u;
  float s32 = (hi - lo) / (float)L;
  float s = bf16_to_f32(f32_to_bf16_up(s32));
  if (!(s >= 0x1p-126f)) s = 0.0f;
  float inv = s > 0.0f ? 1.0f / s : 0.0f;
  for (int k = 0; k < G; ++k) {
    float t = y[k] - lo;
    double v = nearbyint((double)t * (double)inv); /* product of two fp32 is exact in double */
    if (v < 0.0) v = 0.0;
    if (v > (double)L) v = (double)L;
    q[k] = (uint32_t)v;
  }
  *lo_out = lo;
  *s_out = s;
}

/*
 * Receiver side (Algorithm 1, the receiver's step; inverse of §3.3 by H^T):
 *   yhat_k = fmaf(q_k, s, lo);
 *   flagged tile: z = H_G yhat, x'_k = z_k * (1/G) (exact), then undo the pivot swap;
 *   otherwise x = yhat.
 */
void tahref_dequantize(const uint32_t* q, int G, float s, float lo, int flag, int d, float* xhat) {
  for (int k = 0; k < G; ++k) xhat[k] = fmaf((float)q[k], s, lo);
  if (flag) {
    tahref_fwht(xhat, G);
    const float invG = 1.0f / (float)G;
    for (int k = 0; k < G; ++k) xhat[k] = xhat[k] * invG;
    float t = xhat[0];
    xhat[0] = xhat[d];
    xhat[d] = t;
  }
}

/*
 * Top-p% selection of one sample (§3.2): rank the N tiles by entropy, highest
 * first; the first k get the higher width. Reading: equal entropies rank the
 * lower tile index first, so the selection is unique.
 */
typedef struct {
  float h;
  int64_t u;
} hkey;

static int cmp_hkey(const void* a, const void* b) {
  const hkey* x = (const hkey*)a;
  const hkey* y = (const hkey*)b;
  if (x->h > y->h) return -1;
  if (x->h < y->h) return 1;
  return (x->u < y->u) ? -1 : (x->u > y->u);
}

int tahref_allocate(const float* H, int64_t N, int64_t k, uint8_t* hi) {
  hkey* keys = (hkey*)malloc(sizeof(hkey) * (size_t)(N > 0 ? N : 1));
  if (!keys) return TAHREF_ERR_INVALID_ARG;
  for (int64_t u = 0; u < N; ++u) {
    keys[u].h = H[u];
    keys[u].u = u;
    hi[u] = 0;
  }
  qsort(keys, (size_t)N, sizeof(hkey), cmp_hkey);
  for (int64_t i = 0; i < k && i < N; ++i) hi[keys[i].u] = 1;
  free(keys);
  return TAHREF_OK;
}

/*
 * Allocation over every candidate width (allocator 1). The pages rank tiles by
 * entropy and give the top p% the higher of two widths; they define no rule
 * for three or more widths in one sample, so this one is a reading of that
 * ranking as a distortion budget:
 *   - a uniform quantizer of width b over a range D has mean-square error
 *     proportional to D^2 Delta(b), Delta(b) = (2^b - 1)^-2;
 *   - tile u weighs w_u = 2^(2 H_u) (higher entropy, larger weight, as the
 *     ranking of §3.2 asks), so the sample's objective is
 *     sum_u w_u Delta(b_u) under sum_u (b_u - c_1) <= R;
 *   - every tile starts at c_1; upgrade j of tile u (c_j -> c_(j+1), costing
 *     c_(j+1) - c_j bits) lowers the objective by w_u (Delta(c_j) - Delta(c_(j+1))),
 *     and its gain per bit has the base-2 logarithm
 *       kappa(u, j) = 2 H_u + lambda_j,
 *       lambda_j = log2((Delta(c_j) - Delta(c_(j+1))) / (c_(j+1) - c_j));
 *   - upgrades are taken in the order kappa descending, then u ascending,
 *     then j ascending, for as long as the bits taken stay within R; the
 *     first upgrade that would exceed R ends the allocation.
 * Delta is convex, so lambda_j decreases with j and a tile's upgrades come in
 * order. With two candidates every upgrade costs the same, the order is the
 * entropy ranking and the rule is §3.2's top-k.
 * Precision: lambda_j in double from the C library's log2, rounded once to
 * fp32; kappa = 2 H_u + lambda_j in fp32 (2 H_u is exact), the precision the
 * GPU decides in.
 */
static double greedy_delta(int b) {
  const double L = ldexp(1.0, b) - 1.0;
  return 1.0 / (L * L);
}

int tahref_greedy_lambda(int n, const uint8_t* cand, float* lam) {
  if (n < 1 || n > 4 || !cand || !lam) return TAHREF_ERR_INVALID_ARG;
  for (int j = 0; j + 1 < n; ++j) {
    const double gain = greedy_delta(cand[j]) - greedy_delta(cand[j + 1]);
    lam[j] = (float)log2(gain / (double)(cand[j + 1] - cand[j]));
  }
  return TAHREF_OK;
}

typedef struct {
  float kappa;
  int64_t u;
  int j;
} upgrade;

static int cmp_upgrade(const void* a, const void* b) {
  const upgrade* x = (const upgrade*)a;
  const upgrade* y = (const upgrade*)b;
  if (x->kappa > y->kappa) return -1;
  if (x->kappa < y->kappa) return 1;
  if (x->u != y->u) return x->u < y->u ? -1 : 1;
  return (x->j > y->j) - (x->j < y->j);
}

int tahref_allocate_greedy(const float* H, int64_t N, int n, const uint8_t* cand, int64_t R, uint8_t* level) {
  float lam[3];
  if (N < 0 || R < 0 || tahref_greedy_lambda(n, cand, lam) != TAHREF_OK) return TAHREF_ERR_INVALID_ARG;
  for (int64_t u = 0; u < N; ++u) level[u] = 0;
  const int64_t nu = N * (n - 1);
  if (nu == 0) return TAHREF_OK;
  upgrade* up = (upgrade*)malloc(sizeof(upgrade) * (size_t)nu);
  if (!up) return TAHREF_ERR_INVALID_ARG;
  for (int64_t u = 0; u < N; ++u)
    for (int j = 0; j + 1 < n; ++j) {
      upgrade* e = &up[u * (n - 1) + j];
      e->kappa = 2.0f * H[u] + lam[j];
      e->u = u;
      e->j = j;
    }
  qsort(up, (size_t)nu, sizeof(upgrade), cmp_upgrade);
  int64_t spent = 0;
  for (int64_t i = 0; i < nu; ++i) {
    const int cost = cand[up[i].j + 1] - cand[up[i].j];
    if (spent + cost > R) break;
    spent += cost;
    level[up[i].u] += 1; /* the order takes a tile's upgrades j = 0, 1, ... in turn */
  }
  free(up);
  return TAHREF_OK;
}

/* ------------------------------------------------------------------ */
/* whole tensor                                                       */
/* ------------------------------------------------------------------ */

/* Tile t of the [tokens, hidden] tensor: row t / M, channels (t % M) * G ... + G - 1 (§3.1). */
static void load_tile(const void* x, int dtype, const tahref_plan* pl, int64_t t, float* a) {
  int64_t row = t / pl->M, m = t % pl->M;
  int64_t base = row * pl->hidden + m * pl->G;
  if (dtype == TAHREF_F32) {
    const float* xf = (const float*)x;
    for (int k = 0; k < pl->G; ++k) a[k] = xf[base + k];
  } else {
    const uint16_t* xh = (const uint16_t*)x;
    for (int k = 0; k < pl->G; ++k) a[k] = bf16_to_f32(xh[base + k]);
  }
}

/* Entropy of every allocation tile (H[atiles]), the per-sample selection over
 * allocation tiles, and each quantization tile's width index (hi[tiles]: 0/1
 * for b_lo/b_hi under allocator 0, the candidate index under allocator 1):
 * allocation tile u of the tensor covers quantization tiles u*kA ... u*kA + kA - 1. */
static int entropy_and_widths(const void* x, int dtype, const tahref_plan* pl, const tahref_params* p, float* H,
                              uint8_t* hi) {
  float* a = (float*)malloc(sizeof(float) * (size_t)pl->A);
  uint8_t* hiA = (uint8_t*)malloc((size_t)(pl->atiles + 1));
  if (!a || !hiA) {
    free(a);
    free(hiA);
    return TAHREF_ERR_INVALID_ARG;
  }
  for (int64_t u = 0; u < pl->atiles; ++u) {
    for (int64_t g = 0; g < pl->kA; ++g) load_tile(x, dtype, pl, u * pl->kA + g, a + g * pl->G);
    H[u] = tahref_alloc_entropy(a, (int)pl->A, pl->G);
  }
  int rc = TAHREF_OK;
  for (int64_t s = 0; s < pl->nsamples && rc == TAHREF_OK; ++s) {
    int64_t first = s * pl->atiles_per_sample;
    if (pl->allocator == 0)
      rc = tahref_allocate(H + first, pl->atiles_per_sample, pl->k, hiA + first);
    else
      rc = tahref_allocate_greedy(H + first, pl->atiles_per_sample, p->n_candidates, p->candidates, pl->R,
                                  hiA + first);
  }
  for (int64_t t = 0; t < pl->tiles; ++t) hi[t] = hiA[t / pl->kA];
  free(a);
  free(hiA);
  return rc;
}

/* Code width of a tile from its width index. */
static int width_of(const tahref_plan* pl, const tahref_params* p, int idx) {
  if (pl->allocator == 0) return idx ? pl->b_hi : pl->b_lo;
  return p->candidates[idx];
}

int tahref_tile_stats(const void* x, int x_dtype, int64_t tokens, int64_t hidden, const tahref_params* p,
                      float* H, uint8_t* flag, uint8_t* pivot, uint8_t* hi, float* lo, float* scale) {
  if (x_dtype != TAHREF_F32 && x_dtype != TAHREF_BF16) return TAHREF_ERR_INVALID_ARG;
  tahref_plan pl;
  int rc = tahref_plan_make(tokens, hidden, p, &pl);
  if (rc) return rc;
  rc = entropy_and_widths(x, x_dtype, &pl, p, H, hi);
  if (rc) return rc;
  float a[128];
  uint32_t q[128];
  for (int64_t t = 0; t < pl.tiles; ++t) {
    load_tile(x, x_dtype, &pl, t, a);
    int d;
    int f = tahref_outlier(a, pl.G, p->tau, &d, NULL, NULL);
    if (f) {
      float tmp = a[0];
      a[0] = a[d];
      a[d] = tmp;
      tahref_fwht(a, pl.G);
    }
    int b = width_of(&pl, p, hi[t]);
    tahref_quantize(a, pl.G, b, &lo[t], &scale[t], q);
    flag[t] = (uint8_t)f;
    pivot[t] = (uint8_t)d;
  }
  return TAHREF_OK;
}

/*
 * Encoder (Algorithm 1, the sender's step): entropy and widths (§3.2), then per tile the
 * outlier test, pivot swap and Hadamard (§3.3), quantization, and packing of
 * codes and metadata into one fixed-size byte stream (§3.4).
 *
 * Payload (little-endian, sections start on 256-byte boundaries):
 *   header (128 B, zero padded to 256; byte 124 = allocator) | block table:
 *   u32 per run of 64 tiles, the count of b_hi tiles before it (allocator 0)
 *   or the sum of the code widths of the tiles before it (allocator 1) |
 *   width map: u32 words; allocator 0: bit t%32 of word t/32 is 1 iff tile t
 *   has b_hi (2 words per 64 tiles); allocator 1: bits 2(t%16), 2(t%16)+1 of
 *   word t/16 hold the candidate index of tile t (4 words per 64 tiles) |
 *   side byte per tile:
 *   bit 7 = transformed, bits 0..6 = pivot d of a transformed tile (0 for
 *   the others) | scale per tile: bf16 bits |
 *   zero-point per tile: fp32 | codes: one block of G*b/8 bytes per tile in
 *   tile order, code k at stream bits [k*b, k*b + b), least significant bit
 *   first (bit i of the block is bit i%8 of byte i/8). Padding bytes are zero.
 */
int tahref_encode(const void* x, int x_dtype, int64_t tokens, int64_t hidden, const tahref_params* p,
                  uint8_t* P, size_t cap) {
  if (x_dtype != TAHREF_F32 && x_dtype != TAHREF_BF16) return TAHREF_ERR_INVALID_ARG;
  tahref_plan pl;
  int rc = tahref_plan_make(tokens, hidden, p, &pl);
  if (rc) return rc;
  if (!P || (tokens > 0 && !x)) return TAHREF_ERR_INVALID_ARG;
  if ((int64_t)cap < pl.total) return TAHREF_ERR_BUFFER_TOO_SMALL;
  memset(P, 0, (size_t)pl.total);
  write_header(P, &pl, p, x_dtype);

  float* H = (float*)malloc(sizeof(float) * (size_t)(pl.tiles + 1));
  uint8_t* hi = (uint8_t*)malloc((size_t)(pl.tiles + 1));
  if (!H || !hi) {
    free(H);
    free(hi);
    return TAHREF_ERR_INVALID_ARG;
  }
  rc = entropy_and_widths(x, x_dtype, &pl, p, H, hi);
  if (rc) {
    free(H);
    free(hi);
    return rc;
  }

  float a[128];
  uint32_t q[128];
  int64_t code_off = pl.off_codes;
  int64_t hi_count = 0, width_sum = 0;
  for (int64_t t = 0; t < pl.tiles; ++t) {
    if (t % 64 == 0)
      put_u32(P, pl.off_table + 4 * (t / 64), (uint32_t)(pl.allocator == 0 ? hi_count : width_sum));
    if (pl.allocator == 0 && hi[t]) {
      int64_t w = pl.off_bitmap + 4 * (t / 32);
      put_u32(P, w, get_u32(P, w) | (1u << (t % 32)));
      ++hi_count;
    }
    if (pl.allocator == 1) {
      int64_t w = pl.off_bitmap + 4 * (t / 16);
      put_u32(P, w, get_u32(P, w) | ((uint32_t)hi[t] << (2 * (t % 16))));
    }
    load_tile(x, x_dtype, &pl, t, a);
    int d;
    int f = tahref_outlier(a, pl.G, p->tau, &d, NULL, NULL);
    if (f) {
      float tmp = a[0];
      a[0] = a[d];
      a[d] = tmp;
      tahref_fwht(a, pl.G);
    }
    int b = width_of(&pl, p, hi[t]);
    width_sum += b;
    float lo, s;
    tahref_quantize(a, pl.G, b, &lo, &s, q);
    put_u8(P, pl.off_side + t, (uint32_t)(f ? (0x80 | d) : 0)); /* the pivot only matters to a transformed tile */
    put_u16(P, pl.off_scale + 2 * t, f2u(s) >> 16);
    put_u32(P, pl.off_zero + 4 * t, f2u(lo));
    for (int k = 0; k < pl.G; ++k)
      for (int i = 0; i < b; ++i) {
        int64_t bit = (int64_t)k * b + i;
        if ((q[k] >> i) & 1u) P[code_off + bit / 8] |= (uint8_t)(1u << (bit % 8));
      }
    code_off += (int64_t)pl.G * b / 8;
  }
  free(H);
  free(hi);
  return TAHREF_OK;
}

/*
 * Decoder (Algorithm 1, the receiver's step). The shape and parameters come from the caller
 * (pipeline stages know them statically); the header must agree with them.
 * Code blocks are located by a running sum over the width map in tile order;
 * the block table is checked against that sum, and so is the allocation: k
 * b_hi allocation tiles per sample (allocator 0), or candidate indexes in
 * range, equal across an allocation tile, whose widths above c_1 add up to at
 * most R per sample (allocator 1).
 */
int tahref_decode(const uint8_t* P, size_t len, int64_t tokens, int64_t hidden, const tahref_params* p,
                  void* y, int y_dtype) {
  if (y_dtype != TAHREF_F32 && y_dtype != TAHREF_BF16) return TAHREF_ERR_INVALID_ARG;
  tahref_plan pl;
  int rc = tahref_plan_make(tokens, hidden, p, &pl);
  if (rc) return rc;
  if (!P || (tokens > 0 && !y)) return TAHREF_ERR_INVALID_ARG;
  if ((int64_t)len < pl.total) return TAHREF_ERR_BUFFER_TOO_SMALL;
  uint8_t expect[256];
  write_header(expect, &pl, p, P[6]);
  if (P[6] > 1 || memcmp(expect, P, 256) != 0) return TAHREF_ERR_BAD_PAYLOAD;

  float xhat[128];
  uint32_t q[128];
  int64_t code_off = pl.off_codes;
  int64_t hi_count = 0, width_sum = 0, extra = 0;
  int prev_idx = 0;
  for (int64_t t = 0; t < pl.tiles; ++t) {
    if (t % 64 == 0 &&
        get_u32(P, pl.off_table + 4 * (t / 64)) != (uint32_t)(pl.allocator == 0 ? hi_count : width_sum))
      return TAHREF_ERR_BAD_PAYLOAD;
    int idx;
    if (pl.allocator == 0) {
      idx = (get_u32(P, pl.off_bitmap + 4 * (t / 32)) >> (t % 32)) & 1u;
      hi_count += idx;
    } else {
      idx = (get_u32(P, pl.off_bitmap + 4 * (t / 16)) >> (2 * (t % 16))) & 3u;
      if (idx >= p->n_candidates) return TAHREF_ERR_BAD_PAYLOAD;
      if (t % pl.kA != 0 && idx != prev_idx) return TAHREF_ERR_BAD_PAYLOAD; /* one width per allocation tile */
      if (t % pl.tiles_per_sample == 0) extra = 0;
      if (t % pl.kA == 0) extra += p->candidates[idx] - p->candidates[0];
      if (extra > pl.R) return TAHREF_ERR_BAD_PAYLOAD;
      prev_idx = idx;
    }
    int b = width_of(&pl, p, idx);
    width_sum += b;
    uint32_t side = P[pl.off_side + t];
    int f = (side >> 7) & 1, d = side & 0x7f;
    if (d >= pl.G) return TAHREF_ERR_BAD_PAYLOAD;
    float s = bf16_to_f32((uint16_t)get_u16(P, pl.off_scale + 2 * t));
    float lo = u2f(get_u32(P, pl.off_zero + 4 * t));
    for (int k = 0; k < pl.G; ++k) {
      q[k] = 0;
      for (int i = 0; i < b; ++i) {
        int64_t bit = (int64_t)k * b + i;
        q[k] |= (uint32_t)((P[code_off + bit / 8] >> (bit % 8)) & 1u) << i;
      }
    }
    code_off += (int64_t)pl.G * b / 8;
    tahref_dequantize(q, pl.G, s, lo, f, d, xhat);
    int64_t row = t / pl.M, m = t % pl.M;
    int64_t base = row * pl.hidden + m * pl.G;
    if (y_dtype == TAHREF_F32) {
      float* yf = (float*)y;
      for (int k = 0; k < pl.G; ++k) yf[base + k] = xhat[k];
    } else {
      uint16_t* yh = (uint16_t*)y;
      for (int k = 0; k < pl.G; ++k) yh[base + k] = f32_to_bf16_rne(xhat[k]);
    }
  }
  if (pl.allocator == 0 && hi_count != pl.k * pl.kA * pl.nsamples) return TAHREF_ERR_BAD_PAYLOAD;
  return TAHREF_OK;
}

/* ------------------------------------------------------------------ */
/* backward compressor Q_Naive (Algorithm 1 backward, App. H Eq. 24) */
/* ------------------------------------------------------------------ */

static int naive_args_ok(int64_t n, int bits, float c) {
  return n >= 0 && bits >= 2 && bits <= 16 && c > 0.0f && isfinite(c) && isfinite(ldexpf(c, bits - 1));
}

int tahref_naive_payload_bytes(int64_t n, int bits, size_t* out) {
  if (n < 0 || bits < 2 || bits > 16 || !out) return TAHREF_ERR_INVALID_ARG;
  const int64_t groups = (n + 31) / 32; /* 32 codes of b bits fill b whole 32-bit words */
  *out = (size_t)align256(256 + groups * 4 * bits);
  return TAHREF_OK;
}

/*
 * q = clamp(round_half_even(g * c * 2^(b-1)), -2^(b-1), 2^(b-1) - 1).
 * c * 2^(b-1) is exact (a power-of-two scaling), so the product g * c_q is the
 * one fp32 rounding before the integer rounding, the same as rounding c * g
 * and scaling it by 2^(b-1).
 */
int tahref_naive_quantize(float g, int bits, float c, int32_t* q) {
  if (!naive_args_ok(1, bits, c) || !q) return TAHREF_ERR_INVALID_ARG;
  const float cq = ldexpf(c, bits - 1);
  const float y = g * cq;
  const float lo = -ldexpf(1.0f, bits - 1), hi = ldexpf(1.0f, bits - 1) - 1.0f;
  float r = nearbyintf(y); /* the default rounding mode: half to even */
  if (!(r >= lo)) r = lo;  /* also catches NaN */
  if (r > hi) r = hi;
  *q = (int32_t)r;
  return TAHREF_OK;
}

/* g_hat = Q(c g) / c = (q 2^-(b-1)) / c = q / (c 2^(b-1)): one fp32 division of exact operands. */
float tahref_naive_dequantize(int32_t q, int bits, float c) {
  const float cq = ldexpf(c, bits - 1);
  return (float)q / cq;
}

static void naive_header(uint8_t* P, int64_t n, int bits, float c, int dtype, int64_t total) {
  memset(P, 0, 256);
  put_u32(P, 0, 0x4E484154u); /* "TAHN" */
  put_u16(P, 4, 1);
  put_u8(P, 6, (uint32_t)dtype);
  put_u8(P, 7, (uint32_t)bits);
  put_u64(P, 8, (uint64_t)n);
  put_u32(P, 16, f2u(c));
  put_u64(P, 24, (uint64_t)total);
}

int tahref_naive_encode(const void* g, int g_dtype, int64_t n, int bits, float c, uint8_t* P, size_t cap) {
  if (!naive_args_ok(n, bits, c) || (g_dtype != TAHREF_F32 && g_dtype != TAHREF_BF16) || !P || (n > 0 && !g))
    return TAHREF_ERR_INVALID_ARG;
  size_t total;
  tahref_naive_payload_bytes(n, bits, &total);
  if (cap < total) return TAHREF_ERR_BUFFER_TOO_SMALL;
  memset(P, 0, total);
  naive_header(P, n, bits, c, g_dtype, (int64_t)total);
  const uint32_t mask = (bits == 32) ? 0xffffffffu : ((1u << bits) - 1u);
  for (int64_t i = 0; i < n; ++i) {
    const float gi = g_dtype == TAHREF_F32 ? ((const float*)g)[i] : bf16_to_f32(((const uint16_t*)g)[i]);
    int32_t q;
    tahref_naive_quantize(gi, bits, c, &q);
    const uint32_t code = (uint32_t)q & mask;
    for (int k = 0; k < bits; ++k) { /* bit by bit, least significant first */
      const int64_t bit = i * bits + k;
      if ((code >> k) & 1u) P[256 + bit / 8] |= (uint8_t)(1u << (bit % 8));
    }
  }
  return TAHREF_OK;
}

int tahref_naive_decode(const uint8_t* P, size_t len, int64_t n, int bits, float c, void* y, int y_dtype) {
  if (!naive_args_ok(n, bits, c) || (y_dtype != TAHREF_F32 && y_dtype != TAHREF_BF16) || !P || (n > 0 && !y))
    return TAHREF_ERR_INVALID_ARG;
  size_t total;
  tahref_naive_payload_bytes(n, bits, &total);
  if (len < total) return TAHREF_ERR_BUFFER_TOO_SMALL;
  if (get_u32(P, 0) != 0x4E484154u || get_u16(P, 4) != 1 || P[7] != (uint8_t)bits ||
      (uint64_t)get_u32(P, 8) + ((uint64_t)get_u32(P, 12) << 32) != (uint64_t)n || get_u32(P, 16) != f2u(c) ||
      (uint64_t)get_u32(P, 24) + ((uint64_t)get_u32(P, 28) << 32) != (uint64_t)total)
    return TAHREF_ERR_BAD_PAYLOAD;
  for (int64_t i = 0; i < n; ++i) {
    uint32_t code = 0;
    for (int k = 0; k < bits; ++k) {
      const int64_t bit = i * bits + k;
      code |= (uint32_t)((P[256 + bit / 8] >> (bit % 8)) & 1u) << k;
    }
    const int32_t q = (code >> (bits - 1)) & 1u ? (int32_t)code - (int32_t)(1u << bits) : (int32_t)code;
    const float v = tahref_naive_dequantize(q, bits, c);
    if (y_dtype == TAHREF_F32) ((float*)y)[i] = v;
    else ((uint16_t*)y)[i] = f32_to_bf16_rne(v);
  }
  return TAHREF_OK;
}
