/*
 * TAH-Quant reference oracle — TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, single-threaded CPU implementation of the TAH-Quant activation
 * codec (Tile-wise Adaptive Hadamard Quantization), written from
 *   "TAH-Quant: Effective Activation Quantization in Pipeline Parallelism over
 *    Slow Network" (arXiv 2506.01352v2), Sections 3.1-3.5, Eq. (1)-(4),
 *    Algorithm 1 and Appendix F.
 * It exists so that tests, the smoke check and the benchmark's CPU baseline can
 * check the GPU library against it. Nothing in the product path may include,
 * link or call this code, and it shares no code, header or table with the GPU
 * library: the payload format, the fp32 operation order and the log2 tables
 * are restated here independently from the written specification.
 *
 * Precision: every quantity that decides an integer (entropy ranking, outlier
 * flag, pivot, codes) is computed in IEEE fp32 in a fixed, documented
 * operation order, because that is the precision the GPU kernels decide in.
 * The pins in tests/ check these fp32 routines against fp64 / closed forms.
 */
#ifndef TAH_REF_H
#define TAH_REF_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { TAHREF_F32 = 0, TAHREF_BF16 = 1 };

enum {
  TAHREF_OK = 0,
  TAHREF_ERR_INVALID_ARG = 1,
  TAHREF_ERR_UNSUPPORTED = 2,
  TAHREF_ERR_BUFFER_TOO_SMALL = 3,
  TAHREF_ERR_BUDGET_INFEASIBLE = 4,
  TAHREF_ERR_BAD_PAYLOAD = 5
};

/* Codec parameters (paper notation in brackets). */
typedef struct {
  int32_t tile;              /* G: quantization tile (§3.1) */
  int32_t tokens_per_sample; /* S: ranking scope of the top-p% selection; 0 = all tokens (§3.2) */
  float bit_budget;          /* average code bits per element per sample, metadata excluded */
  int32_t n_candidates;      /* number of candidate widths, 1..4 */
  uint8_t candidates[4];     /* strictly increasing, each 1..8 */
  float tau;                 /* outlier threshold tau of Eq. (3); 0 = always, +inf = never (App. F) */
  int32_t alloc_tile;        /* A: allocation tile (§3.2), a multiple of G dividing hidden; 0 = G */
  int32_t allocator;         /* 0: top-p% between the two widths around the budget (§3.2);
                                1: greedy over every candidate width (see tahref_allocate_greedy) */
} tahref_params;

/* Derived sizes and the payload section layout. */
typedef struct {
  int64_t tokens, hidden, S, nsamples, M, tiles, tiles_per_sample, nblocks;
  int32_t G, log2G, b_lo, b_hi;
  int64_t k; /* allocation tiles per sample that get b_hi */
  int64_t off_table, off_bitmap, off_side, off_scale, off_zero, off_codes, code_bytes, total;
  /* allocation tiles (§3.2): A channels = kA quantization tiles; MA = hidden / A per
   * token (the paper's M); atiles in all, atiles_per_sample = S * MA per sample */
  int64_t A, kA, MA, atiles, atiles_per_sample;
  /* allocator 1: R bounds the sum over a sample's allocation tiles of their width
   * minus c_1 (see tahref_allocate_greedy) */
  int64_t allocator, R;
} tahref_plan;

int tahref_plan_make(int64_t tokens, int64_t hidden, const tahref_params* p, tahref_plan* out);

/* Building blocks, exported so the pins can test each one alone. */
float tahref_log2s(float u);
void tahref_fwht(float* v, int G);
float tahref_entropy(const float* alpha, int G);
float tahref_alloc_entropy(const float* alpha, int A, int G);
int tahref_outlier(const float* alpha, int G, float tau, int* d, float* m1, float* m2);
void tahref_quantize(const float* y, int G, int b, float* lo, float* s, uint32_t* q);
void tahref_dequantize(const uint32_t* q, int G, float s, float lo, int flag, int d, float* xhat);
int tahref_allocate(const float* H, int64_t N, int64_t k, uint8_t* hi);
/* Greedy allocation over n candidate widths (allocator 1): lam receives the n-1
 * per-upgrade constants, level[u] the index of tile u's width. */
int tahref_greedy_lambda(int n, const uint8_t* cand, float* lam);
int tahref_allocate_greedy(const float* H, int64_t N, int n, const uint8_t* cand, int64_t R, uint8_t* level);

/* Whole codec over a [tokens, hidden] row-major tensor (host pointers). */
int tahref_encode(const void* x, int x_dtype, int64_t tokens, int64_t hidden, const tahref_params* p,
                  uint8_t* payload, size_t payload_cap);
int tahref_decode(const uint8_t* payload, size_t payload_len, int64_t tokens, int64_t hidden,
                  const tahref_params* p, void* y, int y_dtype);
/* H: one entropy per allocation tile (atiles); the other outputs one per quantization tile
 * (hi: 0/1 for b_lo/b_hi under allocator 0, the candidate index under allocator 1). */
int tahref_tile_stats(const void* x, int x_dtype, int64_t tokens, int64_t hidden, const tahref_params* p,
                      float* H, uint8_t* flag, uint8_t* pivot, uint8_t* hi, float* lo, float* scale);

/*
 * Backward compressor Q_Naive for the activation gradients that travel back
 * across the stage boundary (Algorithm 1, backward pass; §3.5 calls it a simple
 * fixed-point compressor of 6-8 bits) with the scaling of Appendix H,
 * Eq. (24): g_hat = Q(c g) / c. Reading: Q is b-bit signed fixed point with
 * b-1 fractional bits (values k 2^-(b-1), k in [-2^(b-1), 2^(b-1)-1]),
 * round half to even, saturating; c is a positive constant.
 * Payload: 256-byte header region (magic "TAHN", version, input dtype, b, n,
 * c, total), then the n codes as b-bit two's complement, code i at stream
 * bits [i b, i b + b), least significant bit first, zero padded to a whole
 * number of 32-code groups and to 256 bytes.
 */
int tahref_naive_payload_bytes(int64_t n, int bits, size_t* out);
int tahref_naive_quantize(float g, int bits, float c, int32_t* q);
float tahref_naive_dequantize(int32_t q, int bits, float c);
int tahref_naive_encode(const void* g, int g_dtype, int64_t n, int bits, float c, uint8_t* payload,
                        size_t payload_cap);
int tahref_naive_decode(const uint8_t* payload, size_t payload_len, int64_t n, int bits, float c, void* y,
                        int y_dtype);

#ifdef __cplusplus
}
#endif
#endif
