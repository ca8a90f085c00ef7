/*
 * tah.h — C ABI of the MI355X (gfx950) TAH-Quant activation codec.
 *
 * TAH-Quant (Tile-wise Adaptive Hadamard Quantization) compresses the
 * activation tensor that one pipeline stage sends to the next:
 *   "TAH-Quant: Effective Activation Quantization in Pipeline Parallelism over
 *    Slow Network" (arXiv 2506.01352v2), Sections 3.1-3.5 and Algorithm 1.
 * The sender runs tah_encode (Algorithm 1, the sender's quantization step),
 * the receiver tah_decode (its dequantization step); tah_roundtrip does both
 * in one pass over the tensor.
 *
 * Tensor view: x and y are row-major [tokens, hidden], tokens = B * S
 * (micro-batch times sequence), hidden = C channels (§3.1). Each token's
 * channels split into tiles of G contiguous channels; tile t covers row
 * t / (hidden / G), channels (t % (hidden / G)) * G ... + G - 1.
 *
 * Conventions for every call:
 *   - x, y, payload and ws are DEVICE pointers (HIP), 16-byte aligned, owned by
 *     the caller, who keeps them alive until the stream has completed the work.
 *     The library allocates and frees nothing and keeps no pointer after return.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream). Work is
 *     enqueued asynchronously; no call synchronizes except
 *     tah_read_device_status.
 *   - Arguments are validated on the host before anything is enqueued; an
 *     invalid call returns a status other than TAH_OK and enqueues nothing.
 *     A failed kernel launch returns TAH_ERR_HIP.
 *   - Non-finite inputs, and inputs with G * max|x| at or above FLT_MAX, give
 *     undefined (but finite-time, in-bounds) results.
 *   - Calls that share one workspace must not run concurrently.
 */
#ifndef TAH_H
#define TAH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TAH_ABI_VERSION 4

typedef enum { TAH_DTYPE_F32 = 0, TAH_DTYPE_BF16 = 1 } tah_dtype_t;

typedef enum {
  TAH_OK = 0,
  TAH_ERR_INVALID_ARG = 1,       /* bad shape, pointer or parameter */
  TAH_ERR_UNSUPPORTED = 2,       /* valid for the format, not built for the GPU (tile not 32/64/128) */
  TAH_ERR_BUFFER_TOO_SMALL = 3,  /* payload_cap / ws_cap / payload_len below the required size */
  TAH_ERR_BUDGET_INFEASIBLE = 4, /* bit_budget below the smallest candidate width */
  TAH_ERR_BAD_PAYLOAD = 5,       /* payload header disagrees with shape/params (device status word) */
  TAH_ERR_HIP = 6,               /* a HIP runtime call or kernel launch failed */
  TAH_ERR_SCRATCH_LIMIT = 7      /* tah_roundtrip_noalloc: the shape needs more than TAH_NOALLOC_SCRATCH_BYTES */
} tah_status_t;

/*
 * Codec parameters.
 *   tile: G, the quantization tile (§3.1). A power of two dividing hidden;
 *     the GPU kernels are built for 32, 64 and 128 (the format allows 8..128).
 *   tokens_per_sample: S, the ranking scope of the top-p% selection (§3.2:
 *     tiles are ranked within each sample); 0 = all tokens form one sample.
 *     tokens % S must be 0.
 *   bit_budget: average code bits per element of each sample, metadata
 *     excluded. The two candidates around it, b_lo <= budget < b_hi, are used:
 *     the k = floor((budget - b_lo) * N / (b_hi - b_lo)) highest-entropy
 *     allocation tiles of a sample (N = S * hidden / A of them) get b_hi, the
 *     rest b_lo (§3.2, INT4 for the top p%, INT3 for the rest). Equal entropies
 *     rank the lower allocation-tile index first. The budget is read as the
 *     decimal it stands for: the shortest decimal that rounds to the given
 *     fp32 value (3.8f, held as 3.79999995, is 3.8, so 80% of N tiles get b_hi
 *     whenever 0.8 N is an integer); k is computed from it exactly.
 *   n_candidates, candidates: 1..4 widths, strictly increasing, each 1..8.
 *   tau: outlier threshold of Eq. (3) (§3.3, default 2.0); 0 transforms every
 *     non-zero tile, +INFINITY none (Appendix F). Must be >= 0 and not NaN.
 *   alloc_tile: A, the allocation tile of the bit allocation in channels (§3.2
 *     "Tile decomposition"): a multiple of G that divides hidden; 0 means A = G
 *     (the paper's default), A = hidden is token-level allocation. Its entropy
 *     (Eq. 1-2 over all A channels) adds the per-quantization-tile sums
 *     L = sum |a| and S = sum |a| log2 |a| left to right; each quantization
 *     tile takes the width of its allocation tile.
 *   allocator: TAH_ALLOC_TOP_P (0, the paper's rule above) or
 *     TAH_ALLOC_GREEDY (1): every candidate width may occur in a sample. The
 *     paper gives no rule for more than two widths; this one reads its entropy
 *     ranking as a distortion budget. Tile u weighs 2^(2 H_u); upgrade j of a
 *     tile (c_j -> c_(j+1), costing c_(j+1) - c_j bits) has the key
 *       kappa = 2 H_u + lambda_j (fp32),
 *       lambda_j = log2((Delta(c_j) - Delta(c_(j+1))) / (c_(j+1) - c_j)),
 *       Delta(b) = (2^b - 1)^-2,
 *     the log2 of its gain per bit; starting from c_1 everywhere, upgrades are
 *     taken in the order kappa descending, then tile index, then j, while the
 *     bits they add stay within R = floor((budget - c_1) * N) per sample; the
 *     first that does not fit ends the allocation. With two candidates this
 *     is the top-p% rule. Limits: tokens * hidden / tile * c_n below 2^32
 *     (else TAH_ERR_INVALID_ARG) and (c_n - c_1) * N below 2^32 (else
 *     TAH_ERR_UNSUPPORTED).
 */
#define TAH_ALLOC_TOP_P 0
#define TAH_ALLOC_GREEDY 1
typedef struct {
  int32_t tile;
  int32_t tokens_per_sample;
  float bit_budget;
  int32_t n_candidates;
  uint8_t candidates[4];
  float tau;
  int32_t alloc_tile;
  int32_t allocator;
} tah_params_t;

/* Fills the paper's defaults (§5.1): G = A = 64, 80% INT4 + 20% INT3
 * (budget 3.8 over {3, 4}), tau = 2, one sample. */
void tah_params_default(tah_params_t* p);

/*
 * Size in bytes of the payload for this shape and parameters. The payload is a
 * fixed-shape uint8 stream (§3.4): its size depends only on (tokens, hidden,
 * params), never on the values. Layout (little-endian, sections on 256-byte
 * boundaries): 128-byte header (magic "TAHQ", version 2, shape, params,
 * section offsets, allocation tile A as u32 at byte 120, allocator at byte
 * 124) | block table, u32 per run of 64 tiles: the count of b_hi tiles before
 * it (top-p%) or the sum of the code widths of the tiles before it (greedy) |
 * width map, one bit per quantization tile (1 = b_hi; top-p%) or two bits,
 * the candidate index, at bits 2(t%16) of word t/16 (greedy); an allocation
 * tile's entries are equal | side byte per tile (bit 7: Hadamard applied,
 * bits 0-6: pivot index of a transformed tile, 0 otherwise) | bf16 scale per tile | fp32 zero-point per tile |
 * code blocks of G*b/8 bytes in tile order, codes least-significant-bit first.
 * Under the greedy allocator the code section is sized for the whole budget
 * and its unused tail is zero.
 */
tah_status_t tah_payload_bytes(int64_t tokens, int64_t hidden, const tah_params_t* p, size_t* out);

/*
 * tah_roundtrip without a workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation): the same kernels and the same results as tah_roundtrip
 * (every argument has the same meaning), with the library's own scratch in
 * place of ws. That scratch is a file-scope device array of
 * TAH_NOALLOC_SCRATCH_BYTES on each GPU the library runs on, created with the
 * library's code object and held until the process ends; its address on a
 * device is looked up once, at the first call with that device current. No
 * call allocates or frees anything.
 *   - A shape whose workspace (tah_workspace_bytes) exceeds
 *     TAH_NOALLOC_SCRATCH_BYTES returns TAH_ERR_SCRATCH_LIMIT and enqueues
 *     nothing (32 MiB holds about six million tiles of any allocation, e.g.
 *     every 8192 x 8192 and 16384 x 5120 setting).
 *   - Every call on one GPU shares that GPU's scratch, and each call rewrites
 *     what it reads there before reading it (nothing needs to start at zero).
 *     Calls that overlap on one GPU (concurrent streams, or threads) race on
 *     it and give undefined results: serialize them.
 */
#define TAH_NOALLOC_SCRATCH_BYTES (32u << 20)
tah_status_t tah_roundtrip_noalloc(const void* x, tah_dtype_t x_dtype, int64_t tokens, int64_t hidden,
                                   const tah_params_t* p, void* payload, size_t payload_cap, void* y,
                                   tah_dtype_t y_dtype, void* stream);

/* Size in bytes of the device workspace the calls below need for this shape
 * (per-tile entropies, selection state and histograms, the tie candidates of
 * the selection, width map and block table when no payload is written, under
 * the greedy allocator the used width total, the device status word). Every
 * call rewrites what it reads there, so the contents between calls do not
 * matter. */
tah_status_t tah_workspace_bytes(int64_t tokens, int64_t hidden, const tah_params_t* p, size_t* out);

/*
 * Encode x [tokens, hidden] (x_dtype) into payload (payload_cap bytes, at least
 * tah_payload_bytes). Per tile: entropy (Eq. 1-2), width by per-sample ranking
 * (§3.2), outlier test (Eq. 3), pivot swap and Hadamard (Eq. 4) on flagged
 * tiles, asymmetric quantization, packing (§3.4). Per-tile entropies are left
 * in the workspace (tah_workspace_entropy gives their offset).
 */
tah_status_t tah_encode(const void* x, tah_dtype_t x_dtype, int64_t tokens, int64_t hidden, const tah_params_t* p,
                        void* payload, size_t payload_cap, void* ws, size_t ws_cap, void* stream);

/*
 * Decode payload (payload_len bytes) into y [tokens, hidden] (y_dtype; bf16 is
 * rounded to nearest even) — Algorithm 1, the receiver's step: unpack, dequantize, apply
 * H^T / G and undo the pivot swap on flagged tiles. The shape and params must
 * be those of the encode: the device checks the payload header against them
 * and, on a mismatch, writes TAH_ERR_BAD_PAYLOAD to the workspace status word
 * and leaves y untouched (read it with tah_read_device_status).
 */
tah_status_t tah_decode(const void* payload, size_t payload_len, int64_t tokens, int64_t hidden, const tah_params_t* p,
                        void* y, tah_dtype_t y_dtype, void* ws, size_t ws_cap, void* stream);

/*
 * Encode and decode in one pass: y receives exactly what tah_decode would
 * produce from the payload tah_encode writes. payload may be NULL (then
 * payload_cap is ignored and nothing is written to it).
 */
tah_status_t tah_roundtrip(const void* x, tah_dtype_t x_dtype, int64_t tokens, int64_t hidden, const tah_params_t* p,
                           void* payload, size_t payload_cap, void* y, tah_dtype_t y_dtype, void* ws, size_t ws_cap,
                           void* stream);

/*
 * Allocation-tile entropy only (Eq. 1-2, §3.2): h[u] for each of the
 * tokens*hidden/A allocation tiles (A = G unless alloc_tile says otherwise),
 * fp32, device pointer. Needs the same workspace as tah_encode.
 */
tah_status_t tah_tile_entropy(const void* x, tah_dtype_t x_dtype, int64_t tokens, int64_t hidden,
                              const tah_params_t* p, float* h, void* ws, size_t ws_cap, void* stream);

/* Byte offset inside the workspace of the fp32 allocation-tile entropies
 * (tokens*hidden/A of them) written by tah_encode and tah_roundtrip. */
tah_status_t tah_workspace_entropy(int64_t tokens, int64_t hidden, const tah_params_t* p, size_t* offset);

/*
 * Backward compressor for the activation gradients that the next stage sends
 * back (Algorithm 1, the backward pass: a simple fixed-point compressor, §3.5), with
 * the scaling of Appendix H, Eq. (24): g_hat = Q(c g) / c. Q is b-bit signed
 * fixed point with b-1 fractional bits, round half to even, saturating:
 *   q = clamp(rne(g * c * 2^(b-1)), -2^(b-1), 2^(b-1) - 1),  g_hat = q / (c * 2^(b-1)).
 * n elements of a contiguous fp32 or bf16 tensor (any shape, row-major).
 * bits: 2..16; c: positive and finite, with c * 2^(b-1) finite.
 * Payload layout (little-endian): bytes 0-3 "TAHN", 4-5 version 1, 6 input
 * dtype, 7 bits, 8-15 n, 16-19 c (fp32), 24-31 total bytes, zero to byte 255;
 * then the codes as b-bit two's complement, code i at stream bits
 * [i b, i b + b), least significant bit first; zero padding to a whole number
 * of 32-code groups (b 32-bit words each) and to a multiple of 256 bytes.
 */
tah_status_t tah_naive_payload_bytes(int64_t n, int bits, size_t* out);

/* Quantize g (n elements, g_dtype) into payload (payload_cap bytes, at least
 * tah_naive_payload_bytes). */
tah_status_t tah_naive_encode(const void* g, tah_dtype_t g_dtype, int64_t n, int bits, float c, void* payload,
                              size_t payload_cap, void* stream);

/* Dequantize payload into y (n elements, y_dtype; bf16 rounded to nearest
 * even). ws (at least 256 bytes) receives the device status word: the header
 * is checked against n, bits and c (the input-dtype byte is not), and on a
 * mismatch the word is TAH_ERR_BAD_PAYLOAD and y is left untouched. */
tah_status_t tah_naive_decode(const void* payload, size_t payload_len, int64_t n, int bits, float c, void* y,
                              tah_dtype_t y_dtype, void* ws, size_t ws_cap, void* stream);

/*
 * The tile-local Hadamard transform of Eq. (4) alone (§3.3), unnormalized:
 * y_t = H_G x_t for each of n_tiles contiguous tiles of `tile` elements
 * (x: fp32 or bf16, row-major [n_tiles, tile]; y: fp32, same layout; both
 * device pointers, 16-byte aligned, owned by the caller; no pivot swap).
 * H_G is the Sylvester matrix, H[i][j] = (-1)^popcount(i & j).
 * method TAH_HADAMARD_BUTTERFLY: the fast Walsh-Hadamard butterfly the codec
 *   runs (stages of stride 1, 2, 4, ... in fp32), so its results are the
 *   codec's transform bit for bit; tile 32, 64 or 128.
 * method TAH_HADAMARD_MFMA: the same product as a dense matrix multiply on
 *   the matrix cores (the O(G^2) form §3.4 prices); each entry is the exact
 *   fp32 sum of G exact products, added in the hardware's order, so it may
 *   differ from the butterfly's in the last bits. Only tile 64 with bf16
 *   input (else TAH_ERR_UNSUPPORTED).
 * The codec never calls this; it exists to compare the two forms.
 */
#define TAH_HADAMARD_BUTTERFLY 0
#define TAH_HADAMARD_MFMA 1
tah_status_t tah_hadamard(const void* x, tah_dtype_t x_dtype, int64_t n_tiles, int tile, int method, float* y,
                          void* stream);

/* Waits for `stream`, then copies the device status word of the last
 * tah_decode or tah_naive_decode on this workspace into *out (TAH_OK or
 * TAH_ERR_BAD_PAYLOAD). */
tah_status_t tah_read_device_status(const void* ws, void* stream, int32_t* out);

const char* tah_status_string(tah_status_t s);
int tah_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* TAH_H */
