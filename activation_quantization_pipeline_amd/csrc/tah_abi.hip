// Host side of the C ABI (include/tah.h): argument validation, the per-call
// plan (width pair and k of §3.2, payload layout of §3.4, workspace layout) and
// the launch sequence. Validation happens before anything is enqueued.
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "tah_internal.hpp"

namespace tah {

static int64_t align256(int64_t v) { return (v + 255) & ~(int64_t)255; }

static int ilog2(int v) {
  int l = 0;
  while ((1 << l) < v) ++l;
  return l;
}

// The bit budget as the decimal it stands for: the pages give the split as a
// percentage (80% INT4 / 20% INT3, TAH-Quant §3.2 and §5.1), a budget of 3.8
// bits that fp32 holds as 3.79999995, which would make floor(p N) one short
// whenever 0.8 N is an integer. The budget is read as the decimal with the
// fewest fractional digits that rounds to the given fp32 value (the nearest
// one, ties to even): num / den, den = 10^digits. B * 10^digits is exact in
// double (24 + 21 significant bits), so rint rounds the exact product.
static void budget_as_decimal(float B, int64_t* num, int64_t* den) {
  double scale = 1.0;
  for (int digits = 0; digits <= 9; ++digits, scale *= 10.0) {
    const double m = rint((double)B * scale);
    char s[48];
    snprintf(s, sizeof s, "%.0fe-%d", m, digits);
    if (strtof(s, nullptr) == B) {
      *num = (int64_t)m;
      *den = (int64_t)scale;
      return;
    }
  }
  *num = (int64_t)rint((double)B * 1e9);
  *den = 1000000000;
}

// floor((B - base) N / step) for the decimal budget B >= base, in integers.
static int64_t budget_floor(float B, int base, int64_t N, int step) {
  int64_t num = 0, den = 1;
  budget_as_decimal(B, &num, &den);
  const __int128 above = (__int128)num - (__int128)base * den;
  return (int64_t)(above * (__int128)N / ((__int128)step * den));
}

static int bit_width(uint64_t v) {
  int b = 0;
  while (v) {
    ++b;
    v >>= 1;
  }
  return b;
}

// Shape and parameter checks, width pair, k and all offsets.
static tah_status_t make_plan(int64_t tokens, int64_t hidden, const tah_params_t* p, Plan* o) {
  if (!p || !o) return TAH_ERR_INVALID_ARG;
  memset(o, 0, sizeof(*o));
  if (tokens < 0 || hidden <= 0) return TAH_ERR_INVALID_ARG;
  const int G = p->tile;
  if (G < 8 || G > 128 || (G & (G - 1)) || hidden % G) return TAH_ERR_INVALID_ARG;
  if (p->n_candidates < 1 || p->n_candidates > 4) return TAH_ERR_INVALID_ARG;
  for (int i = 0; i < p->n_candidates; ++i) {
    if (p->candidates[i] < 1 || p->candidates[i] > 8) return TAH_ERR_INVALID_ARG;
    if (i > 0 && p->candidates[i] <= p->candidates[i - 1]) return TAH_ERR_INVALID_ARG;
  }
  if (!isfinite(p->bit_budget) || isnan(p->tau) || p->tau < 0.0f || p->tokens_per_sample < 0)
    return TAH_ERR_INVALID_ARG;
  const int64_t S = p->tokens_per_sample == 0 ? tokens : p->tokens_per_sample;
  if (S > 0 && tokens % S) return TAH_ERR_INVALID_ARG;
  const int64_t A = p->alloc_tile == 0 ? G : p->alloc_tile;
  if (A < G || A % G || hidden % A) return TAH_ERR_INVALID_ARG;
  if (p->allocator != TAH_ALLOC_TOP_P && p->allocator != TAH_ALLOC_GREEDY) return TAH_ERR_INVALID_ARG;
  if ((float)p->candidates[0] > p->bit_budget) return TAH_ERR_BUDGET_INFEASIBLE;
  // tile indices of a sample and block-table counts are 32-bit on the device
  const int64_t M = hidden / G;
  if (tokens > 0 && (M > ((int64_t)1 << 40) / tokens || S * M >= ((int64_t)1 << 31) ||
                     tokens * M >= ((int64_t)1 << 40)))
    return TAH_ERR_UNSUPPORTED;

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
  o->M = M;
  o->tiles = tokens * M;
  o->A = A;
  o->kA = A / G;
  o->atiles = tokens * (hidden / A);
  o->N = S * (hidden / A);
  o->G = G;
  o->log2G = ilog2(G);
  o->allocator = p->allocator;
  if (p->allocator == TAH_ALLOC_TOP_P) {
    o->b_lo = b_lo;
    o->b_hi = b_hi;
    // k = floor(p N), p = (B - b_lo) / (b_hi - b_lo) of the decimal budget B
    o->k = (b_hi == b_lo || o->N == 0) ? 0 : budget_floor(p->bit_budget, b_lo, o->N, b_hi - b_lo);
    o->mode = o->k > 0 ? 1 : 0;
  } else {
    // greedy: any candidate per allocation tile; R = floor((B - c_1) N) bits a
    // sample may add above c_1, at most what every tile at c_n would take
    const int c1 = p->candidates[0], cn = p->candidates[p->n_candidates - 1];
    o->b_lo = c1;
    o->b_hi = cn;
    o->k = 0;
    o->mode = 2;
    o->nl = p->n_candidates - 1;
    const int64_t cap = (int64_t)(cn - c1) * o->N;
    // from B = c_n on every upgrade fits; below it the decimal budget decides
    o->R = p->bit_budget >= (float)cn ? cap : budget_floor(p->bit_budget, c1, o->N, 1);
    if (o->R > cap) o->R = cap;
    // the block table's running width sums are 32-bit (a limit of the format)
    if ((uint64_t)o->tiles * (uint64_t)cn > 0xffffffffull) return TAH_ERR_INVALID_ARG;
    // per-sample weights and upgrade indexes are 32-bit on the device
    if ((uint64_t)cap > 0xffffffffull) return TAH_ERR_UNSUPPORTED;
    // every tile takes the same level when nothing or everything fits
    o->glevel = (o->nl == 0 || o->R == 0) ? 0 : (o->R == cap ? o->nl : -1);
    for (int j = 0; j < o->nl; ++j) {
      // lambda_j = log2 of upgrade j's gain per bit, Delta(b) = (2^b - 1)^-2
      const double l0 = ldexp(1.0, p->candidates[j]) - 1.0, l1 = ldexp(1.0, p->candidates[j + 1]) - 1.0;
      const double gain = 1.0 / (l0 * l0) - 1.0 / (l1 * l1);
      o->cost[j] = p->candidates[j + 1] - p->candidates[j];
      o->lam[j] = (float)log2(gain / (double)o->cost[j]);
    }
    o->ngpasses = 0;
    o->ngidx = 0;
    if (o->glevel < 0) {
      // composite = (32-bit key, ib bits of the complemented upgrade index):
      // three grid-wide digits of the key (11/11/10 bits), then the index
      // digits, top first, inside one workgroup per sample
      o->ib = bit_width((uint64_t)(o->N * o->nl - 1));
      if (o->ib < 1) o->ib = 1;
      o->gpasses[o->ngpasses++] = GPass{o->ib + 21, 11};
      o->gpasses[o->ngpasses++] = GPass{o->ib + 10, 11};
      o->gpasses[o->ngpasses++] = GPass{o->ib, 10};
      for (int hi = o->ib; hi > 0; hi -= kDigitBits) {
        const int lo = hi - kDigitBits > 0 ? hi - kDigitBits : 0;
        o->gidx[o->ngidx++] = GPass{lo, hi - lo};
      }
    }
  }
  o->tau = p->tau;
  o->budget = p->bit_budget;
  o->n_candidates = p->n_candidates;
  for (int i = 0; i < 4; ++i) o->candidates[i] = i < p->n_candidates ? p->candidates[i] : 0;
  o->nblocks = (o->tiles + 63) / 64;

  const int64_t map_bytes = (o->allocator == TAH_ALLOC_GREEDY ? 16 : 8) * o->nblocks;  // 1 or 2 bits per tile
  o->off_table = 256;
  o->off_bitmap = align256(o->off_table + 4 * o->nblocks);
  o->off_side = align256(o->off_bitmap + map_bytes);
  o->off_scale = align256(o->off_side + o->tiles);
  o->off_zero = align256(o->off_scale + 2 * o->tiles);
  o->off_codes = align256(o->off_zero + 4 * o->tiles);
  if (o->allocator == TAH_ALLOC_TOP_P) {
    const int64_t nhi = o->k * o->kA * o->nsamples;  // quantization tiles at b_hi
    o->code_bytes = (o->tiles * G * o->b_lo + nhi * G * (o->b_hi - o->b_lo)) / 8;
  } else {  // the most the code blocks can take: A/8 bytes per unit of width, c_1 N + R units per sample
    o->code_bytes = o->nsamples * (A / 8) * ((int64_t)o->b_lo * o->N + o->R);
  }
  o->total = align256(o->off_codes + o->code_bytes);

  const bool mixed = o->mode != 0;  // block table and width map built before the encoder
  const bool sel = o->mode == 1 || o->glevel < 0;  // a select runs
  int64_t w = 0;
  o->ws_status = w;
  w += 256;
  o->ws_state = w;  // two selection states per sample (ping-pong across passes)
  static_assert(sizeof(SampleState) >= sizeof(GState), "one state size serves both selects");
  w = align256(w + 2 * (int64_t)sizeof(SampleState) * (sel ? o->nsamples : 0));
  o->ws_hist = w;  // three rotating histograms per sample
  w = align256(w + 3 * 4 * kBins * (sel ? o->nsamples : 0));
  o->ws_H = w;  // entropy of each allocation tile
  w = align256(w + 4 * o->atiles);
  o->ws_LS = w;  // per-quantization-tile sums (L, S) when an allocation tile spans several
  w = align256(w + 8 * (o->kA > 1 ? o->tiles : 0));
  o->ws_blockcnt = w;
  w = align256(w + 4 * (mixed ? o->nblocks : 0));
  o->ws_table = w;
  w = align256(w + 4 * (mixed ? o->nblocks : 0));
  o->ws_bitmap = w;
  w = align256(w + (mixed ? map_bytes : 0));
  // per sample: a count, a pad word, then the (key, index) pairs whose key
  // matches the threshold's prefix after the second entropy pass (ties at the
  // threshold are broken among them)
  // (greedy: the (key, upgrade index) pairs matching the prefix after the
  // second key digit)
  const int64_t nkeys = o->mode == 2 ? o->N * o->nl : o->N;
  o->ncand = nkeys < kMaxCand ? nkeys : kMaxCand;
  o->cand_stride = 2 + 2 * o->ncand;
  o->ws_cand = w;
  w = align256(w + 4 * o->cand_stride * (sel ? o->nsamples : 0));
  o->ws_wtotal = w;  // greedy: the sum of all code widths (the used part of the code section)
  w = align256(w + (o->mode == 2 ? 4 : 0));
  o->ws_side = w;  // mixed layouts without a payload: the side bytes of the statistics pass
  w = align256(w + (mixed ? o->tiles : 0));
  // top-p% over quantization tiles in samples of whole runs, selected grid-wide
  o->fold = (o->mode == 1 && o->kA == 1 && o->N % 64 == 0 && o->N > kLdsSelect && o->N / 64 <= kFoldMaxRuns)
                ? 1 : 0;
  o->ws_total = w;

  // radix-select passes: three digits of the 32-bit entropy key, then enough
  // digits of the tile index to order tied entropies
  o->npasses = 0;
  if (o->mode == 1) {
    o->passes[o->npasses++] = SelectPass{0, 21, 11, 0};
    o->passes[o->npasses++] = SelectPass{0, 10, 11, 0};
    o->passes[o->npasses++] = SelectPass{0, 0, 10, 1};
    const int nb = bit_width((uint64_t)(o->N - 1));
    for (int top = ((nb + kDigitBits - 1) / kDigitBits) * kDigitBits; top > 0; top -= kDigitBits)
      o->passes[o->npasses++] = SelectPass{1, top - kDigitBits, kDigitBits, 0};
  }
  return TAH_OK;
}

void make_header(const Plan& pl, Header* h) {
  uint8_t b[128];
  memset(b, 0, sizeof(b));
  auto put = [&](int off, const void* src, int n) { memcpy(b + off, src, n); };
  const uint32_t magic = 0x51484154u;  // "TAHQ"
  const uint16_t ver = 2;
  const uint32_t A = (uint32_t)pl.A;
  const uint8_t dt = (uint8_t)pl.x_dtype, lg = (uint8_t)pl.log2G;
  put(0, &magic, 4);
  put(4, &ver, 2);
  put(6, &dt, 1);
  put(7, &lg, 1);
  put(8, &pl.tokens, 8);
  put(16, &pl.hidden, 8);
  put(24, &pl.S, 8);
  put(32, &pl.budget, 4);
  put(36, &pl.tau, 4);
  const uint8_t nc = (uint8_t)pl.n_candidates, bl = (uint8_t)pl.b_lo, bh = (uint8_t)pl.b_hi;
  put(40, &nc, 1);
  put(41, pl.candidates, 4);
  put(45, &bl, 1);
  put(46, &bh, 1);
  put(48, pl.allocator == TAH_ALLOC_TOP_P ? &pl.k : &pl.R, 8);
  put(56, &pl.tiles, 8);
  put(64, &pl.off_table, 8);
  put(72, &pl.off_bitmap, 8);
  put(80, &pl.off_side, 8);
  put(88, &pl.off_scale, 8);
  put(96, &pl.off_zero, 8);
  put(104, &pl.off_codes, 8);
  put(112, &pl.total, 8);
  put(120, &A, 4);
  const uint8_t al = (uint8_t)pl.allocator;
  put(124, &al, 1);
  memcpy(h->w, b, 128);
}

// Byte ranges of the payload that no section covers; the encoder zeroes them.
void make_pads(const Plan& pl, PadRanges* pr) {
  const int64_t ends[7][2] = {
      {128, pl.off_table},
      {pl.off_table + 4 * pl.nblocks, pl.off_bitmap},
      {pl.off_bitmap + (pl.allocator == TAH_ALLOC_GREEDY ? 16 : 8) * pl.nblocks, pl.off_side},
      {pl.off_side + pl.tiles, pl.off_scale},
      {pl.off_scale + 2 * pl.tiles, pl.off_zero},
      {pl.off_zero + 4 * pl.tiles, pl.off_codes},
      {pl.off_codes + pl.code_bytes, pl.total},
  };
  pr->n = 0;
  for (int i = 0; i < 7; ++i)
    if (ends[i][1] > ends[i][0]) {
      pr->off[pr->n] = ends[i][0];
      pr->len[pr->n] = (int32_t)(ends[i][1] - ends[i][0]);
      ++pr->n;
    }
}

static tah_status_t hip_status(hipError_t e) { return e == hipSuccess ? TAH_OK : TAH_ERR_HIP; }

static bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

static bool gpu_tile_ok(int G) { return G == 32 || G == 64 || G == 128; }

// Checks of an encode or round trip that do not involve the workspace.
static tah_status_t check_encode(const Plan& pl, const void* x, tah_dtype_t x_dtype, const void* payload,
                                 size_t payload_cap, const void* y, tah_dtype_t y_dtype, bool want_y) {
  if (x_dtype != TAH_DTYPE_F32 && x_dtype != TAH_DTYPE_BF16) return TAH_ERR_INVALID_ARG;
  if (want_y && y_dtype != TAH_DTYPE_F32 && y_dtype != TAH_DTYPE_BF16) return TAH_ERR_INVALID_ARG;
  if (!gpu_tile_ok(pl.G)) return TAH_ERR_UNSUPPORTED;
  if (payload && !aligned16(payload)) return TAH_ERR_INVALID_ARG;
  if (!want_y && !payload) return TAH_ERR_INVALID_ARG;
  if (pl.tiles > 0 && (!x || !aligned16(x) || (want_y && (!y || !aligned16(y))))) return TAH_ERR_INVALID_ARG;
  if (payload && payload_cap < (size_t)pl.total) return TAH_ERR_BUFFER_TOO_SMALL;
  return TAH_OK;
}

// The launch sequence of an encode or round trip on a checked plan.
static tah_status_t launch_encode_path(Plan& pl, const void* x, tah_dtype_t x_dtype, void* payload, void* y,
                                       tah_dtype_t y_dtype, bool want_y, void* ws, void* stream) {
  pl.x_dtype = x_dtype;
  hipStream_t st = static_cast<hipStream_t>(stream);
  uint8_t* w = static_cast<uint8_t*>(ws);
  // greedy with every tile at one level and allocation tiles of one
  // quantization tile: no select, and the uniform encoder writes the any-width
  // layout itself (its width map and block table are closed-form)
  const bool one_level = pl.mode == 2 && pl.glevel >= 0 && pl.kA == 1;
  const int mode = (pl.tiles > 0 && !one_level) ? pl.mode : 0;
  // mixed layouts: the statistics pass also writes the side bytes (Eq. 3)
  uint8_t* side = payload ? static_cast<uint8_t*>(payload) + pl.off_side : w + pl.ws_side;
  if (mode == 1) {
    hipError_t e = launch_stats(pl, x, reinterpret_cast<float*>(w + pl.ws_H), ws, true, side, st);
    if (e != hipSuccess) return hip_status(e);
    e = launch_select(pl, payload, ws, st);
    if (e != hipSuccess) return hip_status(e);
  } else if (mode == 2) {
    hipError_t e = launch_stats(pl, x, reinterpret_cast<float*>(w + pl.ws_H), ws, pl.glevel < 0, side, st);
    if (e != hipSuccess) return hip_status(e);
    e = launch_greedy(pl, payload, ws, st);
    if (e != hipSuccess) return hip_status(e);
  } else if (pl.kA > 1 && pl.tiles > 0) {
    // no selection, but the workspace still receives the allocation-tile
    // entropies; the encoder's own per-quantization-tile entropies then go to
    // the (by then consumed) partial-sum area
    hipError_t e = launch_stats(pl, x, reinterpret_cast<float*>(w + pl.ws_H), ws, false, nullptr, st);
    if (e != hipSuccess) return hip_status(e);
  }
  return hip_status(launch_encode(pl, x, payload, want_y ? y : nullptr, y_dtype, ws, st, mode));
}

static tah_status_t run_encode(const void* x, tah_dtype_t x_dtype, int64_t tokens, int64_t hidden,
                               const tah_params_t* p, void* payload, size_t payload_cap, void* y,
                               tah_dtype_t y_dtype, bool want_y, void* ws, size_t ws_cap, void* stream) {
  Plan pl;
  tah_status_t rc = make_plan(tokens, hidden, p, &pl);
  if (rc != TAH_OK) return rc;
  rc = check_encode(pl, x, x_dtype, payload, payload_cap, y, y_dtype, want_y);
  if (rc != TAH_OK) return rc;
  if (!ws || !aligned16(ws)) return TAH_ERR_INVALID_ARG;
  if (ws_cap < (size_t)pl.ws_total) return TAH_ERR_BUFFER_TOO_SMALL;
  return launch_encode_path(pl, x, x_dtype, payload, y, y_dtype, want_y, ws, stream);
}

// ---------------------------------------------------------------------------
// Scratch of the allocation-free round trip (tah_roundtrip_noalloc): device
// memory at file scope, TAH_NOALLOC_SCRATCH_BYTES on every GPU the library
// runs on, held until the process ends. It plays the part of the caller's
// workspace in the other calls. In host code the name `scratch` is a host-side
// stand-in, never a device address: kernels only ever receive the address that
// hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) uint8_t scratch[TAH_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
std::atomic<void*> g_scratch_addr[kMaxDevices];
}  // namespace

// Device address of `scratch` on the current device, looked up once per
// device with that device current (each GPU holds its own copy).
static tah_status_t scratch_on_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return TAH_ERR_HIP;
  if (dev >= kMaxDevices) return TAH_ERR_UNSUPPORTED;
  void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_addr[dev].load(std::memory_order_relaxed);
    if (!p) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return TAH_ERR_HIP;
      g_scratch_addr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return TAH_OK;
}

}  // namespace tah

using namespace tah;

extern "C" {

void tah_params_default(tah_params_t* p) {
  if (!p) return;
  memset(p, 0, sizeof(*p));
  p->tile = 64;
  p->tokens_per_sample = 0;
  p->bit_budget = 3.8f;
  p->n_candidates = 2;
  p->candidates[0] = 3;
  p->candidates[1] = 4;
  p->tau = 2.0f;
}

tah_status_t tah_payload_bytes(int64_t tokens, int64_t hidden, const tah_params_t* p, size_t* out) {
  Plan pl;
  tah_status_t rc = make_plan(tokens, hidden, p, &pl);
  if (rc != TAH_OK) return rc;
  if (!out) return TAH_ERR_INVALID_ARG;
  *out = (size_t)pl.total;
  return TAH_OK;
}

tah_status_t tah_workspace_bytes(int64_t tokens, int64_t hidden, const tah_params_t* p, size_t* out) {
  Plan pl;
  tah_status_t rc = make_plan(tokens, hidden, p, &pl);
  if (rc != TAH_OK) return rc;
  if (!out) return TAH_ERR_INVALID_ARG;
  *out = (size_t)pl.ws_total;
  return TAH_OK;
}

tah_status_t tah_workspace_entropy(int64_t tokens, int64_t hidden, const tah_params_t* p, size_t* offset) {
  Plan pl;
  tah_status_t rc = make_plan(tokens, hidden, p, &pl);
  if (rc != TAH_OK) return rc;
  if (!offset) return TAH_ERR_INVALID_ARG;
  *offset = (size_t)pl.ws_H;
  return TAH_OK;
}

tah_status_t tah_encode(const void* x, tah_dtype_t x_dtype, int64_t tokens, int64_t hidden, const tah_params_t* p,
                        void* payload, size_t payload_cap, void* ws, size_t ws_cap, void* stream) {
  if (!payload) return TAH_ERR_INVALID_ARG;
  return run_encode(x, x_dtype, tokens, hidden, p, payload, payload_cap, nullptr, TAH_DTYPE_F32, false, ws, ws_cap,
                    stream);
}

tah_status_t tah_roundtrip(const void* x, tah_dtype_t x_dtype, int64_t tokens, int64_t hidden, const tah_params_t* p,
                           void* payload, size_t payload_cap, void* y, tah_dtype_t y_dtype, void* ws, size_t ws_cap,
                           void* stream) {
  return run_encode(x, x_dtype, tokens, hidden, p, payload, payload_cap, y, y_dtype, true, ws, ws_cap, stream);
}

tah_status_t tah_roundtrip_noalloc(const void* x, tah_dtype_t x_dtype, int64_t tokens, int64_t hidden,
                                   const tah_params_t* p, void* payload, size_t payload_cap, void* y,
                                   tah_dtype_t y_dtype, void* stream) {
  Plan pl;
  tah_status_t rc = make_plan(tokens, hidden, p, &pl);
  if (rc != TAH_OK) return rc;
  rc = check_encode(pl, x, x_dtype, payload, payload_cap, y, y_dtype, true);
  if (rc != TAH_OK) return rc;
  if ((uint64_t)pl.ws_total > (uint64_t)TAH_NOALLOC_SCRATCH_BYTES) return TAH_ERR_SCRATCH_LIMIT;
  void* ws = nullptr;
  rc = scratch_on_current_device(&ws);
  if (rc != TAH_OK) return rc;
  return launch_encode_path(pl, x, x_dtype, payload, y, y_dtype, true, ws, stream);
}

tah_status_t tah_decode(const void* payload, size_t payload_len, int64_t tokens, int64_t hidden, const tah_params_t* p,
                        void* y, tah_dtype_t y_dtype, void* ws, size_t ws_cap, void* stream) {
  Plan pl;
  tah_status_t rc = make_plan(tokens, hidden, p, &pl);
  if (rc != TAH_OK) return rc;
  if (y_dtype != TAH_DTYPE_F32 && y_dtype != TAH_DTYPE_BF16) return TAH_ERR_INVALID_ARG;
  if (!gpu_tile_ok(pl.G)) return TAH_ERR_UNSUPPORTED;
  if (!payload || !aligned16(payload) || !ws || !aligned16(ws)) return TAH_ERR_INVALID_ARG;
  if (pl.tiles > 0 && (!y || !aligned16(y))) return TAH_ERR_INVALID_ARG;
  if (payload_len < (size_t)pl.total) return TAH_ERR_BUFFER_TOO_SMALL;
  if (ws_cap < (size_t)pl.ws_total) return TAH_ERR_BUFFER_TOO_SMALL;
  return hip_status(launch_decode(pl, payload, y, y_dtype, ws, static_cast<hipStream_t>(stream)));
}

tah_status_t tah_tile_entropy(const void* x, tah_dtype_t x_dtype, int64_t tokens, int64_t hidden,
                              const tah_params_t* p, float* h, void* ws, size_t ws_cap, void* stream) {
  Plan pl;
  tah_status_t rc = make_plan(tokens, hidden, p, &pl);
  if (rc != TAH_OK) return rc;
  if (x_dtype != TAH_DTYPE_F32 && x_dtype != TAH_DTYPE_BF16) return TAH_ERR_INVALID_ARG;
  if (!gpu_tile_ok(pl.G)) return TAH_ERR_UNSUPPORTED;
  if (!ws || !aligned16(ws)) return TAH_ERR_INVALID_ARG;
  if (pl.tiles > 0 && (!x || !aligned16(x) || !h || ((uintptr_t)h & 3u))) return TAH_ERR_INVALID_ARG;
  if (ws_cap < (size_t)pl.ws_total) return TAH_ERR_BUFFER_TOO_SMALL;
  if (pl.tiles == 0) return TAH_OK;
  pl.x_dtype = x_dtype;
  return hip_status(launch_stats(pl, x, h, ws, false, nullptr, static_cast<hipStream_t>(stream)));
}

static bool naive_ok(int64_t n, int bits, float c) {
  return n >= 0 && bits >= 2 && bits <= 16 && c > 0.0f && isfinite(c) && isfinite(ldexpf(c, bits - 1));
}

tah_status_t tah_naive_payload_bytes(int64_t n, int bits, size_t* out) {
  if (n < 0 || bits < 2 || bits > 16 || !out) return TAH_ERR_INVALID_ARG;
  *out = (size_t)naive_payload_bytes(n, bits);
  return TAH_OK;
}

tah_status_t tah_naive_encode(const void* g, tah_dtype_t g_dtype, int64_t n, int bits, float c, void* payload,
                              size_t payload_cap, void* stream) {
  if (!naive_ok(n, bits, c)) return TAH_ERR_INVALID_ARG;
  if (g_dtype != TAH_DTYPE_F32 && g_dtype != TAH_DTYPE_BF16) return TAH_ERR_INVALID_ARG;
  if (!payload || !aligned16(payload) || (n > 0 && (!g || !aligned16(g)))) return TAH_ERR_INVALID_ARG;
  if (payload_cap < (size_t)naive_payload_bytes(n, bits)) return TAH_ERR_BUFFER_TOO_SMALL;
  return hip_status(launch_naive_encode(g, g_dtype, n, bits, c, payload, static_cast<hipStream_t>(stream)));
}

tah_status_t tah_naive_decode(const void* payload, size_t payload_len, int64_t n, int bits, float c, void* y,
                              tah_dtype_t y_dtype, void* ws, size_t ws_cap, void* stream) {
  if (!naive_ok(n, bits, c)) return TAH_ERR_INVALID_ARG;
  if (y_dtype != TAH_DTYPE_F32 && y_dtype != TAH_DTYPE_BF16) return TAH_ERR_INVALID_ARG;
  if (!payload || !aligned16(payload) || !ws || !aligned16(ws) || (n > 0 && (!y || !aligned16(y))))
    return TAH_ERR_INVALID_ARG;
  if (payload_len < (size_t)naive_payload_bytes(n, bits)) return TAH_ERR_BUFFER_TOO_SMALL;
  if (ws_cap < 256) return TAH_ERR_BUFFER_TOO_SMALL;
  return hip_status(launch_naive_decode(payload, n, bits, c, y, y_dtype, ws, static_cast<hipStream_t>(stream)));
}

tah_status_t tah_hadamard(const void* x, tah_dtype_t x_dtype, int64_t n_tiles, int tile, int method, float* y,
                          void* stream) {
  if (n_tiles < 0 || (tile != 32 && tile != 64 && tile != 128)) return TAH_ERR_INVALID_ARG;
  if (x_dtype != TAH_DTYPE_F32 && x_dtype != TAH_DTYPE_BF16) return TAH_ERR_INVALID_ARG;
  if (method != TAH_HADAMARD_BUTTERFLY && method != TAH_HADAMARD_MFMA) return TAH_ERR_INVALID_ARG;
  if (n_tiles > 0 && (!x || !aligned16(x) || !y || !aligned16(y))) return TAH_ERR_INVALID_ARG;
  if (method == TAH_HADAMARD_MFMA && (tile != 64 || x_dtype != TAH_DTYPE_BF16)) return TAH_ERR_UNSUPPORTED;
  return hip_status(launch_hadamard(x, x_dtype, n_tiles, tile, method, y, static_cast<hipStream_t>(stream)));
}

tah_status_t tah_read_device_status(const void* ws, void* stream, int32_t* out) {
  if (!ws || !out) return TAH_ERR_INVALID_ARG;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (hipStreamSynchronize(st) != hipSuccess) return TAH_ERR_HIP;
  if (hipMemcpy(out, ws, sizeof(int32_t), hipMemcpyDeviceToHost) != hipSuccess) return TAH_ERR_HIP;
  return TAH_OK;
}

const char* tah_status_string(tah_status_t s) {
  switch (s) {
    case TAH_OK: return "ok";
    case TAH_ERR_INVALID_ARG: return "invalid argument";
    case TAH_ERR_UNSUPPORTED: return "unsupported on this device build";
    case TAH_ERR_BUFFER_TOO_SMALL: return "buffer too small";
    case TAH_ERR_BUDGET_INFEASIBLE: return "bit budget below the smallest candidate width";
    case TAH_ERR_BAD_PAYLOAD: return "payload header does not match shape/params";
    case TAH_ERR_HIP: return "HIP runtime error";
    case TAH_ERR_SCRATCH_LIMIT: return "shape needs more scratch than the allocation-free round trip holds";
  }
  return "unknown status";
}

int tah_abi_version(void) { return TAH_ABI_VERSION; }

}  // extern "C"
