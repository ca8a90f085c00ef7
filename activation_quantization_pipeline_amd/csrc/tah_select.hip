// Per-sample bit allocation of TAH-Quant (§3.2 "Top-p% tile selection") for
// gfx950: the k highest-entropy tiles of every sample get the higher width.
//
// Instead of sorting the S*M entropies of a sample (the paper's
// O(SM log SM) ranking), the k-th largest key is found by a radix select:
//   k_stats  - one lane per tile computes the entropy of Eq. (1)-(2) from the
//              LDS-staged tile and writes it to the workspace; it also resets
//              the selection state and histograms;
//   k_hist   - one pass per digit: a 2048-bin LDS histogram of the current
//              digit over the keys that still match the prefix, merged into
//              the sample's global histogram; the last workgroup to finish
//              (atomic ticket) picks the digit that holds rank r. Three passes
//              cover the 32-bit order-preserving entropy key; then passes over
//              the tile index resolve ties (lower index first);
//   k_mark   - one bit per tile: key above the threshold, or equal to it with
//              an index up to the last selected tie; per-64-tile counts;
//   k_table  - exclusive scan of those counts: b_hi tiles before each run of
//              64 tiles, which locates every variable-width code block.
#include <type_traits>

#include "tah_device.hpp"
#include "tah_internal.hpp"

namespace tah {

// fp32 -> uint32 with the same order (entropies are never NaN).
__device__ __forceinline__ uint32_t orderable(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ------------------------------------------------------------------ stats ----
struct StatsArgs {
  const uint8_t* x;
  float* h;
  SampleState* st;
  uint32_t* hist;
  uint32_t* counter;
  int64_t tiles, nsamples, k, hist_words;
  int32_t init;
};

template <int G, typename TIn>
constexpr int stats_tiles_per_wg() {
  return TileRow<G, TIn>::kBytes <= 128 ? 256 : (TileRow<G, TIn>::kBytes <= 256 ? 128 : 64);
}

template <int G, typename TIn>
__global__ __launch_bounds__((stats_tiles_per_wg<G, TIn>())) void k_stats(StatsArgs a) {
  constexpr int NT = stats_tiles_per_wg<G, TIn>();
  using RI = TileRow<G, TIn>;
  __shared__ __attribute__((aligned(16))) uint8_t xs[NT * RI::kStride];
  __shared__ __attribute__((aligned(16))) float lt[256];  // log2 tables of the entropy
  const int tid = threadIdx.x;
  const int64_t t0 = (int64_t)blockIdx.x * NT;
  if (a.init) {
    const int64_t gid = (int64_t)blockIdx.x * NT + tid, gsz = (int64_t)gridDim.x * NT;
    for (int64_t i = gid; i < a.hist_words; i += gsz) a.hist[i] = 0u;
    for (int64_t s = gid; s < a.nsamples; s += gsz) {
      SampleState z;
      z.key = 0u;
      z.upos = 0u;
      z.r = a.k;
      z.tie_all = 0;
      z.pad = 0;
      a.st[s] = z;
    }
    if (gid == 0) *a.counter = 0u;
  }
  const int n = (int)((a.tiles - t0) < NT ? (a.tiles - t0) : NT);
  if (n <= 0) return;
  load_log2_tab(lt);
  stage_in<G, TIn, NT>(a.x + t0 * RI::kBytes, xs, n);
  __syncthreads();
  if (tid < n) {
    float v[G];
    lds_read_tile<G, TIn>(xs + tid * RI::kStride, v);
    float l1 = 0.0f;
#pragma unroll
    for (int k = 0; k < G; ++k) l1 = l1 + fabsf(v[k]);
    a.h[t0 + tid] = tile_entropy<G, Elem<TIn>::kBytes == 2>(v, l1, lt);  // Eq. (1)-(2)
  }
}

template <int G, typename TIn>
static hipError_t launch_stats_t(const StatsArgs& a, hipStream_t st) {
  constexpr int NT = stats_tiles_per_wg<G, TIn>();
  const int64_t nwg = a.tiles > 0 ? (a.tiles + NT - 1) / NT : 1;
  hipLaunchKernelGGL((k_stats<G, TIn>), dim3((unsigned)nwg), dim3(NT), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_stats(const Plan& pl, const void* x, float* h_out, void* ws, bool init_select, hipStream_t st) {
  uint8_t* w = static_cast<uint8_t*>(ws);
  StatsArgs a;
  a.x = static_cast<const uint8_t*>(x);
  a.h = h_out;
  a.st = reinterpret_cast<SampleState*>(w + pl.ws_state);
  a.hist = reinterpret_cast<uint32_t*>(w + pl.ws_hist);
  a.counter = reinterpret_cast<uint32_t*>(w + pl.ws_counter);
  a.tiles = pl.tiles;
  a.nsamples = pl.nsamples;
  a.k = pl.k;
  a.hist_words = pl.k > 0 ? pl.nsamples * kBins : 0;
  a.init = init_select ? 1 : 0;
  const bool bf = pl.x_dtype == TAH_DTYPE_BF16;
  switch (pl.G) {
    case 32: return bf ? launch_stats_t<32, bf16_t>(a, st) : launch_stats_t<32, float>(a, st);
    case 64: return bf ? launch_stats_t<64, bf16_t>(a, st) : launch_stats_t<64, float>(a, st);
    case 128: return bf ? launch_stats_t<128, bf16_t>(a, st) : launch_stats_t<128, float>(a, st);
    default: return hipErrorInvalidValue;
  }
}

// ------------------------------------------------------------------ hist ----
struct HistArgs {
  const float* H;
  SampleState* st;
  uint32_t* hist;
  uint32_t* counter;
  int64_t N, nsamples, chunks_per_sample;
  uint32_t total_wg;
  SelectPass pass;
};

constexpr int kHistThreads = 256;
constexpr int kHistPerThread = 4;
constexpr int kHistChunk = kHistThreads * kHistPerThread;

// The wave scans one sample's histogram in order (descending digits for the
// entropy key, ascending for the tile index) and keeps the digit where the
// running count reaches r; the histogram is cleared for the next pass.
__device__ void finalize_sample(const HistArgs& a, int64_t s) {
  const int lane = threadIdx.x & 63;
  uint32_t* h = a.hist + s * kBins;
  SampleState S = a.st[s];
  const bool skip = a.pass.kind == 1 && S.tie_all;
  constexpr int PER = kBins / 64;
  uint32_t c[PER];
  uint32_t sum = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int ord = lane * PER + i;
    const int bin = a.pass.kind == 0 ? (kBins - 1 - ord) : ord;
    c[i] = __hip_atomic_load(&h[bin], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    sum += c[i];
  }
  // inclusive prefix of the per-lane sums over the wave
  uint64_t incl = sum;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint64_t o = __shfl_up(incl, off, 64);
    if (lane >= off) incl += o;
  }
  const uint64_t excl = incl - sum;
  const bool here = !skip && (int64_t)excl < S.r && S.r <= (int64_t)incl;
  if (here) {
    int64_t before = (int64_t)excl;
    int ord = lane * PER;
    uint32_t cnt = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      if (before + (int64_t)c[i] >= S.r) {
        ord = lane * PER + i;
        cnt = c[i];
        break;
      }
      before += c[i];
    }
    const uint32_t digit = (uint32_t)(a.pass.kind == 0 ? (kBins - 1 - ord) : ord);
    S.r -= before;
    if (a.pass.kind == 0) {
      S.key |= digit << a.pass.shift;
      if (a.pass.last_h) {
        S.tie_all = (S.r == (int64_t)cnt) ? 1 : 0;
        S.upos = S.tie_all ? 0xffffffffu : 0u;
      }
    } else {
      S.upos |= digit << a.pass.shift;
    }
    a.st[s] = S;
  }
#pragma unroll
  for (int i = 0; i < PER; ++i) h[lane * PER + i] = 0u;
}

__global__ __launch_bounds__(kHistThreads) void k_hist(HistArgs a) {
  __shared__ uint32_t lh[kBins];
  __shared__ int last;
  const int tid = threadIdx.x;
  for (int i = tid; i < kBins; i += kHistThreads) lh[i] = 0u;
  __syncthreads();
  const int64_t s = blockIdx.x / a.chunks_per_sample;
  const int64_t u0 = (blockIdx.x % a.chunks_per_sample) * kHistChunk;
  const SampleState S = a.st[s];
  const int hs = a.pass.shift + a.pass.width;  // bits above the current digit
  const uint32_t dmask = (1u << a.pass.width) - 1u;
#pragma unroll
  for (int i = 0; i < kHistPerThread; ++i) {
    const int64_t u = u0 + i * kHistThreads + tid;
    if (u < a.N) {
      const uint32_t key = orderable(a.H[s * a.N + u]);
      bool match;
      uint32_t digit;
      if (a.pass.kind == 0) {
        match = hs >= 32 || (key >> hs) == (S.key >> hs);
        digit = (key >> a.pass.shift) & dmask;
      } else {
        const uint32_t uu = (uint32_t)u;
        match = !S.tie_all && key == S.key && (hs >= 32 || (uu >> hs) == (S.upos >> hs));
        digit = (uu >> a.pass.shift) & dmask;
      }
      if (match) atomicAdd(&lh[digit], 1u);
    }
  }
  __syncthreads();
  for (int i = tid; i < kBins; i += kHistThreads)
    if (lh[i]) atomicAdd(&a.hist[s * kBins + i], lh[i]);
  __threadfence();
  __syncthreads();
  if (tid == 0) last = (atomicAdd(a.counter, 1u) == a.total_wg - 1u) ? 1 : 0;
  __syncthreads();
  if (!last) return;
  __threadfence();
  for (int64_t s2 = tid >> 6; s2 < a.nsamples; s2 += kHistThreads / 64) finalize_sample(a, s2);
  __syncthreads();
  if (tid == 0) *a.counter = 0u;
}

// ------------------------------------------------------------------ mark ----
struct MarkArgs {
  const float* H;
  const SampleState* st;
  uint32_t* bitmap;
  uint32_t* blockcnt;
  int64_t tiles, N, nblocks;
};

__global__ __launch_bounds__(256) void k_mark(MarkArgs a) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int64_t t = (int64_t)blockIdx.x * 256 + tid;
  bool sel = false;
  if (t < a.tiles) {
    const int64_t s = t / a.N;
    const uint32_t u = (uint32_t)(t - s * a.N);
    const uint32_t key = orderable(a.H[t]);
    const SampleState S = a.st[s];
    sel = key > S.key || (key == S.key && u <= S.upos);
  }
  const uint64_t m = ballot(sel);
  const int64_t blk = ((int64_t)blockIdx.x * 256 + (tid & ~63)) >> 6;
  if (lane == 0 && blk < a.nblocks) {
    a.bitmap[2 * blk] = (uint32_t)m;
    a.bitmap[2 * blk + 1] = (uint32_t)(m >> 32);
    a.blockcnt[blk] = (uint32_t)__popcll(m);
  }
}

// ------------------------------------------------------------------ table ----
constexpr int kScanThreads = 1024;

__global__ __launch_bounds__(kScanThreads) void k_table(const uint32_t* cnt, uint32_t* table, int64_t nblocks) {
  __shared__ uint32_t wsum[kScanThreads / 64];
  __shared__ uint32_t carry_s;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) carry_s = 0u;
  __syncthreads();
  for (int64_t base = 0; base < nblocks; base += kScanThreads) {
    const int64_t i = base + tid;
    const uint32_t v = i < nblocks ? cnt[i] : 0u;
    uint32_t incl = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const uint32_t o = __shfl_up(incl, off, 64);
      if (lane >= off) incl += o;
    }
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    uint32_t before = carry_s;
    for (int w = 0; w < wave; ++w) before += wsum[w];
    if (i < nblocks) table[i] = before + incl - v;
    __syncthreads();
    if (tid == kScanThreads - 1) carry_s = before + incl;
    __syncthreads();
  }
}

hipError_t launch_select(const Plan& pl, void* payload, void* ws, hipStream_t st) {
  uint8_t* w = static_cast<uint8_t*>(ws);
  uint8_t* P = static_cast<uint8_t*>(payload);
  HistArgs h;
  h.H = reinterpret_cast<const float*>(w + pl.ws_H);
  h.st = reinterpret_cast<SampleState*>(w + pl.ws_state);
  h.hist = reinterpret_cast<uint32_t*>(w + pl.ws_hist);
  h.counter = reinterpret_cast<uint32_t*>(w + pl.ws_counter);
  h.N = pl.N;
  h.nsamples = pl.nsamples;
  h.chunks_per_sample = (pl.N + kHistChunk - 1) / kHistChunk;
  const int64_t nwg = h.chunks_per_sample * pl.nsamples;
  h.total_wg = (uint32_t)nwg;
  for (int p = 0; p < pl.npasses; ++p) {
    h.pass = pl.passes[p];
    hipLaunchKernelGGL(k_hist, dim3((unsigned)nwg), dim3(kHistThreads), 0, st, h);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  MarkArgs m;
  m.H = h.H;
  m.st = h.st;
  m.bitmap = reinterpret_cast<uint32_t*>(P ? P + pl.off_bitmap : w + pl.ws_bitmap);
  m.blockcnt = reinterpret_cast<uint32_t*>(w + pl.ws_blockcnt);
  m.tiles = pl.tiles;
  m.N = pl.N;
  m.nblocks = pl.nblocks;
  hipLaunchKernelGGL(k_mark, dim3((unsigned)((pl.tiles + 255) / 256)), dim3(256), 0, st, m);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  uint32_t* table = reinterpret_cast<uint32_t*>(P ? P + pl.off_table : w + pl.ws_table);
  hipLaunchKernelGGL(k_table, dim3(1), dim3(kScanThreads), 0, st, (const uint32_t*)m.blockcnt, table, pl.nblocks);
  return hipGetLastError();
}

}  // namespace tah
