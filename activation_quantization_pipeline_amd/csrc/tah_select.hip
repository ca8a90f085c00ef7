// Per-sample bit allocation of TAH-Quant (§3.2 "Top-p% tile selection") for
// gfx950: the k highest-entropy tiles of every sample get the higher width.
//
// Instead of sorting the S*M entropies of a sample (the paper's
// O(SM log SM) ranking), the k-th largest key is found by a radix select:
//   k_stats  - one lane per tile computes the entropy of Eq. (1)-(2) from the
//              LDS-staged tile and writes it to the workspace; it also resets
//              the selection state and histograms. When an allocation tile
//              spans kA > 1 quantization tiles, the lane writes the tile's two
//              sums (L, S) instead and k_alloc_entropy adds them up per
//              allocation tile, left to right, into its entropy (when kA
//              divides 64 the workgroup adds them itself);
//   k_hist   - one launch per digit pass. Each workgroup first applies the
//              previous pass (one wavefront reads that pass's histogram of the
//              sample in coalesced slices and finds the digit that holds rank
//              r), then builds a 2048-bin LDS histogram of the current digit
//              over the keys that still match the prefix (on the first digit,
//              where entropy keys cluster, lanes of a wavefront that share a
//              digit add once) and adds it into the sample's global
//              histogram. Three passes cover the 32-bit
//              order-preserving entropy key. Histograms rotate over three
//              buffers (read the previous, add to the current, clear the next)
//              and states over two, so kernel boundaries are the only
//              synchronisation: a last-workgroup ticket would need a
//              device-scope release per workgroup, which on this multi-die part
//              writes back the L2;
//   k_resolve - one workgroup per sample applies the last pass: the final
//              threshold state. Ties at the threshold key are broken by tile
//              index (lower first) by digit passes over the sample inside this
//              workgroup, only when they occur;
//   k_mark   - one bit per quantization tile, from its allocation tile: key
//              above the threshold, or equal to it with an index up to the last
//              selected tie; per-64-tile counts;
//   k_table  - exclusive scan of those counts: b_hi tiles before each run of
//              64 tiles, which locates every variable-width code block.
// When samples are whole runs of 64 allocation tiles (at most kFoldMaxRuns
// runs of quantization tiles) and an allocation tile is 1, 2, 4, ... or 64
// quantization tiles, k_mark and k_table do not run: the last k_hist pass
// writes the width-map bits of the keys above the threshold's prefix (each
// allocation tile's bit once per quantization tile) and each run's count, and
// k_resolve adds the selected keys that match the prefix and scans the run
// counts into the block table.
// Samples of at most kLdsSelect keys skip k_hist and k_resolve: one
// workgroup per sample (k_select_lds) holds the keys in LDS, runs every digit
// pass there and, when samples cover whole runs of 64 tiles, writes the width
// map and block table itself.
#include <type_traits>

#include "tah_device.hpp"
#include "tah_internal.hpp"
#include "tah_scan.hpp"

namespace tah {

// fp32 -> uint32 with the same order (entropies are never NaN).
__device__ __forceinline__ uint32_t orderable(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ------------------------------------------------------------------ stats ----
struct StatsArgs {
  const uint8_t* x;
  float* h;     // entropy per tile (allocation tile = quantization tile)
  float2* ls;   // (L, S) per tile (allocation tile of several quantization tiles)
  uint32_t* hist;
  uint8_t* side;  // Eq. (3) per tile as the payload's side byte (mixed layouts), or null
  float tau;
  int64_t tiles, hist_words;
  int32_t init;
  // SUMS with kA dividing 64: each workgroup's 64 quantization tiles hold
  // whole allocation tiles, whose entropies it then forms itself into h
  int32_t kA_fused;
};

// An allocation tile's entropy from its kA quantization tiles' sums in LDS
// (lsum / ssum, the workgroup's tiles in order), added left to right from 0
// as k_alloc_entropy adds them; lane u < n / kA writes allocation tile
// t0 / kA + u. Called by every lane of the workgroup.
__device__ __forceinline__ void fused_alloc_entropy(const StatsArgs& a, const float* lsum, const float* ssum,
                                                    const float* lt, int64_t t0, int n, int tid) {
  const int kA = a.kA_fused;
  if (tid < n / kA) {
    float L = 0.0f, S = 0.0f;
    for (int gq = 0; gq < kA; ++gq) {
      L = L + lsum[tid * kA + gq];
      S = S + ssum[tid * kA + gq];
    }
    a.h[t0 / kA + tid] = entropy_from_sums(L, S, lt);
  }
}

// Tiles (= threads) per workgroup of the statistics pass for rows of up to 128
// bytes: one-wavefront workgroups, so 4096 x 2048 bf16 (131,072 tiles)
// spreads over 2,048 workgroups instead of 512, eight per compute unit (round
// trip 43.0 -> 41.6 us; 8192 x 8192 within 0.3 us; 128 and 512 tiles per
// workgroup were no faster). Wider rows take k_stats_rounds below.
template <int G, typename TIn>
constexpr int stats_tiles_per_wg() {
  static_assert(TileRow<G, TIn>::kBytes <= 128, "wider rows are staged in rounds");
  return 64;
}

// SIDE: also the outlier test of Eq. (3), m1 > tau (m2 + rho), and the side
// byte (bit 7 the flag, bits 0-6 the pivot of a transformed tile), which the
// mixed-width encoder then reads instead of finding the top two magnitudes.
template <int G, typename TIn, bool SUMS, bool SIDE, int NT = stats_tiles_per_wg<G, TIn>()>
__global__ __launch_bounds__(NT) void k_stats(StatsArgs a) {
  using RI = TileRow<G, TIn>;
  __shared__ __attribute__((aligned(16))) uint8_t xs[NT * RI::kStride];
  __shared__ __attribute__((aligned(16))) float lt[256];  // log2 tables of the entropy
  __shared__ float lsum[SUMS ? NT : 1], ssum[SUMS ? NT : 1];
  const int tid = threadIdx.x;
  const int64_t t0 = (int64_t)blockIdx.x * NT;
  if (a.init) {  // the first selection pass's histograms start at zero
    const int64_t gid = (int64_t)blockIdx.x * NT + tid, gsz = (int64_t)gridDim.x * NT;
    for (int64_t i = gid; i < a.hist_words; i += gsz) a.hist[i] = 0u;
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
    if constexpr (SIDE) {
      float m1, m2;
      int d;
      tile_stats_regs<G, Elem<TIn>::kBytes == 2>(v, m1, m2, d, l1);
      const bool flag = m1 > a.tau * (m2 + kRho);  // Eq. (3) without the division
      a.side[t0 + tid] = (uint8_t)(flag ? (0x80 | d) : 0);
    } else {
#pragma unroll
      for (int k = 0; k < G; ++k) l1 = l1 + fabsf(v[k]);
    }
    if constexpr (SUMS) {
      const float S = tile_logsum<G, Elem<TIn>::kBytes == 2>(v, lt);
      if (a.kA_fused) {
        lsum[tid] = l1;
        ssum[tid] = S;
      } else {
        a.ls[t0 + tid] = make_float2(l1, S);
      }
    } else {
      a.h[t0 + tid] = tile_entropy<G, Elem<TIn>::kBytes == 2>(v, l1, lt);  // Eq. (1)-(2)
    }
  }
  if constexpr (SUMS) {
    if (a.kA_fused) {
      __syncthreads();
      fused_alloc_entropy(a, lsum, ssum, lt, t0, n, tid);
    }
  }
}

// Tiles wider than 128 bytes (fp32 tiles of 64 or 128 elements, bf16 tiles of
// 128): a whole tile row per lane needs 272 or 528 bytes of LDS per tile and
// up to 128 registers for its values, which left one or two wavefronts per
// SIMD. Here a one-wavefront workgroup of 64 tiles stages each tile 128 bytes
// at a time (rounds r = 0, 1, ...: bytes 128 r ... 128 r + 127 of every tile
// into 144-byte LDS rows, 10 KB with the log2 table, so 16 workgroups share a
// compute unit), the next round's loads in flight while the lane streams the
// current one, and carries the statistics from round to round in element
// order: the same operations in the same order as tile_stats_regs,
// tile_logsum and tile_entropy over the whole tile.
template <int G, typename TIn>
constexpr int stats_rounds() { return G * Elem<TIn>::kBytes / 128; }

template <int G, typename TIn, bool SUMS, bool SIDE>
__global__ __launch_bounds__(64) void k_stats_rounds(StatsArgs a) {
  constexpr int NT = 64;
  constexpr int EB = Elem<TIn>::kBytes;
  constexpr int kBytes = G * EB;
  constexpr int R = stats_rounds<G, TIn>();
  constexpr int kStride = 128 + 16;
  static_assert(R >= 2 && R * 128 == kBytes, "rows of whole 128-byte rounds");
  __shared__ __attribute__((aligned(16))) uint8_t xs[NT * kStride];
  __shared__ __attribute__((aligned(16))) float lt[256];  // log2 tables of the entropy
  __shared__ float lsum[SUMS ? NT : 1], ssum[SUMS ? NT : 1];
  const int tid = threadIdx.x;
  const int64_t t0 = (int64_t)blockIdx.x * NT;
  if (a.init) {  // the first selection pass's histograms start at zero
    const int64_t gid = (int64_t)blockIdx.x * NT + tid, gsz = (int64_t)gridDim.x * NT;
    for (int64_t i = gid; i < a.hist_words; i += gsz) a.hist[i] = 0u;
  }
  const int n = (int)((a.tiles - t0) < NT ? (a.tiles - t0) : NT);
  if (n <= 0) return;
  load_log2_tab(lt);
  // chunk c = tid + 64 i of a round: tile c / 8, 16-byte part c % 8 of the
  // round's 128 bytes (eight lanes read one 128-byte line)
  const uint8_t* base = a.x + t0 * kBytes;
  uint4 cur[8], nxt[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int c = tid + 64 * i;
    cur[i] = (c >> 3) < n ? *reinterpret_cast<const uint4*>(base + (int64_t)(c >> 3) * kBytes + (c & 7) * 16)
                          : make_uint4(0u, 0u, 0u, 0u);
  }
  float s = 0.0f, S = 0.0f, a1 = 0.0f, a2 = 0.0f;  // fp32: sums, top two magnitudes
  int dd = 0;
  uint32_t k1 = 0u, k2 = 0u;  // bf16: top-two keys
  const uint4* rd = reinterpret_cast<const uint4*>(xs + tid * kStride);
#pragma unroll
  for (int r = 0; r < R; ++r) {
    if (r > 0) __syncthreads();  // every lane is done with the previous round's rows
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int c = tid + 64 * i;
      *reinterpret_cast<uint4*>(xs + (c >> 3) * kStride + (c & 7) * 16) = cur[i];
    }
    __syncthreads();
    if (r + 1 < R) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int c = tid + 64 * i;
        nxt[i] = (c >> 3) < n ? *reinterpret_cast<const uint4*>(base + (int64_t)(c >> 3) * kBytes + (r + 1) * 128 +
                                                                 (c & 7) * 16)
                              : make_uint4(0u, 0u, 0u, 0u);
      }
    }
    if (tid < n) {
#pragma unroll
      for (int cc = 0; cc < 8; ++cc) {
        const uint4 q = rd[cc];
        const uint32_t u[4] = {q.x, q.y, q.z, q.w};
        if constexpr (EB == 2) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int k = 64 * r + 8 * cc + 2 * i;
            uint32_t xl, xh;  // the widened values, opaque (one bit-field extract for the table)
            asm("v_lshlrev_b32 %0, 16, %1" : "=v"(xl) : "v"(u[i]));
            asm("v_and_b32 %0, 0xffff0000, %1" : "=v"(xh) : "v"(u[i]));
            const float vl = __uint_as_float(xl), vh = __uint_as_float(xh);
            s = s + fabsf(vl);
            if constexpr (SIDE) {
              const uint32_t kl = (xl & 0x7fff0000u) | (uint32_t)(G - 1 - k);
              k2 = umed3(k2, kl, k1);
              k1 = max(k1, kl);
            }
            S = __builtin_fmaf(fabsf(vl), log2_node(vl, lt), S);
            s = s + fabsf(vh);
            if constexpr (SIDE) {
              const uint32_t kh = (u[i] & 0x7fff0000u) | (uint32_t)(G - 2 - k);
              k2 = umed3(k2, kh, k1);
              k1 = max(k1, kh);
            }
            S = __builtin_fmaf(fabsf(vh), log2_node(vh, lt), S);
          }
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int k = 32 * r + 4 * cc + i;
            const float av = fabsf(__uint_as_float(u[i]));
            s = s + av;
            if constexpr (SIDE) {
              if (k == 0) {
                a1 = av;
                a2 = 0.0f;
                dd = 0;
              } else {
                const bool c = av > a1;
                a2 = __builtin_amdgcn_fmed3f(a2, av, a1);
                a1 = fmaxf(a1, av);
                dd = c ? k : dd;
              }
            }
            S = __builtin_fmaf(av, log2_full(av, lt), S);
          }
        }
      }
    }
    if (r + 1 < R) {
#pragma unroll
      for (int i = 0; i < 8; ++i) cur[i] = nxt[i];
    }
  }
  if (tid < n) {
    if constexpr (SIDE) {
      float m1, m2;
      int d;
      if constexpr (EB == 2) {
        m1 = __uint_as_float(k1 & 0xffff0000u);
        m2 = __uint_as_float(k2 & 0xffff0000u);
        d = G - 1 - (int)(k1 & 0xffffu);
      } else {
        m1 = a1;
        m2 = a2;
        d = dd;
      }
      const bool flag = m1 > a.tau * (m2 + kRho);  // Eq. (3) without the division
      a.side[t0 + tid] = (uint8_t)(flag ? (0x80 | d) : 0);
    }
    if constexpr (SUMS) {
      asm volatile("" : "+v"(S));  // the sum is complete here
      if (a.kA_fused) {
        lsum[tid] = s;
        ssum[tid] = S;
      } else {
        a.ls[t0 + tid] = make_float2(s, S);
      }
    } else {
      a.h[t0 + tid] = entropy_from_sums(s, S, lt);  // Eq. (1)-(2)
    }
  }
  if constexpr (SUMS) {
    if (a.kA_fused) {
      __syncthreads();
      fused_alloc_entropy(a, lsum, ssum, lt, t0, n, tid);
    }
  }
}

// Entropy of each allocation tile u of kA quantization tiles (u * kA ...
// u * kA + kA - 1): their sums added left to right from 0, then the identity
// H = log2 L - S / L.
__global__ __launch_bounds__(256) void k_alloc_entropy(const float2* ls, float* h, int64_t atiles, int64_t kA) {
  __shared__ __attribute__((aligned(16))) float lt[256];
  load_log2_tab(lt);
  __syncthreads();
  const int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (u >= atiles) return;
  const float2* p = ls + u * kA;
  float L = 0.0f, S = 0.0f;
  // unrolled so that eight loads are in flight ahead of the in-order adds
  // (token-level allocation at 8192 x 8192: 132.4 -> 121.6 us per round trip)
#pragma unroll 8
  for (int64_t g = 0; g < kA; ++g) {
    const float2 q = p[g];
    L = L + q.x;
    S = S + q.y;
  }
  h[u] = entropy_from_sums(L, S, lt);
}

template <int G, typename TIn>
static hipError_t launch_stats_t(const StatsArgs& a, bool sums, hipStream_t st) {
  if constexpr (G * Elem<TIn>::kBytes > 128) {
    const int64_t nwg = a.tiles > 0 ? (a.tiles + 63) / 64 : 1;
    const dim3 grid((unsigned)nwg), block(64);
    if (sums && a.side) hipLaunchKernelGGL((k_stats_rounds<G, TIn, true, true>), grid, block, 0, st, a);
    else if (sums) hipLaunchKernelGGL((k_stats_rounds<G, TIn, true, false>), grid, block, 0, st, a);
    else if (a.side) hipLaunchKernelGGL((k_stats_rounds<G, TIn, false, true>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((k_stats_rounds<G, TIn, false, false>), grid, block, 0, st, a);
  } else if (sums && a.kA_fused == 128) {
    // token-level allocation over 128 quantization tiles: two-wavefront
    // workgroups of 128 tiles, so that each holds whole allocation tiles
    const int64_t nwg = a.tiles > 0 ? (a.tiles + 127) / 128 : 1;
    const dim3 grid((unsigned)nwg), block(128);
    if (a.side) hipLaunchKernelGGL((k_stats<G, TIn, true, true, 128>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((k_stats<G, TIn, true, false, 128>), grid, block, 0, st, a);
  } else {
    constexpr int NT = stats_tiles_per_wg<G, TIn>();
    const int64_t nwg = a.tiles > 0 ? (a.tiles + NT - 1) / NT : 1;
    const dim3 grid((unsigned)nwg), block(NT);
    if (sums && a.side) hipLaunchKernelGGL((k_stats<G, TIn, true, true>), grid, block, 0, st, a);
    else if (sums) hipLaunchKernelGGL((k_stats<G, TIn, true, false>), grid, block, 0, st, a);
    else if (a.side) hipLaunchKernelGGL((k_stats<G, TIn, false, true>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((k_stats<G, TIn, false, false>), grid, block, 0, st, a);
  }
  return hipGetLastError();
}

hipError_t launch_stats(const Plan& pl, const void* x, float* h_out, void* ws, bool init_select, uint8_t* side,
                        hipStream_t st) {
  uint8_t* w = static_cast<uint8_t*>(ws);
  StatsArgs a;
  a.x = static_cast<const uint8_t*>(x);
  a.h = h_out;
  a.side = side;
  a.tau = pl.tau;
  a.ls = reinterpret_cast<float2*>(w + pl.ws_LS);
  a.hist = reinterpret_cast<uint32_t*>(w + pl.ws_hist);
  a.tiles = pl.tiles;
  a.hist_words = init_select ? pl.nsamples * kBins : 0;
  a.init = init_select ? 1 : 0;
  const bool bf = pl.x_dtype == TAH_DTYPE_BF16, sums = pl.kA > 1;
  // every statistics workgroup takes 64 quantization tiles, from a multiple of
  // 64 (128 for allocation tiles of 128 rows of at most 128 bytes)
  const bool narrow = pl.G * (bf ? 2 : 4) <= 128;
  a.kA_fused = (sums && (64 % pl.kA == 0 || (pl.kA == 128 && narrow))) ? (int32_t)pl.kA : 0;
  hipError_t e;
  switch (pl.G) {
    case 32: e = bf ? launch_stats_t<32, bf16_t>(a, sums, st) : launch_stats_t<32, float>(a, sums, st); break;
    case 64: e = bf ? launch_stats_t<64, bf16_t>(a, sums, st) : launch_stats_t<64, float>(a, sums, st); break;
    case 128: e = bf ? launch_stats_t<128, bf16_t>(a, sums, st) : launch_stats_t<128, float>(a, sums, st); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess || !sums || a.kA_fused || pl.atiles == 0) return e;
  hipLaunchKernelGGL(k_alloc_entropy, dim3((unsigned)((pl.atiles + 255) / 256)), dim3(256), 0, st,
                     (const float2*)a.ls, h_out, pl.atiles, pl.kA);
  return hipGetLastError();
}

// ------------------------------------------------------------------ hist ----
struct HistArgs {
  const float* H;
  const SampleState* st_prev;  // state before the previous pass (unused on pass 0)
  SampleState* st_cur;         // state before this pass, written by each sample's first block
  const uint32_t* hist_prev;   // previous pass's histograms
  uint32_t* hist_cur;          // this pass's histograms (zero on entry)
  uint32_t* hist_clear;        // the next pass's histograms, cleared here
  uint32_t* cand;  // per sample: count, pad, then up to ncand (key, index) pairs
  // fold (last entropy pass only): the width map's sure bits and the count
  // of each run of 64 tiles
  uint32_t* fold_bitmap;
  uint32_t* fold_run;
  int64_t N, nsamples, chunks_per_sample, k, ncand, cand_stride;
  SelectPass pass, prev;
  int32_t has_prev, fold;
  int32_t kA;  // fold: quantization tiles per allocation tile (a power of two)
};

// Large workgroups of P keys per thread (a chunk of 1024 P keys each, whole
// runs of 64 tiles). The launch takes the smallest P in {1, 2, 4, 8} that
// keeps the grid within kHistMaxWgs workgroups: a million keys at P = 8 (128
// workgroups) add fewer partial histograms into the same global bins than at
// P = 4 (80/20 round trip at 8192 x 8192: 121.4 -> 120.8 us; P = 16 left most
// of the chip idle; P = 2 and 1 added too many global atomics: 125.3 -> 135.4
// us against P = 4), while 131,072 keys run best as 128 workgroups of P = 1
// (4096 x 2048 round trip: 45.5 us at P = 4, 42.8 at P = 2, 42.0 at P = 1).
constexpr int kHistThreads = 1024;
constexpr int64_t kHistMaxWgs = 128;

// Apply one pass to a sample's state: one wavefront finds the bin of the
// pass's histogram where the running count, bins in order (descending digits
// for the entropy key, ascending for the tile index), reaches r.
__device__ __forceinline__ SampleState apply_pass(SampleState S, const uint32_t* h, const SelectPass& ps) {
  if (ps.kind == 1 && S.tie_all) return S;
  uint32_t digit, cnt, before;
  // a sample holds fewer than 2^31 keys, so r and every count fit in 32 bits
  if (!find_rank<kBins>(h, ps.kind == 0, (uint32_t)S.r, digit, cnt, before))
    return S;  // rank beyond the histogram: cannot happen for 1 <= r <= count
  S.r -= (int64_t)before;
  if (ps.kind == 0) {
    S.key |= digit << ps.shift;
    if (ps.last_h) {
      S.tie_all = (S.r == (int64_t)cnt) ? 1 : 0;
      S.upos = S.tie_all ? 0xffffffffu : 0u;
    }
  } else {
    S.upos |= digit << ps.shift;
  }
  return S;
}

template <int P>
__global__ __launch_bounds__(kHistThreads) void k_hist(HistArgs a) {
  __shared__ __attribute__((aligned(16))) uint32_t lh[kBins];
  __shared__ SampleState ss;
  __shared__ uint2 lc[kCandPerChunk];  // candidates of the last entropy pass
  __shared__ uint32_t lcn, lbase;
  const int tid = threadIdx.x, lane = tid & 63;
  const int64_t s = blockIdx.x / a.chunks_per_sample;
  const int64_t c = blockIdx.x % a.chunks_per_sample;
  const int64_t u0 = c * (int64_t)(kHistThreads * P);
  // the keys first: their loads are in flight while the previous pass is applied
  float hv[P];
#pragma unroll
  for (int i = 0; i < P; ++i) {
    const int64_t u = u0 + i * kHistThreads + tid;
    hv[i] = u < a.N ? a.H[s * a.N + u] : 0.0f;
  }
  // the next pass's histogram of this sample, cleared in slices by the sample's blocks
  {
    const int64_t per = (kBins + a.chunks_per_sample - 1) / a.chunks_per_sample;
    const int64_t b0 = c * per, b1 = b0 + per < kBins ? b0 + per : kBins;
    for (int64_t i = b0 + tid; i < b1; i += kHistThreads) a.hist_clear[s * kBins + i] = 0u;
  }
  for (int i = tid; i < kBins; i += kHistThreads) lh[i] = 0u;
  if (tid == 0) lcn = 0u;
  if (tid < 64) {
    SampleState S;
    if (a.has_prev) {
      S = apply_pass(a.st_prev[s], a.hist_prev + s * kBins, a.prev);
    } else {
      S.key = 0u;
      S.upos = 0u;
      S.r = a.k;
      S.tie_all = 0;
      S.pad = 0;
    }
    if (tid == 0) {
      ss = S;
      if (c == 0) a.st_cur[s] = S;
      if (c == 0 && !a.has_prev) a.cand[s * a.cand_stride] = 0u;  // appended to by the last pass
    }
  }
  __syncthreads();
  const SampleState S = ss;
  const int hs = a.pass.shift + a.pass.width;  // bits above the current digit
  const uint32_t dmask = (1u << a.pass.width) - 1u;
#pragma unroll
  for (int i = 0; i < P; ++i) {
    const int64_t u = u0 + i * kHistThreads + tid;
    bool want = false;
    uint32_t digit = 0;
    if (u < a.N) {  // entropy-key digits only: tile-index digits run in k_resolve
      const uint32_t key = orderable(hv[i]);
      want = hs >= 32 || (key >> hs) == (S.key >> hs);
      digit = (key >> a.pass.shift) & dmask;
    }
    if (a.pass.last_h) {
      // the keys matching the prefix, a superset of the threshold's ties, into
      // this workgroup's LDS list (appended to the sample's list at the end)
      const uint64_t wm = ballot(want);
      if (wm != 0) {
        const int leader = __ffsll((unsigned long long)wm) - 1;
        uint32_t base = 0;
        if (lane == leader) base = atomicAdd(&lcn, (uint32_t)__popcll(wm));
        base = (uint32_t)__builtin_amdgcn_readlane((int)base, leader);
        const uint32_t pos = base + lanes_below(wm);
        if (want && pos < (uint32_t)kCandPerChunk) lc[pos] = make_uint2(orderable(hv[i]), (uint32_t)u);
      }
      if (a.fold) {
        // keys above the threshold's prefix are selected whatever the last
        // digit: the run's width-map words and count (the keys matching the
        // prefix are added by k_resolve); a wavefront's 64 keys are one run
        const bool sure = u < a.N && hs < 32 && (orderable(hv[i]) >> hs) > (S.key >> hs);
        const uint64_t m = ballot(sure);
        const int64_t ub = u0 + i * kHistThreads + (tid & ~63);
        if (ub < a.N) {
          if (a.kA == 1) {
            const int64_t run = (s * a.N + ub) >> 6;
            if (lane < 2) a.fold_bitmap[2 * run + lane] = (uint32_t)(m >> (32 * lane));
            if (lane == 0) a.fold_run[run] = (uint32_t)__popcll(m);
          } else {
            // the 64 allocation tiles are kA runs of 64 quantization tiles:
            // each allocation tile's bit kA times, and each run's count
            const int lk = __ffs(a.kA) - 1;
            const int64_t run0 = ((s * a.N + ub) << lk) >> 6;
            for (int wv = lane; wv < 2 * a.kA; wv += 64) {
              uint32_t word = 0u;
              if (lk >= 5) {  // a word inside one allocation tile
                word = ((m >> ((32 * wv) >> lk)) & 1ull) ? ~0u : 0u;
              } else {
#pragma unroll
                for (int bq = 0; bq < 32; ++bq) word |= (uint32_t)((m >> ((32 * wv + bq) >> lk)) & 1ull) << bq;
              }
              a.fold_bitmap[2 * run0 + wv] = word;
            }
            for (int rk = lane; rk < a.kA; rk += 64) {
              uint32_t cnt;
              if (lk >= 6) {  // a run inside one allocation tile
                cnt = ((m >> ((64 * rk) >> lk)) & 1ull) ? 64u : 0u;
              } else {
                const int per = 64 >> lk;  // allocation tiles per run
                cnt = (uint32_t)a.kA * (uint32_t)__popcll((m >> (rk * per)) & ((1ull << per) - 1ull));
              }
              a.fold_run[run0 + rk] = cnt;
            }
          }
        }
      }
    }
    // first digit (entropy keys cluster there): lanes with the same digit as
    // the first remaining lane add together (twice), the rest one by one; the
    // later digits spread over the bins, and every lane adds its own key
    // (80/20 round trip at 8192 x 8192: 114.0 -> 111.6 us)
#pragma unroll
    for (int round = 0; !a.has_prev && round < 2; ++round) {
      const uint64_t wm = ballot(want);
      if (wm == 0) break;
      const int leader = __ffsll((unsigned long long)wm) - 1;
      const uint32_t d0 = (uint32_t)__builtin_amdgcn_readlane((int)digit, leader);
      const bool same = want && digit == d0;
      const uint64_t sm = ballot(same);
      if (lane == leader) atomicAdd(&lh[d0], (uint32_t)__popcll(sm));
      want = want && !same;
    }
    if (want) atomicAdd(&lh[digit], 1u);
  }
  __syncthreads();
  for (int i = tid; i < kBins; i += kHistThreads)
    if (lh[i]) atomicAdd(&a.hist_cur[s * kBins + i], lh[i]);
  if (a.pass.last_h) {
    // one reservation in the sample's list per workgroup; a count above the
    // list's capacity (or a workgroup past kCandPerChunk) marks it overflowed
    const uint32_t n = lcn;
    if (n != 0) {
      uint32_t* cl = a.cand + s * a.cand_stride;
      // (ncand + 1 per overflowing workgroup keeps the sum below 2^32 for any N < 2^31)
      if (tid == 0) lbase = atomicAdd(cl, n > (uint32_t)kCandPerChunk ? (uint32_t)(a.ncand + 1) : n);
      __syncthreads();
      const uint32_t base = lbase;
      for (uint32_t i = tid; i < n && i < (uint32_t)kCandPerChunk; i += kHistThreads)
        if ((int64_t)(base + i) < a.ncand) reinterpret_cast<uint2*>(cl + 2)[base + i] = lc[i];
    }
  }
}

// One workgroup per sample: applies the last entropy pass, which fixes the
// k-th largest key K and the rank r still to place among the keys equal to K.
// When every tile with key K is selected (the usual case: entropies rarely
// tie) that is the final state. Otherwise the r-th lowest tile index among the
// keys equal to K is found here by digit passes over the sample's keys with an
// LDS histogram: one launch instead of one per index digit. The digit passes
// run over the (key, index) pairs that the last entropy pass listed (those
// matching the threshold's prefix: 871 of the 1048576 keys of the 8192 x 8192
// GeLU tensor); only when the list overflowed does this workgroup scan the
// whole sample.
struct ResolveArgs {
  const float* H;
  const SampleState* st_prev;
  SampleState* st_out;
  const uint32_t* hist_last;
  const uint32_t* cand;
  // fold: the selected tiles among those matching the threshold's prefix go
  // into the width map and the run counts, which are then scanned into the
  // block table
  uint32_t* fold_bitmap;
  const uint32_t* fold_run;
  uint32_t* table;
  int64_t N, ncand, cand_stride, k;
  SelectPass last;
  int32_t nidx, fold;
  int32_t kA;  // fold: quantization tiles per allocation tile
  SelectPass idx[kMaxPasses];
};

constexpr int kResolveThreads = 1024;

__global__ __launch_bounds__(kResolveThreads) void k_resolve(ResolveArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint32_t rc[];  // fold: the sample's run counts
  __shared__ __attribute__((aligned(16))) uint32_t lh[kBins];
  __shared__ SampleState ss;
  __shared__ uint2 lk[kMaxCand];  // the sample's candidate list
  __shared__ uint32_t wsum[kResolveThreads / 64];
  const int tid = threadIdx.x;
  const int64_t s = blockIdx.x;
  // fold: the sample's run counts, loaded first (in flight during the rest)
  constexpr int kRound = 4 * kResolveThreads;
  constexpr int kPer = (int)(kFoldMaxRuns / kResolveThreads);
  const int64_t runs = a.N * a.kA / 64, r0 = s * runs;
  const int nr = a.fold ? (int)((runs + kRound - 1) / kRound) : 0;
  uint32_t rv[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int64_t j = (int64_t)i * kResolveThreads + tid;
    rv[i] = 0u;
    if (i < 4 * nr && j < runs) rv[i] = a.fold_run[r0 + j];
  }
  // the listed pairs into LDS by the other wavefronts while the first one
  // applies the last pass
  const uint32_t* cl = a.cand + s * a.cand_stride;
  if (tid >= 64) {
    const int64_t nc0 = cl[0];
    if (nc0 <= a.ncand)
      for (int64_t i = tid - 64; i < nc0; i += kResolveThreads - 64) lk[i] = reinterpret_cast<const uint2*>(cl + 2)[i];
  }
  if (tid < 64) {
    const SampleState S = apply_pass(a.st_prev[s], a.hist_last + s * kBins, a.last);
    if (tid == 0) ss = S;
  }
  __syncthreads();
  SampleState S = ss;
  const float* h = a.H + s * a.N;
  const int64_t nc = cl[0];
  const bool listed = nc <= a.ncand;  // else scan the whole sample
  const int64_t n = listed ? nc : a.N;
  // Few tied keys (at most 64, listed): one wavefront gathers their tile
  // indexes and takes the r-th lowest directly, the same index the digit
  // passes below would find.
  __shared__ int few_done;
  if (!S.tie_all && listed) {
    if (tid < 64) {
      const int lane = tid;
      int cnt = 0;  // tied keys gathered so far (uniform)
      for (int64_t i0 = 0; i0 < nc && cnt <= 64; i0 += 64) {
        const int64_t i = i0 + lane;
        const bool tied = i < nc && lk[i].x == S.key;
        const uint64_t m = ballot(tied);
        const int pos = cnt + (int)lanes_below(m);
        if (tied && pos < 64) lh[pos] = lk[i].y;
        cnt += __popcll(m);
      }
      __threadfence_block();
      int ok = 0;
      if (cnt <= 64) {
        const uint32_t mine = lane < cnt ? lh[lane] : 0xffffffffu;
        int rank = 0;  // tied indexes below this one (indexes are unique)
        for (int j = 0; j < cnt; ++j) rank += (uint32_t)__shfl((int)mine, j, 64) < mine ? 1 : 0;
        const uint64_t hit = ballot(lane < cnt && (int64_t)rank == S.r - 1);
        if (hit != 0) {
          const int src = __ffsll((unsigned long long)hit) - 1;
          const uint32_t up = (uint32_t)__builtin_amdgcn_readlane((int)mine, src);
          if (lane == 0) {
            SampleState T = S;
            T.upos = up;
            T.r = 1;
            ss = T;
          }
          ok = 1;
        }
      }
      if (lane == 0) few_done = ok;
    }
    __syncthreads();
    if (few_done) S = ss;
  }
  if (!S.tie_all && !(listed && few_done)) {
    for (int p = 0; p < a.nidx; ++p) {
      const SelectPass ps = a.idx[p];
      for (int i = tid; i < kBins; i += kResolveThreads) lh[i] = 0u;
      __syncthreads();
      const int hs = ps.shift + ps.width;  // index bits above the current digit
      const uint32_t dmask = (1u << ps.width) - 1u;
      for (int64_t i = tid; i < n; i += kResolveThreads) {
        uint32_t key, uu;
        if (listed) {
          key = lk[i].x;
          uu = lk[i].y;
        } else {
          key = orderable(h[i]);
          uu = (uint32_t)i;
        }
        if (key == S.key && (hs >= 32 || (uu >> hs) == (S.upos >> hs)))
          atomicAdd(&lh[(uu >> ps.shift) & dmask], 1u);
      }
      __syncthreads();
      if (tid < 64) {
        const SampleState T = apply_pass(S, lh, ps);
        if (tid == 0) ss = T;
      }
      __syncthreads();
      S = ss;
    }
  }
  if (a.fold) {
    // the sample's run counts in LDS, plus the selected tiles among those
    // matching the threshold's prefix (the sure ones are counted already)
    // (an LDS array of nr times kRound counts, zero past the sample's runs)
#pragma unroll
    for (int i = 0; i < kPer; ++i)
      if (i < 4 * nr) rc[i * kResolveThreads + tid] = rv[i];
    __syncthreads();
    const int hs = a.last.shift + a.last.width;  // the prefix the last entropy pass matched
    for (int64_t i = tid; i < n; i += kResolveThreads) {
      uint32_t key, uu;
      if (listed) {
        key = lk[i].x;
        uu = lk[i].y;
      } else {
        key = orderable(h[i]);
        uu = (uint32_t)i;
      }
      if ((key >> hs) == (S.key >> hs) && (key > S.key || (key == S.key && uu <= S.upos))) {
        // the allocation tile's kA quantization tiles (kA divides 64: one
        // run, and one word unless kA = 64)
        const int64_t t = (s * a.N + uu) * a.kA;
        if (a.kA >= 32) {
          for (int wv = 0; wv < a.kA / 32; ++wv) atomicOr(&a.fold_bitmap[(t >> 5) + wv], ~0u);
        } else {
          atomicOr(&a.fold_bitmap[t >> 5], ((1u << a.kA) - 1u) << (t & 31));
        }
        if (a.kA >= 64) {
          for (int rk = 0; rk < a.kA / 64; ++rk) atomicAdd(&rc[(((int64_t)uu * a.kA) >> 6) + rk], 64u);
        } else {
          atomicAdd(&rc[((int64_t)uu * a.kA) >> 6], (uint32_t)a.kA);
        }
      }
    }
    __syncthreads();
    // block table: every earlier sample holds k upgraded tiles, then the
    // exclusive scan of this sample's run counts
    lds_scan_store<kResolveThreads, (int)(kFoldMaxRuns / kRound)>(
        rc, nr, (uint32_t)s * (uint32_t)a.k * (uint32_t)a.kA, a.table + r0, runs, wsum);
  }
  if (tid == 0) a.st_out[s] = S;
}

// Samples of at most kLdsSelect keys: one workgroup per sample holds the
// sample's order-preserving keys in LDS (dynamic shared memory, 4 bytes per
// key) and runs every digit pass of the select there, the three key digits and, when the
// threshold key is shared by more tiles than remain to be selected, the
// tile-index digits: the same passes and apply_pass as the grid-wide form, so
// the same final state, from one read of the keys and one launch instead of
// one launch per digit, k_resolve, k_mark and k_table. The limit is 4096
// keys, where the grid-wide passes run at most four workgroups per sample
// anyway: with 32768-key samples a workgroup per sample is
// latency-bound (32 dependent rounds per thread and pass) and the 4096 x 2048
// round trip took 76.1 us against 47.7 us grid-wide, with the keys in LDS as
// when they were re-read from global memory in every pass (78.2 us).
// When a sample covers whole runs of 64 quantization tiles, the same
// workgroup then writes the sample's width-map words and block-table entries:
// every sample has k upgraded allocation tiles, so the block table at the
// sample's first run is s * k * kA, and the runs inside the sample add their
// own counts. Otherwise it writes the final state for k_mark.
constexpr int64_t kLdsMarkRuns = 4096;
constexpr int kLdsThreads = 1024;

struct LdsSelectArgs {
  const float* H;
  SampleState* st_out;
  uint32_t* bitmap;  // width map (payload or workspace), fused marking only
  uint32_t* table;   // block table (payload or workspace), fused marking only
  int64_t N, k, kA;
  int32_t fused;
  int32_t npasses;
  SelectPass passes[kMaxPasses];
};

__global__ __launch_bounds__(kLdsThreads) void k_select_lds(LdsSelectArgs a) {
  extern __shared__ uint32_t keys[];  // the sample's N keys
  __shared__ __attribute__((aligned(16))) uint32_t lh[kBins];
  __shared__ SampleState ss;
  __shared__ uint32_t wsum[kLdsThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t s = blockIdx.x;
  {
    const float* h = a.H + s * a.N;
    int64_t i = tid;
    for (; i + 3 * kLdsThreads < a.N; i += 4 * kLdsThreads) {  // four loads in flight per thread
      const float h0 = h[i], h1 = h[i + kLdsThreads], h2 = h[i + 2 * kLdsThreads], h3 = h[i + 3 * kLdsThreads];
      keys[i] = orderable(h0);
      keys[i + kLdsThreads] = orderable(h1);
      keys[i + 2 * kLdsThreads] = orderable(h2);
      keys[i + 3 * kLdsThreads] = orderable(h3);
    }
    for (; i < a.N; i += kLdsThreads) keys[i] = orderable(h[i]);
  }
  if (tid == 0) {
    SampleState S;
    S.key = 0u;
    S.upos = 0u;
    S.r = a.k;
    S.tie_all = 0;
    S.pad = 0;
    ss = S;
  }
  for (int p = 0; p < a.npasses; ++p) {
    const SelectPass ps = a.passes[p];
    for (int i = tid; i < kBins; i += kLdsThreads) lh[i] = 0u;
    __syncthreads();
    const SampleState S = ss;
    if (ps.kind == 1 && S.tie_all) break;  // every tile with the threshold key is selected
    const int hs = ps.shift + ps.width;  // bits above the current digit
    const uint32_t dmask = (1u << ps.width) - 1u;
    for (int64_t i0 = 0; i0 < a.N; i0 += kLdsThreads) {  // uniform trip count: ballots need every lane
      const int64_t i = i0 + tid;
      bool want = false;
      uint32_t digit = 0;
      if (i < a.N) {
        const uint32_t key = keys[i];
        if (ps.kind == 0) {
          want = hs >= 32 || (key >> hs) == (S.key >> hs);
          digit = (key >> ps.shift) & dmask;
        } else {
          const uint32_t u = (uint32_t)i;
          want = key == S.key && (hs >= 32 || (u >> hs) == (S.upos >> hs));
          digit = (u >> ps.shift) & dmask;
        }
      }
      // first digit: lanes with the same digit as the first remaining lane
      // add together (twice: entropy keys cluster), the rest one by one
#pragma unroll
      for (int round = 0; p == 0 && round < 2; ++round) {
        const uint64_t wm = ballot(want);
        if (wm == 0) break;
        const int leader = __ffsll((unsigned long long)wm) - 1;
        const uint32_t d0 = (uint32_t)__builtin_amdgcn_readlane((int)digit, leader);
        const bool same = want && digit == d0;
        const uint64_t sm = ballot(same);
        if (lane == leader) atomicAdd(&lh[d0], (uint32_t)__popcll(sm));
        want = want && !same;
      }
      if (want) atomicAdd(&lh[digit], 1u);
    }
    __syncthreads();
    if (tid < 64) {
      const SampleState T = apply_pass(S, lh, ps);
      if (tid == 0) ss = T;
    }
    __syncthreads();
  }
  __syncthreads();
  const SampleState S = ss;
  if (!a.fused) {
    if (tid == 0) a.st_out[s] = S;
    return;
  }
  // width map and block table of the sample's runs of 64 quantization tiles;
  // lh holds each run's count, chunk by chunk
  const int64_t nb = a.N * a.kA / 64;  // runs in the sample
  const int64_t b0 = s * nb;           // the sample's first run in the tensor
  uint32_t carry = (uint32_t)s * (uint32_t)a.k * (uint32_t)a.kA;
  for (int64_t c0 = 0; c0 < nb; c0 += kLdsThreads) {
    const int64_t cn = nb - c0 < kLdsThreads ? nb - c0 : kLdsThreads;
    for (int64_t b = c0 + wave; b < c0 + cn; b += kLdsThreads / 64) {
      const int64_t u = (b * 64 + lane) / a.kA;  // the lane's allocation tile
      const uint32_t key = keys[u];
      const bool sel = key > S.key || (key == S.key && (uint32_t)u <= S.upos);
      const uint64_t m = ballot(sel);
      if (lane < 2) a.bitmap[2 * (b0 + b) + lane] = (uint32_t)(m >> (32 * lane));
      if (lane == 0) lh[b - c0] = (uint32_t)__popcll(m);
    }
    __syncthreads();
    // exclusive scan of the chunk's counts
    const uint32_t v = tid < cn ? lh[tid] : 0u;
    uint32_t incl = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const uint32_t o = __shfl_up(incl, off, 64);
      if (lane >= off) incl += o;
    }
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    uint32_t before = carry;
    for (int w = 0; w < wave; ++w) before += wsum[w];
    if (tid < cn) a.table[b0 + c0 + tid] = before + incl - v;
    for (int w = 0; w < kLdsThreads / 64; ++w) carry += wsum[w];
    __syncthreads();  // lh and wsum are reused by the next chunk
  }
}

// ------------------------------------------------------------------ mark ----
struct MarkArgs {
  const float* H;  // per allocation tile
  const SampleState* st;
  uint32_t* bitmap;
  uint32_t* blockcnt;
  int64_t tiles, N, nblocks, kA;
};

__global__ __launch_bounds__(256) void k_mark(MarkArgs a) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int64_t t = (int64_t)blockIdx.x * 256 + tid;
  bool sel = false;
  if (t < a.tiles) {
    const int64_t ta = a.kA == 1 ? t : t / a.kA;  // allocation tile
    const int64_t s = ta / a.N;
    const uint32_t u = (uint32_t)(ta - s * a.N);
    const uint32_t key = orderable(a.H[ta]);
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
constexpr int kScanPer = 8;  // counts per thread and step
constexpr int kScanStep = kScanThreads * kScanPer;

// Exclusive scan of the per-64-tile counts. Global memory is read and written
// coalesced (through an LDS copy of the step); each thread scans kScanPer
// consecutive counts, then the threads' totals are scanned across the block.
// total (may be null) receives the sum of all counts.
__global__ __launch_bounds__(kScanThreads) void k_table(const uint32_t* cnt, uint32_t* table, uint32_t* total,
                                                        int64_t nblocks) {
  __shared__ uint32_t buf[kScanStep];
  __shared__ uint32_t wsum[kScanThreads / 64];
  __shared__ uint32_t carry_s;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) carry_s = 0u;
  for (int64_t base = 0; base < nblocks; base += kScanStep) {
    uint32_t ld[kScanPer];
#pragma unroll
    for (int j = 0; j < kScanPer; ++j) {
      const int64_t i = base + j * kScanThreads + tid;
      ld[j] = i < nblocks ? cnt[i] : 0u;
    }
#pragma unroll
    for (int j = 0; j < kScanPer; ++j) buf[j * kScanThreads + tid] = ld[j];
    __syncthreads();
    uint32_t v[kScanPer];
    uint32_t tot = 0;
#pragma unroll
    for (int j = 0; j < kScanPer; ++j) {
      v[j] = buf[tid * kScanPer + j];
      tot += v[j];
    }
    uint32_t incl = tot;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const uint32_t o = __shfl_up(incl, off, 64);
      if (lane >= off) incl += o;
    }
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    uint32_t before = carry_s;
    for (int w = 0; w < wave; ++w) before += wsum[w];
    uint32_t run = before + incl - tot;
#pragma unroll
    for (int j = 0; j < kScanPer; ++j) {
      buf[tid * kScanPer + j] = run;
      run += v[j];
    }
    __syncthreads();
    if (tid == kScanThreads - 1) carry_s = run;
#pragma unroll
    for (int j = 0; j < kScanPer; ++j) {
      const int64_t i = base + j * kScanThreads + tid;
      if (i < nblocks) table[i] = buf[j * kScanThreads + tid];
    }
    __syncthreads();
  }
  if (total && tid == 0) *total = carry_s;
}

hipError_t launch_table(const uint32_t* cnt, uint32_t* table, uint32_t* total, int64_t nblocks, hipStream_t st) {
  hipLaunchKernelGGL(k_table, dim3(1), dim3(kScanThreads), 0, st, cnt, table, total, nblocks);
  return hipGetLastError();
}

// Width map and per-64-tile counts from the final states, then the block table.
static hipError_t mark_and_table(const Plan& pl, uint8_t* P, uint8_t* w, const SampleState* st_final, hipStream_t st) {
  MarkArgs m;
  m.H = reinterpret_cast<const float*>(w + pl.ws_H);
  m.st = st_final;
  m.bitmap = reinterpret_cast<uint32_t*>(P ? P + pl.off_bitmap : w + pl.ws_bitmap);
  m.blockcnt = reinterpret_cast<uint32_t*>(w + pl.ws_blockcnt);
  m.tiles = pl.tiles;
  m.N = pl.N;
  m.nblocks = pl.nblocks;
  m.kA = pl.kA;
  hipLaunchKernelGGL(k_mark, dim3((unsigned)((pl.tiles + 255) / 256)), dim3(256), 0, st, m);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  uint32_t* table = reinterpret_cast<uint32_t*>(P ? P + pl.off_table : w + pl.ws_table);
  return launch_table(m.blockcnt, table, nullptr, pl.nblocks, st);
}

hipError_t launch_select(const Plan& pl, void* payload, void* ws, hipStream_t st) {
  uint8_t* w = static_cast<uint8_t*>(ws);
  uint8_t* P = static_cast<uint8_t*>(payload);
  SampleState* states = reinterpret_cast<SampleState*>(w + pl.ws_state);
  if (pl.N <= kLdsSelect) {
    LdsSelectArgs sa;
    sa.H = reinterpret_cast<const float*>(w + pl.ws_H);
    sa.st_out = states;
    sa.bitmap = reinterpret_cast<uint32_t*>(P ? P + pl.off_bitmap : w + pl.ws_bitmap);
    sa.table = reinterpret_cast<uint32_t*>(P ? P + pl.off_table : w + pl.ws_table);
    sa.N = pl.N;
    sa.k = pl.k;
    sa.kA = pl.kA;
    // samples of whole runs of 64 tiles, few enough runs for one workgroup
    // (token-level allocation of a large tensor marks grid-wide)
    sa.fused = ((pl.N * pl.kA) % 64 == 0 && pl.N * pl.kA / 64 <= kLdsMarkRuns) ? 1 : 0;
    static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(k_select_lds),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                                       (int)(4 * kLdsSelect));
    if (attr != hipSuccess) return attr;
    sa.npasses = pl.npasses;
    for (int i = 0; i < kMaxPasses; ++i) sa.passes[i] = pl.passes[i];
    hipLaunchKernelGGL(k_select_lds, dim3((unsigned)pl.nsamples), dim3(kLdsThreads), (size_t)(4 * pl.N), st, sa);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess || sa.fused) return e;
    return mark_and_table(pl, P, w, states, st);
  }
  uint32_t* hists = reinterpret_cast<uint32_t*>(w + pl.ws_hist);
  const int64_t hsz = pl.nsamples * kBins;
  HistArgs h;
  h.H = reinterpret_cast<const float*>(w + pl.ws_H);
  h.N = pl.N;
  h.nsamples = pl.nsamples;
  h.k = pl.k;
  int per = 1;  // keys per thread
  while (per < 8 && pl.nsamples * ((pl.N + kHistThreads * per - 1) / (kHistThreads * per)) > kHistMaxWgs) per *= 2;
  const int64_t chunk = (int64_t)kHistThreads * per;
  h.chunks_per_sample = (pl.N + chunk - 1) / chunk;
  h.cand = reinterpret_cast<uint32_t*>(w + pl.ws_cand);
  h.ncand = pl.ncand;
  h.cand_stride = pl.cand_stride;
  h.fold_bitmap = reinterpret_cast<uint32_t*>(P ? P + pl.off_bitmap : w + pl.ws_bitmap);
  h.fold_run = reinterpret_cast<uint32_t*>(w + pl.ws_blockcnt);
  // the fold also covers allocation tiles of kA quantization tiles when kA
  // divides 64 and samples are whole runs of 64 allocation tiles
  const bool fold_wide = pl.mode == 1 && pl.kA > 1 && (pl.kA & (pl.kA - 1)) == 0 && pl.N % 64 == 0 &&
                         pl.N > kLdsSelect && pl.N * pl.kA / 64 <= kFoldMaxRuns;
  const bool fold = pl.fold || fold_wide;
  h.kA = fold_wide ? (int32_t)pl.kA : 1;
  const int64_t nwg = h.chunks_per_sample * pl.nsamples;
  // entropy-key passes; pass p: state p in states[p % 2], histogram p in
  // hists[p % 3] (zeroed by k_stats for p = 0). The tile-index passes that
  // follow them in the plan run inside k_resolve.
  int nkey = 0;
  while (nkey < pl.npasses && pl.passes[nkey].kind == 0) ++nkey;
  for (int p = 0; p < nkey; ++p) {
    h.pass = pl.passes[p];
    h.has_prev = p > 0;
    h.prev = p > 0 ? pl.passes[p - 1] : pl.passes[p];
    h.st_prev = states + ((p + 1) % 2) * pl.nsamples;
    h.st_cur = states + (p % 2) * pl.nsamples;
    h.hist_prev = hists + ((p + 2) % 3) * hsz;
    h.hist_cur = hists + (p % 3) * hsz;
    h.hist_clear = hists + ((p + 1) % 3) * hsz;
    h.fold = fold && h.pass.last_h;
    if (per == 1) hipLaunchKernelGGL(k_hist<1>, dim3((unsigned)nwg), dim3(kHistThreads), 0, st, h);
    else if (per == 2) hipLaunchKernelGGL(k_hist<2>, dim3((unsigned)nwg), dim3(kHistThreads), 0, st, h);
    else if (per == 4) hipLaunchKernelGGL(k_hist<4>, dim3((unsigned)nwg), dim3(kHistThreads), 0, st, h);
    else hipLaunchKernelGGL(k_hist<8>, dim3((unsigned)nwg), dim3(kHistThreads), 0, st, h);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // the final state goes to states[nkey % 2]
  ResolveArgs rs;
  rs.H = h.H;
  rs.st_prev = states + ((nkey + 1) % 2) * pl.nsamples;
  rs.st_out = states + (nkey % 2) * pl.nsamples;
  rs.hist_last = hists + ((nkey + 2) % 3) * hsz;
  rs.cand = h.cand;
  rs.N = pl.N;
  rs.ncand = pl.ncand;
  rs.cand_stride = pl.cand_stride;
  rs.last = pl.passes[nkey - 1];
  rs.nidx = pl.npasses - nkey;
  for (int i = 0; i < rs.nidx; ++i) rs.idx[i] = pl.passes[nkey + i];
  rs.fold_bitmap = h.fold_bitmap;
  rs.fold_run = h.fold_run;
  rs.table = reinterpret_cast<uint32_t*>(P ? P + pl.off_table : w + pl.ws_table);
  rs.k = pl.k;
  rs.fold = fold;
  rs.kA = h.kA;
  static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(k_resolve),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                                     (int)(4 * kFoldMaxRuns));
  if (attr != hipSuccess) return attr;
  // the run counts in whole rounds of 4 per thread
  const int64_t rc_round = 4 * kResolveThreads;
  const int64_t nruns = pl.N * h.kA / 64;
  const size_t rc_bytes = fold ? (size_t)(4 * ((nruns + rc_round - 1) / rc_round) * rc_round) : 0;
  hipLaunchKernelGGL(k_resolve, dim3((unsigned)pl.nsamples), dim3(kResolveThreads), rc_bytes, st, rs);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || fold) return e;  // fold: width map and block table are complete
  return mark_and_table(pl, P, w, rs.st_out, st);
}

}  // namespace tah
