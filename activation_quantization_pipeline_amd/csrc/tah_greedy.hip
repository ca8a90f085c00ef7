// Greedy bit allocation over every candidate width for gfx950 (the allocator
// TAH_ALLOC_GREEDY of tah.h). The pages rank a sample's tiles by entropy and
// give the top p% the higher of two widths (TAH-Quant §3.2); for more widths
// this allocator takes upgrades c_j -> c_(j+1) in order of their gain per bit,
// whose log2 is kappa = 2 H_u + lambda_j, while the sample's R bits last.
//
// The upgrades taken form a prefix of the order (kappa descending, tile index
// ascending, j ascending), so the allocation is fixed by its first upgrade
// that does not fit, e*. Each upgrade is one 64-bit composite: the 32-bit
// order-preserving key of kappa above the complemented upgrade index
// u * nl + j; composites are unique and a larger one comes first. e* is the
// composite where the running cost first exceeds R, found by a radix select
// whose histograms add each upgrade's cost instead of 1:
//   k_ghist  - one launch per digit of the 32-bit key (11/11/10 bits). Each
//              workgroup applies the previous digit (one wavefront scans that
//              histogram of the sample, descending, and finds the bin where
//              the running cost reaches r = remaining budget + 1), then adds
//              the costs of the upgrades that match the prefix into a
//              2048-bin LDS histogram and into the sample's global one. The
//              last digit also lists the (key, index) pairs that match the
//              22-bit prefix. Histograms rotate over three buffers and states
//              over two, so kernel boundaries are the only synchronisation;
//   k_gresolve - one workgroup per sample applies the last key digit, then
//              finds e*'s index among the upgrades with e*'s key by digit
//              passes over that list, ascending, in LDS: e*'s composite;
//   k_glevel - one lane per quantization tile: its level is the count of its
//              allocation tile's upgrades whose composite is above e*'s; the
//              2-bit level map and the sum of the widths per 64 tiles;
//   k_table  - (tah_select.hip) exclusive scan of those sums: the block table,
//              which locates every code block, and the total width (the used
//              part of the code section).
// When no upgrade or every upgrade fits (R = 0, one candidate, or R covering
// all of them) the select is skipped and every tile takes the same level; a
// sample of at most kGSmall upgrades is selected by one workgroup
// (k_gselect_small) in one launch.
#include "tah_device.hpp"
#include "tah_internal.hpp"
#include "tah_scan.hpp"

namespace tah {

// fp32 -> uint32 with the same order (keys are finite).
__device__ __forceinline__ uint32_t key_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

struct GArgs {
  const float* H;  // entropy per allocation tile
  int64_t N;       // allocation tiles per sample
  int32_t nl, ib;  // upgrades per tile, index bits of the composite
  float lam[3];    // lambda_j
  int32_t cost[3]; // c_(j+1) - c_j
};

// Upgrade j of tile u of a sample: kappa = 2 H_u + lambda_j in fp32 (2 H_u is
// exact, so a fused multiply-add rounds the same), above the complemented index.
__device__ __forceinline__ uint64_t composite(const GArgs& g, float h, int64_t u, int j) {
  const float kappa = 2.0f * h + g.lam[j];
  const uint64_t imax = (1ull << g.ib) - 1ull;
  const uint64_t idx = (uint64_t)u * (uint64_t)g.nl + (uint64_t)j;
  return ((uint64_t)key_bits(kappa) << g.ib) | (imax - idx);
}

// One wavefront: finds the bin of histogram h that holds cost position r
// (1-based), bins taken in descending order (DESC, composite digits) or
// ascending (index digits); returns its digit and the cost before it. r never
// exceeds the histogram's total: the host runs the select only when R is
// below the cost of all upgrades.
template <bool DESC>
__device__ __forceinline__ void find_bin(const uint32_t* h, int64_t r, uint32_t& digit, int64_t& before_out) {
  // the plan keeps a sample's cost of all upgrades below 2^32, so r and every
  // partial sum of a histogram fit in 32 bits
  uint32_t cnt, before = 0;
  if (r < 1 || r > (int64_t)0xffffffff || !find_rank<kBins>(h, DESC, (uint32_t)r, digit, cnt, before)) {
    digit = 0u;  // cannot happen for 1 <= r <= total
    before = 0u;
  }
  before_out = (int64_t)before;
}

// Narrows a sample's state to the bin of a composite digit.
__device__ __forceinline__ GState apply_gpass(GState S, const uint32_t* h, const GPass& ps) {
  uint32_t digit;
  int64_t before;
  find_bin<true>(h, S.r, digit, before);
  S.r -= before;
  S.prefix |= (uint64_t)digit << ps.shift;
  return S;
}

// ------------------------------------------------------------------ hist ----
struct GHistArgs {
  GArgs g;
  const GState* st_prev;      // state before the previous pass (unused on pass 0)
  GState* st_cur;             // state before this pass, written by each sample's first block
  const uint32_t* hist_prev;  // previous pass's histograms
  uint32_t* hist_cur;         // this pass's histograms (zero on entry)
  uint32_t* hist_clear;       // the next pass's histograms, cleared here
  uint32_t* cand;  // per sample: count, pad, then up to ncand (key, index) pairs
  // fold (last key digit, one sample): each tile's level from the upgrades
  // whose key lies above the 22-bit prefix, the 2-bit level map and each
  // run's width sum; the upgrades that match the prefix are added by k_gresolve
  uint32_t* fold_map;
  uint32_t* fold_run;
  int64_t chunks_per_sample, R, ncand, cand_stride;
  GPass pass, prev;
  int32_t has_prev, last_key;  // last_key: the last of the three key digits
  int32_t fold;
  uint32_t cands;  // candidate widths, one byte each, c_1 lowest
};

// P tiles per thread (a chunk of 1024 P allocation tiles per workgroup), the
// smallest P in {1, 2, 4} that keeps the grid within kGMaxWgs workgroups: a
// million tiles at P = 4 fill the chip (with five grid-wide digits, 16 per
// thread ran 29 us slower on an 8192 x 8192 tensor; 2 and 1 per thread, 15
// and 43 us slower), while the four samples of 32,768 tiles of the 4096 x 2048
// tensor take 128 workgroups at P = 1.
constexpr int kGThreads = 1024;
constexpr int64_t kGMaxWgs = 256;

template <int P>
__global__ __launch_bounds__(kGThreads) void k_ghist(GHistArgs a) {
  __shared__ __attribute__((aligned(16))) uint32_t lh[kBins];
  __shared__ GState ss;
  __shared__ uint2 lc[kCandPerChunk];  // candidates of the last key digit
  __shared__ uint32_t lcn, lbase;
  const int tid = threadIdx.x, lane = tid & 63;
  const int64_t s = blockIdx.x / a.chunks_per_sample;
  const int64_t c = blockIdx.x % a.chunks_per_sample;
  const int64_t u0 = c * (int64_t)(kGThreads * P);
  {  // the next pass's histogram of this sample, cleared in slices by the sample's blocks
    const int64_t per = (kBins + a.chunks_per_sample - 1) / a.chunks_per_sample;
    const int64_t b0 = c * per, b1 = b0 + per < kBins ? b0 + per : kBins;
    for (int64_t i = b0 + tid; i < b1; i += kGThreads) a.hist_clear[s * kBins + i] = 0u;
  }
  for (int i = tid; i < kBins; i += kGThreads) lh[i] = 0u;
  if (tid == 0) lcn = 0u;
  if (tid < 64) {
    GState S;
    if (a.has_prev) {
      S = apply_gpass(a.st_prev[s], a.hist_prev + s * kBins, a.prev);
    } else {
      S.prefix = 0ull;
      S.r = a.R + 1;  // the first upgrade whose running cost exceeds R
    }
    if (tid == 0) {
      ss = S;
      if (c == 0) a.st_cur[s] = S;
      if (c == 0 && !a.has_prev) a.cand[s * a.cand_stride] = 0u;  // appended to by the last key digit
    }
  }
  __syncthreads();
  const GState S = ss;
  const int hs = a.pass.shift + a.pass.width;  // composite bits above the current digit
  const uint64_t dmask = (1ull << a.pass.width) - 1ull;
  const uint64_t want_hi = hs >= 64 ? 0ull : (S.prefix >> hs);
  float hv[P];  // all loads in flight before the first use
#pragma unroll
  for (int i = 0; i < P; ++i) {
    const int64_t u = u0 + i * kGThreads + tid;
    hv[i] = u < a.g.N ? a.g.H[s * a.g.N + u] : 0.0f;
  }
  int lv[P];  // fold: upgrades of the tile above the prefix
#pragma unroll
  for (int i = 0; i < P; ++i) lv[i] = 0;
  for (int j = 0; j < a.g.nl; ++j) {
    const uint32_t cost = (uint32_t)a.g.cost[j];
#pragma unroll
    for (int i = 0; i < P; ++i) {
      const int64_t u = u0 + i * kGThreads + tid;
      bool want = false;
      uint32_t digit = 0;
      uint64_t C = 0;
      if (u < a.g.N) {
        C = composite(a.g, hv[i], u, j);
        want = hs >= 64 || (C >> hs) == want_hi;
        digit = (uint32_t)((C >> a.pass.shift) & dmask);
        if (a.fold && hs < 64 && (C >> hs) > want_hi) ++lv[i];
      }
      if (a.last_key) {
        // upgrades whose key matches the prefix, a superset of the ties at
        // e*'s key, into this workgroup's LDS list (appended to the sample's
        // list at the end): (key, index)
        const uint64_t wm = ballot(want);
        if (wm != 0) {
          const int leader = __ffsll((unsigned long long)wm) - 1;
          uint32_t base = 0;
          if (lane == leader) base = atomicAdd(&lcn, (uint32_t)__popcll(wm));
          base = (uint32_t)__shfl((int)base, leader, 64);
          const uint32_t pos = base + lanes_below(wm);
          if (want && pos < (uint32_t)kCandPerChunk)
            lc[pos] = make_uint2((uint32_t)(C >> a.g.ib), (uint32_t)((uint64_t)u * (uint64_t)a.g.nl + (uint64_t)j));
        }
      }
      // first digit: lanes with the same digit as the first remaining lane
      // add together (twice), the rest one by one (later digits spread)
#pragma unroll
      for (int round = 0; !a.has_prev && round < 2; ++round) {
        const uint64_t wm = ballot(want);
        if (wm == 0) break;
        const int leader = __ffsll((unsigned long long)wm) - 1;
        const uint32_t d0 = (uint32_t)__shfl((int)digit, leader, 64);
        const bool same = want && digit == d0;
        const uint64_t sm = ballot(same);
        if (lane == leader) atomicAdd(&lh[d0], (uint32_t)__popcll(sm) * cost);
        want = want && !same;
      }
      if (want) atomicAdd(&lh[digit], cost);
    }
  }
  if (a.fold) {
    // a wavefront's 64 tiles are one run: its level-map words and width sum
    // (one sample, so the tile index is the upgrade's tile index)
#pragma unroll
    for (int i = 0; i < P; ++i) {
      const int64_t ub = u0 + i * kGThreads + (tid & ~63);
      if (ub < a.g.N) {
        const bool in = ub + lane < a.g.N;
        const int l = in ? lv[i] : 0;
        uint32_t f = (uint32_t)l << (2 * (lane & 15));
#pragma unroll
        for (int off = 1; off < 16; off <<= 1) f |= (uint32_t)__shfl_xor((int)f, off, 64);
        int w = in ? (int)((a.cands >> (8 * l)) & 255u) : 0;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) w += __shfl_xor(w, off, 64);
        const int64_t run = ub >> 6;
        if ((lane & 15) == 0) a.fold_map[4 * run + (lane >> 4)] = f;
        if (lane == 0) a.fold_run[run] = (uint32_t)w;
      }
    }
  }
  __syncthreads();
  for (int i = tid; i < kBins; i += kGThreads)
    if (lh[i]) atomicAdd(&a.hist_cur[s * kBins + i], lh[i]);
  if (a.last_key) {
    // one reservation in the sample's list per workgroup; a count above the
    // list's capacity (or a workgroup past kCandPerChunk) marks it overflowed
    const uint32_t n = lcn;
    if (n != 0) {
      uint32_t* cl = a.cand + s * a.cand_stride;
      if (tid == 0) lbase = atomicAdd(cl, n > (uint32_t)kCandPerChunk ? (uint32_t)(a.ncand + 1) : n);
      __syncthreads();
      const uint32_t base = lbase;
      for (uint32_t i = tid; i < n && i < (uint32_t)kCandPerChunk; i += kGThreads)
        if ((int64_t)(base + i) < a.ncand) reinterpret_cast<uint2*>(cl + 2)[base + i] = lc[i];
    }
  }
}

// One workgroup per sample: applies the last key digit, which fixes e*'s key
// K and the cost position r still to place among the upgrades with key K;
// then e*'s upgrade index (the lowest index first among equal keys) by
// cost-weighted digit passes over an LDS histogram, ascending. The passes run
// over the (key, index) pairs the last key digit listed (those matching the
// 22-bit key prefix, usually a few thousand at most); only when that list
// overflowed does this workgroup go through every upgrade of the sample.
struct GResolveArgs {
  GArgs g;
  const GState* st_prev;
  GState* st_out;
  const uint32_t* hist_last;
  const uint32_t* cand;
  // fold (one sample): the selected upgrades among those matching the 22-bit
  // key prefix raise their tile's level and their run's width sum, which are
  // then scanned into the block table and the total width
  uint32_t* fold_map;
  const uint32_t* fold_run;
  uint32_t* table;
  uint32_t* wtotal;
  int64_t ncand, cand_stride;
  GPass last;
  int32_t nidx, fold;
  GPass idx[3];  // digits of the upgrade index, top first
};

constexpr int kGResolveThreads = 1024;

__global__ __launch_bounds__(kGResolveThreads) void k_gresolve(GResolveArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint32_t rs[];  // fold: the run width sums
  __shared__ uint32_t wsum[kGResolveThreads / 64];
  __shared__ __attribute__((aligned(16))) uint32_t lh[kBins];
  __shared__ GState ss;
  __shared__ uint32_t ipre_s;
  __shared__ uint2 lk[kMaxCand];
  const int tid = threadIdx.x;
  const int64_t s = blockIdx.x;
  // the listed pairs into LDS by the other wavefronts while the first one
  // applies the last key digit
  const uint32_t* cl = a.cand + s * a.cand_stride;
  if (tid >= 64) {
    const int64_t nc0 = cl[0];
    if (nc0 <= a.ncand)
      for (int64_t i = tid - 64; i < nc0; i += kGResolveThreads - 64)
        lk[i] = reinterpret_cast<const uint2*>(cl + 2)[i];
  }
  if (tid < 64) {
    const GState S = apply_gpass(a.st_prev[s], a.hist_last + s * kBins, a.last);
    if (tid == 0) {
      ss = S;
      ipre_s = 0u;
    }
  }
  __syncthreads();
  const GState S = ss;
  const uint32_t K = (uint32_t)(S.prefix >> a.g.ib);
  int64_t r = S.r;
  const int64_t nc = cl[0];
  const bool listed = nc <= a.ncand;  // else go through every upgrade of the sample
  const int64_t n = listed ? nc : a.g.N * a.g.nl;
  const float* h = a.g.H + s * a.g.N;
  // At most 64 listed upgrades with e*'s key: one wavefront gathers them and
  // takes e* directly, the upgrade whose running cost in index order (lowest
  // first) reaches r, the same upgrade the digit passes below would find.
  __shared__ int few_done;
  if (listed) {
    if (tid < 64) {
      const int lane = tid;
      int cnt = 0;  // upgrades with key K gathered so far (uniform)
      for (int64_t i0 = 0; i0 < nc && cnt <= 64; i0 += 64) {
        const int64_t i = i0 + lane;
        const bool tied = i < nc && lk[i].x == K;
        const uint64_t m = ballot(tied);
        const int pos = cnt + (int)lanes_below(m);
        if (tied && pos < 64) lh[pos] = lk[i].y;
        cnt += __popcll(m);
      }
      __threadfence_block();
      int ok = 0;
      if (cnt <= 64) {
        const uint32_t mine = lane < cnt ? lh[lane] : 0xffffffffu;
        const int64_t cost = lane < cnt ? (int64_t)a.g.cost[mine % (uint32_t)a.g.nl] : 0;
        int64_t before = 0;  // cost of the tied upgrades with a lower index
        for (int j = 0; j < cnt; ++j) {
          const uint32_t o = (uint32_t)__shfl((int)mine, j, 64);
          if (o < mine) before += (int64_t)a.g.cost[o % (uint32_t)a.g.nl];
        }
        const uint64_t hit = ballot(lane < cnt && before < r && r <= before + cost);
        if (hit != 0) {
          const int src = __ffsll((unsigned long long)hit) - 1;
          const uint32_t e = (uint32_t)__builtin_amdgcn_readlane((int)mine, src);
          const int64_t b = (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(before >> 32), src) << 32) |
                                      (uint32_t)__builtin_amdgcn_readlane((int)before, src));
          r -= b;
          if (lane == 0) ipre_s = e;
          ok = 1;
        }
      }
      if (lane == 0) few_done = ok;
    }
    __syncthreads();
  }
  const bool skip_idx = listed && few_done;
  for (int p = 0; p < (skip_idx ? 0 : a.nidx); ++p) {
    const GPass ps = a.idx[p];
    for (int i = tid; i < kBins; i += kGResolveThreads) lh[i] = 0u;
    __syncthreads();
    const uint32_t ipre = ipre_s;
    const int hs = ps.shift + ps.width;  // index bits above the current digit
    const uint32_t dmask = (1u << ps.width) - 1u;
    for (int64_t i = tid; i < n; i += kGResolveThreads) {
      uint32_t key, idx;
      if (listed) {
        key = lk[i].x;
        idx = lk[i].y;
      } else {
        const int64_t u = i / a.g.nl;
        const int j = (int)(i - u * a.g.nl);
        key = (uint32_t)(composite(a.g, h[u], u, j) >> a.g.ib);
        idx = (uint32_t)i;
      }
      if (key == K && (hs >= 32 || (idx >> hs) == (ipre >> hs)))
        atomicAdd(&lh[(idx >> ps.shift) & dmask], (uint32_t)a.g.cost[idx % (uint32_t)a.g.nl]);
    }
    __syncthreads();
    if (tid < 64) {
      uint32_t digit;
      int64_t before;
      find_bin<false>(lh, r, digit, before);
      if (tid == 0) ipre_s = ipre | (digit << ps.shift);
      r -= before;  // only wavefront 0's r is used
    }
    __syncthreads();
  }
  if (a.fold) {
    // run width sums in LDS (kRound per round, zero past the runs), then the
    // selected upgrades that match the prefix; e* itself is not selected
    constexpr int kRound = 4 * kGResolveThreads;
    constexpr int kPer = (int)(kFoldMaxRuns / kGResolveThreads);
    const int64_t runs = (a.g.N + 63) / 64;
    const int nr = (int)((runs + kRound - 1) / kRound);
    {
      uint32_t v[kPer];
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        const int64_t j = (int64_t)i * kGResolveThreads + tid;
        v[i] = 0u;
        if (i < 4 * nr && j < runs) v[i] = a.fold_run[j];
      }
#pragma unroll
      for (int i = 0; i < kPer; ++i)
        if (i < 4 * nr) rs[i * kGResolveThreads + tid] = v[i];
    }
    __syncthreads();
    const uint32_t ip = ipre_s;
    for (int64_t i = tid; i < n; i += kGResolveThreads) {
      uint32_t key, idx;
      if (listed) {
        key = lk[i].x;
        idx = lk[i].y;
      } else {
        const int64_t u = i / a.g.nl;
        const int j = (int)(i - u * a.g.nl);
        key = (uint32_t)(composite(a.g, h[u], u, j) >> a.g.ib);
        idx = (uint32_t)i;
      }
      if ((key >> 10) == (K >> 10) && (key > K || (key == K && idx < ip))) {
        const uint32_t u = idx / (uint32_t)a.g.nl;
        atomicAdd(&a.fold_map[u >> 4], 1u << (2 * (u & 15)));
        atomicAdd(&rs[u >> 6], (uint32_t)a.g.cost[idx - u * (uint32_t)a.g.nl]);
      }
    }
    __syncthreads();
    const uint32_t total = lds_scan_store<kGResolveThreads, (int)(kFoldMaxRuns / kRound)>(rs, nr, 0u, a.table, runs, wsum);
    if (tid == 0) *a.wtotal = total;
  }
  if (tid == 0) {
    GState T;
    T.prefix = ((uint64_t)K << a.g.ib) | (((1ull << a.g.ib) - 1ull) - (uint64_t)ipre_s);
    T.r = r;
    a.st_out[s] = T;
  }
}

// Samples of at most kGSmall upgrades: one workgroup per sample runs the three
// key digits and the index digits of the select in LDS (the same composites,
// costs and find_bin as k_ghist and k_gresolve) in one launch. Up to this size
// the grid-wide digits would run one workgroup per sample as well.
constexpr int64_t kGSmall = 4096;

struct GSmallArgs {
  GArgs g;
  GState* st_out;
  int64_t R;
  GPass key[3];
  int32_t nidx;
  GPass idx[3];
};

__global__ __launch_bounds__(kGThreads) void k_gselect_small(GSmallArgs a) {
  __shared__ __attribute__((aligned(16))) uint32_t lh[kBins];
  __shared__ GState ss;
  __shared__ uint32_t ipre_s;
  const int tid = threadIdx.x, lane = tid & 63;
  const int64_t s = blockIdx.x;
  const float* h = a.g.H + s * a.g.N;
  if (tid == 0) {
    GState S;
    S.prefix = 0ull;
    S.r = a.R + 1;  // the first upgrade whose running cost exceeds R
    ss = S;
    ipre_s = 0u;
  }
  // key digits: descending composites, each upgrade adds its cost
  for (int p = 0; p < 3; ++p) {
    const GPass ps = a.key[p];
    for (int i = tid; i < kBins; i += kGThreads) lh[i] = 0u;
    __syncthreads();
    const GState S = ss;
    const int hs = ps.shift + ps.width;
    const uint64_t dmask = (1ull << ps.width) - 1ull;
    const uint64_t want_hi = hs >= 64 ? 0ull : (S.prefix >> hs);
    for (int j = 0; j < a.g.nl; ++j) {
      const uint32_t cost = (uint32_t)a.g.cost[j];
      for (int64_t u0 = 0; u0 < a.g.N; u0 += kGThreads) {  // uniform trip count: ballots need every lane
        const int64_t u = u0 + tid;
        bool want = false;
        uint32_t digit = 0;
        if (u < a.g.N) {
          const uint64_t C = composite(a.g, h[u], u, j);
          want = hs >= 64 || (C >> hs) == want_hi;
          digit = (uint32_t)((C >> ps.shift) & dmask);
        }
#pragma unroll
        for (int round = 0; p == 0 && round < 2; ++round) {  // first digit only, as in k_ghist
          const uint64_t wm = ballot(want);
          if (wm == 0) break;
          const int leader = __ffsll((unsigned long long)wm) - 1;
          const uint32_t d0 = (uint32_t)__shfl((int)digit, leader, 64);
          const bool same = want && digit == d0;
          const uint64_t sm = ballot(same);
          if (lane == leader) atomicAdd(&lh[d0], (uint32_t)__popcll(sm) * cost);
          want = want && !same;
        }
        if (want) atomicAdd(&lh[digit], cost);
      }
    }
    __syncthreads();
    if (tid < 64) {
      const GState T = apply_gpass(S, lh, ps);
      if (tid == 0) ss = T;
    }
    __syncthreads();
  }
  // index digits among the upgrades with e*'s key, ascending
  const uint32_t K = (uint32_t)(ss.prefix >> a.g.ib);
  int64_t r = ss.r;
  for (int p = 0; p < a.nidx; ++p) {
    const GPass ps = a.idx[p];
    for (int i = tid; i < kBins; i += kGThreads) lh[i] = 0u;
    __syncthreads();
    const uint32_t ipre = ipre_s;
    const int hs = ps.shift + ps.width;
    const uint32_t dmask = (1u << ps.width) - 1u;
    for (int j = 0; j < a.g.nl; ++j) {
      for (int64_t u = tid; u < a.g.N; u += kGThreads) {
        const uint32_t key = (uint32_t)(composite(a.g, h[u], u, j) >> a.g.ib);
        const uint32_t idx = (uint32_t)(u * a.g.nl + j);
        if (key == K && (hs >= 32 || (idx >> hs) == (ipre >> hs)))
          atomicAdd(&lh[(idx >> ps.shift) & dmask], (uint32_t)a.g.cost[j]);
      }
    }
    __syncthreads();
    if (tid < 64) {
      uint32_t digit;
      int64_t before;
      find_bin<false>(lh, r, digit, before);
      if (tid == 0) ipre_s = ipre | (digit << ps.shift);
      r -= before;  // only wavefront 0's r is used
    }
    __syncthreads();
  }
  if (tid == 0) {
    GState T;
    T.prefix = ((uint64_t)K << a.g.ib) | (((1ull << a.g.ib) - 1ull) - (uint64_t)ipre_s);
    T.r = r;
    a.st_out[s] = T;
  }
}

// ------------------------------------------------------------------ levels ----
struct LevelArgs {
  GArgs g;
  const GState* st;  // e* per sample (unused when glevel >= 0)
  uint32_t* map;     // 2 bits per tile, 4 words per 64 tiles
  uint32_t* wsum;    // per 64 tiles: the sum of their code widths
  int64_t tiles, nblocks, kA;
  int32_t glevel;    // >= 0: every tile takes this level
  uint32_t cands;    // candidate widths, one byte each, c_1 lowest
};

__global__ __launch_bounds__(256) void k_glevel(LevelArgs a) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int64_t t = (int64_t)blockIdx.x * 256 + tid;
  int lv = 0, w = 0;
  if (t < a.tiles) {
    if (a.glevel >= 0) {
      lv = a.glevel;
    } else {
      const int64_t ta = a.kA == 1 ? t : t / a.kA;  // allocation tile
      const int64_t s = ta / a.g.N;
      const int64_t u = ta - s * a.g.N;
      const float h = a.g.H[ta];
      const uint64_t P = a.st[s].prefix;
      for (int j = 0; j < a.g.nl; ++j) lv += composite(a.g, h, u, j) > P ? 1 : 0;
    }
    w = (int)((a.cands >> (8 * lv)) & 255u);
  }
  uint32_t f = (uint32_t)lv << (2 * (lane & 15));
#pragma unroll
  for (int off = 1; off < 16; off <<= 1) f |= (uint32_t)__shfl_xor((int)f, off, 64);
  int sum = w;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) sum += __shfl_xor(sum, off, 64);
  const int64_t blk = ((int64_t)blockIdx.x * 256 + (tid & ~63)) >> 6;
  if (blk < a.nblocks) {
    if ((lane & 15) == 0) a.map[4 * blk + (lane >> 4)] = f;
    if (lane == 0) a.wsum[blk] = (uint32_t)sum;
  }
}

hipError_t launch_greedy(const Plan& pl, void* payload, void* ws, hipStream_t st) {
  uint8_t* w = static_cast<uint8_t*>(ws);
  uint8_t* P = static_cast<uint8_t*>(payload);
  GArgs g;
  g.H = reinterpret_cast<const float*>(w + pl.ws_H);
  g.N = pl.N;
  g.nl = pl.nl;
  g.ib = pl.ib;
  for (int j = 0; j < 3; ++j) {
    g.lam[j] = pl.lam[j];
    g.cost[j] = pl.cost[j];
  }
  GState* states = reinterpret_cast<GState*>(w + pl.ws_state);
  const int64_t ns = pl.nsamples;
  GState* final_st = nullptr;
  if (pl.glevel < 0 && pl.N * pl.nl <= kGSmall) {
    GSmallArgs sa;
    sa.g = g;
    sa.st_out = states;
    sa.R = pl.R;
    for (int i = 0; i < 3; ++i) {
      sa.key[i] = pl.gpasses[i];
      sa.idx[i] = pl.gidx[i];
    }
    sa.nidx = pl.ngidx;
    hipLaunchKernelGGL(k_gselect_small, dim3((unsigned)ns), dim3(kGThreads), 0, st, sa);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    final_st = states;
  } else if (pl.glevel < 0) {
    // one sample of quantization tiles, few enough runs for one resolve
    // workgroup: the level map, width sums, block table and total are built
    // by the last key digit and k_gresolve (no k_glevel or k_table launch)
    const bool fold = pl.kA == 1 && ns == 1 && (pl.N + 63) / 64 <= kFoldMaxRuns;
    uint32_t* map = reinterpret_cast<uint32_t*>(P ? P + pl.off_bitmap : w + pl.ws_bitmap);
    uint32_t* run_sums = reinterpret_cast<uint32_t*>(w + pl.ws_blockcnt);
    uint32_t cands = 0;
    for (int i = 0; i < pl.n_candidates; ++i) cands |= (uint32_t)pl.candidates[i] << (8 * i);
    uint32_t* hists = reinterpret_cast<uint32_t*>(w + pl.ws_hist);
    const int64_t hsz = ns * kBins;
    GHistArgs h;
    h.g = g;
    h.fold_map = map;
    h.fold_run = run_sums;
    h.cands = cands;
    h.cand = reinterpret_cast<uint32_t*>(w + pl.ws_cand);
    int per = 1;  // tiles per thread
    while (per < 4 && ns * ((pl.N + kGThreads * per - 1) / (kGThreads * per)) > kGMaxWgs) per *= 2;
    const int64_t chunk = (int64_t)kGThreads * per;
    h.chunks_per_sample = (pl.N + chunk - 1) / chunk;
    h.R = pl.R;
    h.ncand = pl.ncand;
    h.cand_stride = pl.cand_stride;
    const int np = pl.ngpasses;
    // key digit p: state p in states[p % 2], histogram p in hists[p % 3]
    // (zeroed by k_stats for p = 0)
    for (int p = 0; p < np; ++p) {
      h.pass = pl.gpasses[p];
      h.last_key = p == np - 1;
      h.has_prev = p > 0;
      h.prev = p > 0 ? pl.gpasses[p - 1] : pl.gpasses[p];
      h.st_prev = states + ((p + 1) % 2) * ns;
      h.st_cur = states + (p % 2) * ns;
      h.hist_prev = hists + ((p + 2) % 3) * hsz;
      h.hist_cur = hists + (p % 3) * hsz;
      h.hist_clear = hists + ((p + 1) % 3) * hsz;
      h.fold = fold && h.last_key;
      const dim3 grid((unsigned)(h.chunks_per_sample * ns));
      if (per == 1) hipLaunchKernelGGL(k_ghist<1>, grid, dim3(kGThreads), 0, st, h);
      else if (per == 2) hipLaunchKernelGGL(k_ghist<2>, grid, dim3(kGThreads), 0, st, h);
      else hipLaunchKernelGGL(k_ghist<4>, grid, dim3(kGThreads), 0, st, h);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    final_st = states + (np % 2) * ns;
    GResolveArgs rs;
    rs.g = g;
    rs.st_prev = states + ((np + 1) % 2) * ns;
    rs.st_out = final_st;
    rs.hist_last = hists + ((np + 2) % 3) * hsz;
    rs.cand = h.cand;
    rs.ncand = pl.ncand;
    rs.cand_stride = pl.cand_stride;
    rs.last = pl.gpasses[np - 1];
    rs.nidx = pl.ngidx;
    for (int i = 0; i < 3; ++i) rs.idx[i] = pl.gidx[i];
    rs.fold_map = map;
    rs.fold_run = run_sums;
    rs.table = reinterpret_cast<uint32_t*>(P ? P + pl.off_table : w + pl.ws_table);
    rs.wtotal = reinterpret_cast<uint32_t*>(w + pl.ws_wtotal);
    rs.fold = fold;
    static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(k_gresolve),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                                       (int)(4 * kFoldMaxRuns));
    if (attr != hipSuccess) return attr;
    // the run width sums in whole rounds of 4 per thread
    const int64_t round = 4 * kGResolveThreads;
    const size_t rs_bytes = fold ? (size_t)(4 * (((pl.N + 63) / 64 + round - 1) / round) * round) : 0;
    hipLaunchKernelGGL(k_gresolve, dim3((unsigned)ns), dim3(kGResolveThreads), rs_bytes, st, rs);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess || fold) return e;  // fold: level map, table and total are complete
  }
  LevelArgs L;
  L.g = g;
  L.st = final_st;
  L.map = reinterpret_cast<uint32_t*>(P ? P + pl.off_bitmap : w + pl.ws_bitmap);
  L.wsum = reinterpret_cast<uint32_t*>(w + pl.ws_blockcnt);
  L.tiles = pl.tiles;
  L.nblocks = pl.nblocks;
  L.kA = pl.kA;
  L.glevel = pl.glevel;
  L.cands = 0;
  for (int i = 0; i < pl.n_candidates; ++i) L.cands |= (uint32_t)pl.candidates[i] << (8 * i);
  hipLaunchKernelGGL(k_glevel, dim3((unsigned)((pl.tiles + 255) / 256)), dim3(256), 0, st, L);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  uint32_t* table = reinterpret_cast<uint32_t*>(P ? P + pl.off_table : w + pl.ws_table);
  return launch_table(L.wsum, table, reinterpret_cast<uint32_t*>(w + pl.ws_wtotal), pl.nblocks, st);
}

}  // namespace tah
