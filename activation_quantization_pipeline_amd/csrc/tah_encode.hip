// Encode and fused encode+decode kernels of the TAH-Quant codec for gfx950.
//
// A workgroup is one wavefront; it takes groups of 64 consecutive tiles, one
// tile per lane:
//  1. stage:   the 64 tiles (contiguous in HBM) arrive with 16-byte coalesced
//              loads (in the round trip and the mixed-width encoder prefetched
//              one group ahead) and go into padded LDS rows;
//  2. phase A: lane i reads tile i from LDS and computes the outlier ratio of
//              Eq. (3) (top-2 magnitudes, pivot d, flag) and, for a uniform
//              allocation, the tile entropy of Eq. (1)-(2); with a mixed
//              allocation the width comes from the selection pass instead
//              (a bit of the width map, or a 2-bit level of the greedy one).
//              It fixes the tile's code-block offset (§3.4 packing order);
//  3. forward: a flagged tile gets the pivot swap P_d in its own LDS row and
//              the Hadamard transform of Eq. (4) in the lane's registers (in
//              the encode-only kernel, by 16-lane groups through LDS slots);
//  4. quantize: every lane quantizes its (transformed or not) tile
//              asymmetrically (§3.3), packs the codes and stores code block,
//              scale and zero-point; the fused variant dequantizes from the
//              codes in registers;
//  5. inverse: a flagged tile gets H^T / G in registers and, once written to
//              its LDS row, the swap undone there;
//  6. out:     the rebuilt tiles leave LDS with 16-byte coalesced stores.
#include "tah_device.hpp"
#include "tah_internal.hpp"

namespace tah {

struct EncArgs {
  const uint8_t* x;
  uint8_t* y;
  uint8_t* payload;  // null: payload sections are not written
  uint32_t* table;   // block table (payload or workspace)
  uint32_t* bitmap;  // width map (payload or workspace)
  float* H;          // per-tile entropies (workspace)
  const uint8_t* side_in;  // mixed layouts: the side bytes the statistics pass wrote
  // one width everywhere: the width map's words per 64 tiles, their value, and
  // the block table's step per 64 tiles
  int32_t map_words;
  uint32_t map_fill, table_step;
  int64_t tiles;
  int64_t off_side, off_scale, off_zero, off_codes;
  int32_t b_lo, b_hi, sz_lo, sz_hi;
  uint32_t cands;           // candidate widths, one byte each (any-width layout)
  const uint32_t* wtotal;   // any-width layout: the sum of all code widths
  int64_t code_end;         // end of the code section
  float tau;
  Header hdr;
  PadRanges pads;
};

// The round trip of bf16 tiles of up to 64 channels with a bf16 output, and
// the encode-only kernel of such tiles with one width, run four wavefronts per
// SIMD (at most 128 VGPRs, and at most 10 KB of LDS per workgroup, so sixteen
// share a compute unit): with one width the statistics and entropy are formed
// from the LDS row chunk by chunk, every layout reads the tile from its row
// when it quantizes it (with the word-by-word quantizer unless one width is
// rebuilt), the flagged tiles are transformed by their own lanes, and no next
// group is prefetched into registers. 8192 x 8192 one width: round trip 57.2
// -> 55.3 us (58.7 against 60.8 us in the first launches after an idle
// spell), encode only 41.3 -> 40.1 us; 16384 x 4096: round trip 59.0 -> 57.2
// us, encode only 49.4 -> 41.7 us; round trip at the 80/20 split 118.6 ->
// 116.6 us, greedy 124.7 -> 123.4 us (one box, interleaved). The mixed-width
// encode-only kernel stays at three wavefronts (the 80/20 encode at 8192 x
// 8192: 100.1 against 101.1 us at four).
template <int G, typename T, int OUT, int MODE>
constexpr bool kFourWaves() {
  return G <= 64 && Elem<T>::kBytes == 2 && (OUT == 2 || (OUT == 0 && MODE == 0));
}

// Minimum waves per SIMD the register allocator must leave room for.
template <int G, typename T, int OUT, int MODE>
constexpr int kMinWaves() {
  return kFourWaves<G, T, OUT, MODE>() ? 4 : ((G <= 64 && Elem<T>::kBytes == 2) ? 3 : (G <= 64 ? 2 : 1));
}

template <int G, int B>
__device__ __forceinline__ void store_codes(const uint32_t (&mq)[G], uint8_t* dst) {
  constexpr int W = G * B / 32;
  uint32_t w[W];
  pack_codes<G, B>(mq, w);
  // Every code block offset is a multiple of G/8 bytes (one bit per code) past
  // a 256-byte aligned base, whatever the widths of the blocks before it.
  if constexpr (G >= 128) {
#pragma unroll
    for (int i = 0; i < W / 4; ++i)
      reinterpret_cast<uint4*>(dst)[i] = make_uint4(w[4 * i], w[4 * i + 1], w[4 * i + 2], w[4 * i + 3]);
  } else if constexpr (G >= 64) {
#pragma unroll
    for (int i = 0; i < W / 2; ++i) reinterpret_cast<uint2*>(dst)[i] = make_uint2(w[2 * i], w[2 * i + 1]);
  } else {
#pragma unroll
    for (int i = 0; i < W; ++i) reinterpret_cast<uint32_t*>(dst)[i] = w[i];
  }
}

template <int G>
__device__ __forceinline__ void store_codes_b(int b, const uint32_t (&mq)[G], uint8_t* dst) {
  switch (b) {
    case 1: store_codes<G, 1>(mq, dst); break;
    case 2: store_codes<G, 2>(mq, dst); break;
    case 3: store_codes<G, 3>(mq, dst); break;
    case 4: store_codes<G, 4>(mq, dst); break;
    case 5: store_codes<G, 5>(mq, dst); break;
    case 6: store_codes<G, 6>(mq, dst); break;
    case 7: store_codes<G, 7>(mq, dst); break;
    default: store_codes<G, 8>(mq, dst); break;
  }
}


// Phase-A statistics of one tile read from LDS (Eq. 3 and Eq. 1):
// m1 = max |a_k|, d = first index holding m1, m2 = max |a_k| over k != d,
// l1 = sum |a_k| left to right; v receives the tile as fp32.
// bf16 tiles: the magnitude bits and (G-1-k) share one 32-bit key (bf16
// leaves the low 16 bits free), so max/median on unsigned keys give the top
// two magnitudes, the lowest index among ties, and no float compares.
template <int G, typename TIn>
__device__ __forceinline__ void tile_stats(const uint8_t* row, float (&v)[G], float& m1, float& m2, int& d,
                                           float& l1) {
  if constexpr (Elem<TIn>::kBytes == 2) {
    const uint4* p = reinterpret_cast<const uint4*>(row);
    uint32_t k1 = 0u, k2 = 0u;
    float s = 0.0f;
#pragma unroll
    for (int c = 0; c < G / 8; ++c) {
      const uint4 q = p[c];
      const uint32_t u[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int k = 8 * c + 2 * i;
        // the widened values, made opaque to the compiler so that the entropy's
        // table offset stays one bit-field extract of them (folded into u's
        // bits it takes two instructions)
        uint32_t xl, xh;
        asm("v_lshlrev_b32 %0, 16, %1" : "=v"(xl) : "v"(u[i]));
        asm("v_and_b32 %0, 0xffff0000, %1" : "=v"(xh) : "v"(u[i]));
        const uint32_t kl = (xl & 0x7fff0000u) | (uint32_t)(G - 1 - k);
        const uint32_t kh = (u[i] & 0x7fff0000u) | (uint32_t)(G - 2 - k);
        v[k] = __uint_as_float(xl);
        v[k + 1] = __uint_as_float(xh);
        s = s + fabsf(v[k]);
        k2 = umed3(k2, kl, k1);
        k1 = max(k1, kl);
        s = s + fabsf(v[k + 1]);
        k2 = umed3(k2, kh, k1);
        k1 = max(k1, kh);
      }
    }
    m1 = __uint_as_float(k1 & 0xffff0000u);
    m2 = __uint_as_float(k2 & 0xffff0000u);
    d = G - 1 - (int)(k1 & 0xffffu);
    l1 = s;
  } else {
    lds_read_tile<G, TIn>(row, v);
    float a1 = fabsf(v[0]), a2 = 0.0f, s = 0.0f + fabsf(v[0]);
    int dd = 0;
#pragma unroll
    for (int k = 1; k < G; ++k) {
      const float av = fabsf(v[k]);
      s = s + av;
      const bool c = av > a1;
      a2 = __builtin_amdgcn_fmed3f(a2, av, a1);
      a1 = fmaxf(a1, av);
      dd = c ? k : dd;
    }
    m1 = a1;
    m2 = a2;
    d = dd;
    l1 = s;
  }
}

// Phase-A statistics and entropy of a bf16 tile read from its LDS row chunk
// by chunk: the same m1, m2, d as tile_stats and the same entropy as
// tile_entropy (L and S summed left to right from 0), without the G values
// held in registers at once.
template <int G>
__device__ __forceinline__ float tile_stats_entropy_bf16(const uint8_t* row, const float* lt, float& m1, float& m2,
                                                         int& d) {
  const uint4* p = reinterpret_cast<const uint4*>(row);
  float l1 = 0.0f, S = 0.0f;
  uint32_t k1 = 0u, k2 = 0u;
#pragma unroll
  for (int c = 0; c < G / 8; ++c) {
    const uint4 q = p[c];
    const uint32_t u[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int k = 8 * c + 2 * i;
      uint32_t xl, xh;  // opaque widened values (see tile_stats)
      asm("v_lshlrev_b32 %0, 16, %1" : "=v"(xl) : "v"(u[i]));
      asm("v_and_b32 %0, 0xffff0000, %1" : "=v"(xh) : "v"(u[i]));
      const float vl = __uint_as_float(xl), vh = __uint_as_float(xh);
      const uint32_t kl = (xl & 0x7fff0000u) | (uint32_t)(G - 1 - k);
      const uint32_t kh = (u[i] & 0x7fff0000u) | (uint32_t)(G - 2 - k);
      l1 = l1 + fabsf(vl);
      k2 = umed3(k2, kl, k1);
      k1 = max(k1, kl);
      S = __builtin_fmaf(fabsf(vl), log2_node(vl, lt), S);
      l1 = l1 + fabsf(vh);
      k2 = umed3(k2, kh, k1);
      k1 = max(k1, kh);
      S = __builtin_fmaf(fabsf(vh), log2_node(vh, lt), S);
    }
  }
  m1 = __uint_as_float(k1 & 0xffff0000u);
  m2 = __uint_as_float(k2 & 0xffff0000u);
  d = G - 1 - (int)(k1 & 0xffffu);
  return entropy_from_sums(l1, S, lt);
}

// Whether the receiver's H then 1/G (Eq. 4 inverted) may take the 1/G first,
// as fmaf(q, s/G, lo/G), with bit-identical results. G is a power of two, so
// scaling by 1/G commutes with every rounding that stays in the normal range.
// With s = 0 or s >= 2^-112 (s has 8 significant bits) and lo = 0 or
// |lo| >= 2^-96, every q s + lo is a multiple of 2^-119, and so is every sum
// and difference of the butterflies; divided by G <= 128 such a value is 0 or
// at least 2^-126, never subnormal, so each scaled result is the unscaled one
// over G, exactly, and so is the last product by 1/G. With |lo|, |hv| < 2^120
// no unscaled sum of at most 128 values overflows either. Anything else (NaN,
// infinities, tiny or huge tiles) keeps the product by 1/G after H.
__device__ __forceinline__ bool prescale_exact(float s, float lo, float hv) {
  const float alo = fabsf(lo);
  return (s == 0.0f || s >= 0x1p-112f) && (lo == 0.0f || alo >= 0x1p-96f) && alo < 0x1p120f &&
         fabsf(hv) < 0x1p120f;
}

// Step s rounded up to bf16 and its reciprocal (§3.3 asymmetric quantizer).
__device__ __forceinline__ void step_of(float lo, float hv, int b, float& s, float& inv) {
  const float L = (float)((1 << b) - 1);
  uint32_t sb = __float_as_uint((hv - lo) / L);
  if (sb & 0xffffu) sb = (sb & 0xffff0000u) + 0x10000u;
  s = __uint_as_float(sb);
  if (!(s >= 0x1p-126f)) s = 0.0f;
  inv = s > 0.0f ? 1.0f / s : 0.0f;
}

// Quantize one tile held in registers (§3.3): zero-point lo = min, step from
// the range, codes q_k = round-half-even of the exact (y_k - lo) * inv (one
// fused rounding against 2^23); store code block, scale and zero-point. With
// OUT the tile is replaced by its dequantized values (the receiver's step of
// Algorithm 1, from the codes in registers).
// GUARD: skip a code block that would end past the code section (the
// any-width layout, whose offsets come from the allocator's tables).
// tr: the tile was transformed, so its dequantized values go through H and
// the 1/G. Returns true when the 1/G is already applied here, as the step
// s/G and zero-point lo/G of the dequantization (exact, see prescale_exact).
template <int G, int OUT, bool GUARD = false>
__device__ __forceinline__ bool quantize_tile(const EncArgs& a, float (&v)[G], int64_t t, int b, int64_t code_off,
                                              bool tr = false) {
  float lo = v[0], hv = v[0];
#pragma unroll
  for (int k = 1; k < G; ++k) {
    lo = fminf(lo, v[k]);
    hv = fmaxf(hv, v[k]);
  }
  lo = lo + 0.0f;
  hv = hv + 0.0f;
  float s, inv;
  step_of(lo, hv, b, s, inv);
  uint32_t mq[G];
#pragma unroll
  for (int k = 0; k < G; ++k) mq[k] = __float_as_uint(__builtin_fmaf(v[k] - lo, inv, 0x1p23f));
  if (a.payload) {
    if (!GUARD || code_off + (int64_t)(G / 8) * b <= a.code_end) store_codes_b<G>(b, mq, a.payload + code_off);
    reinterpret_cast<uint16_t*>(a.payload + a.off_scale)[t] = (uint16_t)(__float_as_uint(s) >> 16);
    reinterpret_cast<float*>(a.payload + a.off_zero)[t] = lo;
  }
  bool pre = false;
  if constexpr (OUT != 0) {
    pre = tr && prescale_exact(s, lo, hv);
    const float sd = pre ? s * (1.0f / G) : s, ld = pre ? lo * (1.0f / G) : lo;
#pragma unroll
    for (int k = 0; k < G; ++k) v[k] = __builtin_fmaf(__uint_as_float(mq[k]) - 0x1p23f, sd, ld);
  }
  return pre;
}

// The quantizer that forms, packs and stores the codes word by word (defined
// with the 128-channel kernel below).
template <int G, int OUT, bool GUARD>
__device__ __forceinline__ bool quantize_stream(const EncArgs& a, float (&v)[G], int64_t t, int b, int64_t code_off,
                                                bool tr);

// OUT: 0 = no reconstruction, 1 = fp32, 2 = bf16.
// MODE: the width layout: 0 one width (the entropy is computed here), 1 two
// widths from the 1-bit width map and the count table, 2 any candidate from
// the 2-bit level map and the width-sum table.
// A workgroup is one wavefront with LDS rows of its own; group g of 64 tiles
// goes to workgroup g mod gridDim.x. The launch gives every group a workgroup
// of its own (see launch_one); with a smaller grid a workgroup takes several
// groups, and in the round trip and the mixed-width encoder it then
// prefetches the next group into registers while the current one is
// processed.
//
// In the round trip a flagged tile (Eq. 3) is transformed by its own lane
// with fwht<G>, the stage order of the oracle. The wavefront runs the
// butterflies whenever one of its 64 tiles is flagged; measured on the
// 8192x8192 round trip this beats handing the flagged tiles to 16-lane groups
// through LDS (barriers and round trips per group), forward and inverse or
// forward alone. The encode-only kernel does hand them over (see kCoopH).
template <int G, typename TIn, int OUT, int MODE>
__global__ __launch_bounds__(64, (kMinWaves<G, TIn, OUT, MODE>())) void k_encode(EncArgs a) {
  constexpr int NT = 64;
  constexpr bool MIXED = MODE != 0;
  using RI = TileRow<G, TIn>;
  using TOut = typename std::conditional<OUT == 1, float, bf16_t>::type;
  using RO = TileRow<G, TOut>;
  // The next group is prefetched into registers in the round trip and in the
  // encode-only kernel of the mixed layouts (8192 x 8192 at the 80/20 split:
  // 107.7 -> 100.7 us per encode). The encode-only kernel with one width,
  // which also computes the entropies, runs faster without it (41.9 against
  // 45.4 us at 8192 x 8192, three waves per SIMD either way).
  constexpr bool kFour = kFourWaves<G, TIn, OUT, MODE>();
  constexpr bool kPrefetch = RI::kChunks <= 8 && (OUT != 0 || MIXED) && !kFour;
  // Each LDS row is read and rewritten only by its own lane, so a rebuilt tile
  // goes back into its own row when rows have the same width; otherwise
  // rebuilt tiles get rows of their own.
  constexpr bool kSameRow = OUT == 0 || RO::kStride == RI::kStride;

  // Encode only at three wavefronts (the mixed layouts): flagged tiles go
  // through H by 16-lane groups, kCoop tiles per round through fp32 slots
  // (44.7 us against 47.7 us per-lane for the 8192 x 8192 encode at the time).
  // The round trip keeps the per-lane butterflies (60.8 us against 63.5 us):
  // there the cooperative form, forward and inverse, cost more in registers
  // and barriers than it saved; so does the four-wave encode-only kernel.
  constexpr bool kCoopH = OUT == 0 && !kFourWaves<G, TIn, OUT, MODE>();
  constexpr int V = G / 16;     // elements per lane in a 16-lane transform group
  constexpr int kCoop = 8;      // flagged tiles per round
  constexpr int kSlot = G + 4;  // fp32 slot stride
  // One LDS block with only what this instantiation uses: the tile rows, rows
  // for rebuilt tiles of another width, the transform slots and list of the
  // encode-only kernel, the log2 tables of the entropy (one width only).
  constexpr int kXs = NT * RI::kStride;
  constexpr int kYs = kSameRow ? 0 : NT * RO::kStride;
  constexpr int kTs = kCoopH ? 4 * kCoop * kSlot : 0;
  constexpr int kFl = kCoopH ? 4 * NT : 0;
  constexpr int kLt = MIXED ? 0 : 4 * 256;
  static_assert(!kFour || kXs + kLt <= 10240, "sixteen workgroups per compute unit");
  __shared__ __attribute__((aligned(16))) uint8_t smem[kXs + kYs + kTs + kFl + kLt];
  uint8_t* xs = smem;
  uint8_t* ys = kSameRow ? xs : smem + kXs;
  float* ts = reinterpret_cast<float*>(smem + kXs + kYs);
  uint32_t* flist = reinterpret_cast<uint32_t*>(smem + kXs + kYs + kTs);
  float* lt = reinterpret_cast<float*>(smem + kXs + kYs + kTs + kFl);

  const int lane = threadIdx.x;
  const int q4 = lane >> 4, r16 = lane & 15;

  if (blockIdx.x == 0 && a.payload) {
    if (lane < 32) reinterpret_cast<uint32_t*>(a.payload)[lane] = a.hdr.w[lane];
    for (int r = 0; r < a.pads.n; ++r)
      for (int i = lane; i < a.pads.len[r]; i += NT) a.payload[a.pads.off[r] + i] = 0;
  }
  if constexpr (MODE == 2) {
    // the code section is sized for the whole budget: its unused tail is zero
    if (a.payload) {
      const int64_t used = a.off_codes + (int64_t)(G / 8) * (int64_t)a.wtotal[0];
      for (int64_t i = used + (int64_t)blockIdx.x * NT + lane; i < a.code_end; i += (int64_t)gridDim.x * NT)
        a.payload[i] = 0;
    }
  }

  if constexpr (!MIXED) load_log2_tab(lt);  // read after the first barrier of the loop

  const int64_t ngroups = (a.tiles + NT - 1) / NT;
  int64_t g = blockIdx.x;
  GroupRegs<G, TIn> pre;
  if (kPrefetch && g < ngroups) {
    const int64_t t0 = g * NT;
    group_load<G, TIn, NT>(a.x + t0 * RI::kBytes, (int)min<int64_t>(NT, a.tiles - t0), pre);
  }

  // The rebuilt tiles of a group leave LDS at the top of the next iteration,
  // after the prefetched tiles have arrived: loads and stores share one
  // completion counter on this target, so waiting for the prefetch only ever
  // drains stores issued a whole group earlier.
  int64_t prev_t0 = -1;
  int prev_n = 0;
  for (; g < ngroups; g += gridDim.x) {
    const int64_t t0 = g * NT;
    const int n = (int)min<int64_t>(NT, a.tiles - t0);
    if constexpr (!kPrefetch) group_load<G, TIn, NT>(a.x + t0 * RI::kBytes, n, pre);
    group_wait(pre);
    if constexpr (OUT != 0) {
      if (prev_t0 >= 0) stage_out<G, TOut, NT>(ys, a.y + prev_t0 * RO::kBytes, prev_n);
    }
    group_to_lds<G, TIn, NT>(pre, xs, n);
    __syncthreads();
    if constexpr (kPrefetch) {  // the next group of this workgroup
      const int64_t gn = g + gridDim.x;
      if (gn < ngroups) {
        const int64_t tn = gn * NT;
        group_load<G, TIn, NT>(a.x + tn * RI::kBytes, (int)min<int64_t>(NT, a.tiles - tn), pre);
      } else {
        // last group: the old contents are dead (without this the compiler keeps
        // them alive through the iteration for the wait at the loop top)
        pre = GroupRegs<G, TIn>{};
      }
    }

    // ---------------- phase A: lane owns tile t0 + lane ----------------
    const bool act = lane < n;
    const int64_t t = t0 + lane;
    int flag = 0, piv = 0, hi = 0, bw = 0;
    float v[G];
    if (act) {
      if constexpr (!MIXED) {
        float m1, m2;
        int d;
        if constexpr (kFour) {
          a.H[t] = tile_stats_entropy_bf16<G>(xs + lane * RI::kStride, lt, m1, m2, d);  // Eq. (1)-(2)
        } else {
          float l1;
          tile_stats<G, TIn>(xs + lane * RI::kStride, v, m1, m2, d, l1);
          a.H[t] = tile_entropy<G, Elem<TIn>::kBytes == 2>(v, l1, lt);  // Eq. (1)-(2)
        }
        flag = m1 > a.tau * (m2 + kRho);  // Eq. (3) without the division
        piv = d;
        // side byte: the flag, and the pivot of a transformed tile (0 for the others)
        if (a.payload) a.payload[a.off_side + t] = (uint8_t)(flag ? (0x80 | piv) : 0);
      } else {
        // the statistics pass already took Eq. (3) and wrote the side byte
        const uint32_t sb = a.side_in[t];
        flag = (int)(sb >> 7);
        piv = (int)(sb & 127u);
        if constexpr (!kFour) lds_read_tile<G, TIn>(xs + lane * RI::kStride, v);
        if constexpr (MODE == 1) {
          hi = (a.bitmap[t >> 5] >> (t & 31)) & 1u;
        } else {
          const uint32_t lv = (a.bitmap[t >> 4] >> (2 * (t & 15))) & 3u;
          bw = (int)((a.cands >> (8 * lv)) & 255u);
        }
      }
    }

    // Code-block offsets: tile t starts at t*sz_lo + (b_hi tiles before t)*(sz_hi - sz_lo);
    // the 64 tiles of a group are one run of the block table.
    const uint64_t hmask = ballot(act && hi);
    int64_t code_off = a.off_codes + t * a.sz_lo;
    if constexpr (MODE == 2) {
      // G/8 bytes per unit of width: the table's sum before the group plus the
      // widths of the lanes below
      uint32_t incl = (uint32_t)bw;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t o = (uint32_t)__shfl_up((int)incl, off, 64);
        if (lane >= off) incl += o;
      }
      code_off = a.off_codes + (int64_t)(G / 8) * ((int64_t)a.table[t0 >> 6] + (int64_t)(incl - (uint32_t)bw));
    } else if constexpr (MIXED) {
      const uint32_t hb = a.table[t0 >> 6] + lanes_below(hmask);
      code_off += (int64_t)hb * (a.sz_hi - a.sz_lo);
    } else {
      // uniform allocation: no tile has b_hi
      if (lane < a.map_words && a.bitmap) {
        // one width everywhere: the width map's words are constant and the
        // block table is closed-form (no b_hi tile in the two-width layout;
        // 64 times the width per run in the any-width layout)
        const int64_t blk = t0 >> 6;
        // entries past the last tile stay zero
        const int per_word = 64 / a.map_words;
        const int64_t left = a.tiles - t0 - (int64_t)lane * per_word;
        uint32_t fill = a.map_fill;
        if (left < per_word) fill = left <= 0 ? 0u : fill & ((1u << (left * (a.map_words >> 1))) - 1u);
        a.bitmap[a.map_words * blk + lane] = fill;
        if (lane == 0) a.table[blk] = (uint32_t)blk * a.table_step;
      }
    }

    // ---------------- transformed tiles (§3.3) and quantization ----------------
    const int b = MODE == 2 ? bw : (hi ? a.b_hi : a.b_lo);
    if constexpr (kCoopH) {
      const uint64_t fmask = ballot(act && flag);
      const int nf = (int)__popcll(fmask);
      const int slot = (int)lanes_below(fmask);
      if (act && flag) {  // P_d in the lane's own row
        uint8_t* row = xs + lane * RI::kStride;
        const uint32_t x0 = lds_elem_bits<TIn>(row, 0), xd = lds_elem_bits<TIn>(row, piv);
        lds_elem_set<TIn>(row, 0, xd);
        lds_elem_set<TIn>(row, piv, x0);
        flist[slot] = (uint32_t)lane;
      }
      if (nf != 0) {
        // H of Eq. (4) on the swapped rows by 16-lane groups (fwht16: the same
        // butterflies in the same order as fwht<G>); each tile's own lane
        // then reads its transformed tile from the slot
        __syncthreads();
        for (int j_lo = 0; j_lo < nf; j_lo += kCoop) {
          const int j_hi = nf < j_lo + kCoop ? nf : j_lo + kCoop;
          for (int j0 = j_lo; j0 < j_hi; j0 += 4) {
            const int j = j0 + q4;
            if (j < j_hi) {
              float y[V];
              lds_read_part<V, TIn>(xs + flist[j] * RI::kStride, r16, y);
              fwht16<V>(y, r16);
              lds_write_part<V, float>(reinterpret_cast<uint8_t*>(ts + (j - j_lo) * kSlot), r16, y);
            }
          }
          __syncthreads();
          if (act && flag && slot >= j_lo && slot < j_hi)
            lds_read_tile<G, float>(reinterpret_cast<const uint8_t*>(ts + (slot - j_lo) * kSlot), v);
          __syncthreads();
        }
      }
      // codes packed word by word: the 64 codes never sit in registers at
      // once (137 against 168 VGPRs with a spill; 43.5 -> 41.9 us for the
      // 8192 x 8192 encode)
      if (act) quantize_stream<G, OUT, MODE == 2>(a, v, t, b, code_off, false);
    } else if (act) {
      if (flag) {  // P_d in the lane's own row, then H of Eq. (4) in registers
        uint8_t* row = xs + lane * RI::kStride;
        const uint32_t x0 = lds_elem_bits<TIn>(row, 0), xd = lds_elem_bits<TIn>(row, piv);
        lds_elem_set<TIn>(row, 0, xd);
        lds_elem_set<TIn>(row, piv, x0);
        if constexpr (!kFour) lds_read_tile<G, TIn>(row, v);
      }
      if constexpr (kFour) lds_read_tile<G, TIn>(xs + lane * RI::kStride, v);  // the tile from its row
      if (flag) fwht<G>(v);
      bool scaled;
      if constexpr (kFour && (MIXED || OUT == 0)) scaled = quantize_stream<G, OUT, MODE == 2>(a, v, t, b, code_off, flag != 0);
      else scaled = quantize_tile<G, OUT, MODE == 2>(a, v, t, b, code_off, flag != 0);
      if constexpr (OUT != 0) {
        if (flag) fwht<G>(v);  // H^T = H
        // the 1/G where the dequantization did not take it (rare: skipped by
        // the whole wavefront when no lane needs it)
        if (ballot(flag && !scaled) != 0) {
          if (flag && !scaled) {
#pragma unroll
            for (int k = 0; k < G; ++k) v[k] = v[k] * (1.0f / G);
          }
        }
        uint8_t* orow = ys + lane * RO::kStride;
        lds_write_tile<G, TOut>(orow, v);
        if (flag) {  // element d takes y_0, element 0 takes y_d
          const uint32_t y0 = lds_elem_bits<TOut>(orow, 0), yd = lds_elem_bits<TOut>(orow, piv);
          lds_elem_set<TOut>(orow, piv, y0);
          lds_elem_set<TOut>(orow, 0, yd);
        }
      }
    }

    if constexpr (OUT != 0) {
      prev_t0 = t0;
      prev_n = n;
    }
    __syncthreads();  // LDS rows are read by other lanes next
  }
  if constexpr (OUT != 0) {
    if (prev_t0 >= 0) stage_out<G, TOut, NT>(ys, a.y + prev_t0 * RO::kBytes, prev_n);
  }
}

// ---------------------------------------------------------------------------
// Tiles of 128 channels. One lane per tile needs the whole tile in registers
// (128 values), and staging a whole 64-tile group through LDS takes 33 KB of
// fp32 rows: one wavefront per SIMD. This kernel stages the group in two
// rounds of 32 tiles (17 KB), computes the statistics from registers, and
// forms, packs and dequantizes the codes word by word instead of holding all
// 128 codes, so two wavefronts fit on a SIMD.

// Codes of width B of a tile in registers, packed word by word as pack_codes
// does (code k at stream bits [kB, kB + B), LSB first), each code dequantized
// into v (OUT) as soon as its last bit is in a word; stores the code block at
// dst (GUARD: unless it would end past the code section). The same code
// values, words and dequantized values as quantize_tile (sd, ld: the step and
// zero-point of the dequantization, s and lo or both over G).
template <int G, int B, int OUT, bool GUARD>
__device__ __forceinline__ void quant_pack(const EncArgs& a, float (&v)[G], float lo, float inv, float sd, float ld,
                                           int64_t code_off) {
  constexpr int W = G * B / 32;
  uint32_t w[W];
  uint32_t carry = 0u;  // a code that began in the previous word
#pragma unroll
  for (int i = 0; i < W; ++i) {
    const int lo_bit = 32 * i;
    const int k0 = lo_bit / B;
    const int k1 = (lo_bit + 31) / B;
    uint32_t acc = 0u;
#pragma unroll
    for (int k = k0; k <= k1; ++k) {
      const int n = (k < k1) ? B : (lo_bit + 32 - k1 * B);
      const uint32_t q = (k * B < lo_bit) ? carry : __float_as_uint(__builtin_fmaf(v[k] - lo, inv, 0x1p23f));
      acc = __builtin_amdgcn_alignbit(q, acc, (uint32_t)n);
      if ((k + 1) * B <= lo_bit + 32) {
        if constexpr (OUT != 0) v[k] = __builtin_fmaf(__uint_as_float(q) - 0x1p23f, sd, ld);
      } else {
        carry = q;
      }
    }
    w[i] = acc;
  }
  if (a.payload && (!GUARD || code_off + (int64_t)(G / 8) * B <= a.code_end)) {
    // 16-, 8- or 4-byte stores by the block's size (every offset is a
    // multiple of G/8 bytes)
    if constexpr (W % 4 == 0) {
      uint4* dst = reinterpret_cast<uint4*>(a.payload + code_off);
#pragma unroll
      for (int i = 0; i < W / 4; ++i) dst[i] = make_uint4(w[4 * i], w[4 * i + 1], w[4 * i + 2], w[4 * i + 3]);
    } else if constexpr (W % 2 == 0) {
      uint2* dst = reinterpret_cast<uint2*>(a.payload + code_off);
#pragma unroll
      for (int i = 0; i < W / 2; ++i) dst[i] = make_uint2(w[2 * i], w[2 * i + 1]);
    } else {
      uint32_t* dst = reinterpret_cast<uint32_t*>(a.payload + code_off);
#pragma unroll
      for (int i = 0; i < W; ++i) dst[i] = w[i];
    }
  }
}

// tr and the result: as for quantize_tile.
template <int G, int OUT, bool GUARD>
__device__ __forceinline__ bool quantize_stream(const EncArgs& a, float (&v)[G], int64_t t, int b, int64_t code_off,
                                                bool tr) {
  float lo = v[0], hv = v[0];
#pragma unroll
  for (int k = 1; k < G; ++k) {
    lo = fminf(lo, v[k]);
    hv = fmaxf(hv, v[k]);
  }
  lo = lo + 0.0f;
  hv = hv + 0.0f;
  float s, inv;
  step_of(lo, hv, b, s, inv);
  const bool pre = OUT != 0 && tr && prescale_exact(s, lo, hv);
  const float sd = pre ? s * (1.0f / G) : s, ld = pre ? lo * (1.0f / G) : lo;
  switch (b) {
    case 1: quant_pack<G, 1, OUT, GUARD>(a, v, lo, inv, sd, ld, code_off); break;
    case 2: quant_pack<G, 2, OUT, GUARD>(a, v, lo, inv, sd, ld, code_off); break;
    case 3: quant_pack<G, 3, OUT, GUARD>(a, v, lo, inv, sd, ld, code_off); break;
    case 4: quant_pack<G, 4, OUT, GUARD>(a, v, lo, inv, sd, ld, code_off); break;
    case 5: quant_pack<G, 5, OUT, GUARD>(a, v, lo, inv, sd, ld, code_off); break;
    case 6: quant_pack<G, 6, OUT, GUARD>(a, v, lo, inv, sd, ld, code_off); break;
    case 7: quant_pack<G, 7, OUT, GUARD>(a, v, lo, inv, sd, ld, code_off); break;
    default: quant_pack<G, 8, OUT, GUARD>(a, v, lo, inv, sd, ld, code_off); break;
  }
  if (a.payload) {
    reinterpret_cast<uint16_t*>(a.payload + a.off_scale)[t] = (uint16_t)(__float_as_uint(s) >> 16);
    reinterpret_cast<float*>(a.payload + a.off_zero)[t] = lo;
  }
  return pre;
}

// n (<= 32) contiguous tiles of BYTES bytes between global memory and LDS rows
// of STRIDE bytes, 16 bytes per lane and step, streamed (touched once per call),
// every step of a round in flight at once (16 for fp32 rows: 168.6 -> 163.4 us
// for the 16384 x 5120 round trip against 8).
template <int BYTES, int STRIDE>
__device__ __forceinline__ void rows_in(const uint8_t* __restrict__ src, uint8_t* lds, int n) {
  constexpr int CH = BYTES / 16, PER = 32 * CH / 64, BATCH = PER < 16 ? PER : 16;
  const uint4* s = reinterpret_cast<const uint4*>(src);
  const int nch = n * CH;
  // addresses formed here at each call: hoisted out of the group loop, the
  // 32 of them would not fit beside the tiles
  int tid = (int)threadIdx.x;
  asm volatile("" : "+v"(tid));
#pragma unroll
  for (int i0 = 0; i0 < PER; i0 += BATCH) {
    uint4 buf[BATCH];
#pragma unroll
    for (int i = 0; i < BATCH; ++i) {  // the batch's loads in flight before its first LDS write
      const int c = tid + 64 * (i0 + i);
      buf[i] = load_stream(&s[c < nch ? c : nch - 1]);
    }
#pragma unroll
    for (int i = 0; i < BATCH; ++i) {
      const int c = tid + 64 * (i0 + i);
      if (c < nch) *reinterpret_cast<uint4*>(lds + (c / CH) * STRIDE + (c % CH) * 16) = buf[i];
    }
  }
}
template <int BYTES, int STRIDE>
__device__ __forceinline__ void rows_out(const uint8_t* lds, uint8_t* __restrict__ dst, int n) {
  constexpr int CH = BYTES / 16, PER = 32 * CH / 64, BATCH = PER < 16 ? PER : 16;
  uint4* d = reinterpret_cast<uint4*>(dst);
  const int nch = n * CH;
  int tid = (int)threadIdx.x;
  asm volatile("" : "+v"(tid));
#pragma unroll
  for (int i0 = 0; i0 < PER; i0 += BATCH) {
    uint4 buf[BATCH];
#pragma unroll
    for (int i = 0; i < BATCH; ++i) {
      const int c = tid + 64 * (i0 + i);
      const int cc = c < nch ? c : 0;
      buf[i] = *reinterpret_cast<const uint4*>(lds + (cc / CH) * STRIDE + (cc % CH) * 16);
    }
#pragma unroll
    for (int i = 0; i < BATCH; ++i) {
      const int c = tid + 64 * (i0 + i);
      if (c < nch) store_stream(&d[c], buf[i]);
    }
  }
}

// tile_entropy with the sum formed in chunks of CH elements: an empty asm on
// the running sum between chunks keeps the scheduler from issuing the table
// reads of the whole tile ahead of the sums (128 fp32 values and their
// interpolation slopes would not fit next to the tile). Same fp32 order.
template <int G, bool NODE, int CH>
__device__ __forceinline__ float tile_entropy_chunked(const float (&v)[G], float l1, const float* lt) {
  float S = 0.0f;
#pragma unroll
  for (int k0 = 0; k0 < G; k0 += CH) {
#pragma unroll
    for (int k = k0; k < k0 + CH; ++k) {
      // log2_full reads only the exponent and mantissa bits: the same on v as
      // on |v|, which then stays a source modifier of the fma
      const float lg = NODE ? log2_node(v[k], lt) : log2_full(v[k], lt);
      S = __builtin_fmaf(fabsf(v[k]), lg, S);
    }
    asm volatile("" : "+v"(S));
  }
  return l1 > 0.0f ? log2_full(l1, lt) - S / l1 : 0.0f;
}

template <typename TIn, int OUT, int MODE>
__global__ __launch_bounds__(64, 2) void k_encode128(EncArgs a) {
  constexpr int G = 128, NT = 64, RT = 32;  // tiles per group, tiles per LDS round
  constexpr bool MIXED = MODE != 0;
  constexpr bool NODE = Elem<TIn>::kBytes == 2;
  using RI = TileRow<G, TIn>;
  using TOut = typename std::conditional<OUT == 1, float, bf16_t>::type;
  using RO = TileRow<G, TOut>;
  constexpr int kStride = TileRow<G, float>::kStride;  // fp32 rows (the pivot swap goes through them)
  __shared__ __attribute__((aligned(16))) uint8_t st[RT * kStride];
  __shared__ __attribute__((aligned(16))) float lt[256];  // log2 tables of the entropy
  const int lane = threadIdx.x;
  const int half = lane >> 5;
  uint8_t* row = st + (lane & 31) * kStride;  // this lane's row in its round

  if (blockIdx.x == 0 && a.payload) {
    if (lane < 32) reinterpret_cast<uint32_t*>(a.payload)[lane] = a.hdr.w[lane];
    for (int r = 0; r < a.pads.n; ++r)
      for (int i = lane; i < a.pads.len[r]; i += NT) a.payload[a.pads.off[r] + i] = 0;
  }
  if constexpr (MODE == 2) {
    if (a.payload) {
      const int64_t used = a.off_codes + (int64_t)(G / 8) * (int64_t)a.wtotal[0];
      for (int64_t i = used + (int64_t)blockIdx.x * NT + lane; i < a.code_end; i += (int64_t)gridDim.x * NT)
        a.payload[i] = 0;
    }
  }
  if constexpr (!MIXED) load_log2_tab(lt);  // read after the first barrier of the loop

  const int64_t ngroups = (a.tiles + NT - 1) / NT;
  for (int64_t g = blockIdx.x; g < ngroups; g += gridDim.x) {
    const int64_t t0 = g * NT;
    const int n = (int)min<int64_t>(NT, a.tiles - t0);
    const bool act = lane < n;
    const int64_t t = t0 + lane;
    float v[G];
    // ---- in: two rounds of 32 tiles through LDS
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int nr = min(max(n - r * RT, 0), RT);
      if (nr > 0) {
        __syncthreads();  // the rows are free
        rows_in<RI::kBytes, kStride>(a.x + (t0 + r * RT) * RI::kBytes, st, nr);
        __syncthreads();
        if (half == r && act) lds_read_tile<G, TIn>(row, v);
      }
    }

    // ---- phase A: lane owns tile t0 + lane
    int flag = 0, piv = 0, hi = 0, bw = 0;
    if (act) {
      if constexpr (!MIXED) {
        float m1, m2, l1;
        int d;
        tile_stats_regs<G, NODE>(v, m1, m2, d, l1);
        flag = m1 > a.tau * (m2 + kRho);  // Eq. (3) without the division
        piv = d;
        a.H[t] = tile_entropy_chunked<G, NODE, 16>(v, l1, lt);  // Eq. (1)-(2)
        if (a.payload) a.payload[a.off_side + t] = (uint8_t)(flag ? (0x80 | piv) : 0);
      } else {
        // the statistics pass already took Eq. (3) and wrote the side byte
        const uint32_t sb = a.side_in[t];
        flag = (int)(sb >> 7);
        piv = (int)(sb & 127u);
        if constexpr (MODE == 1) {
          hi = (a.bitmap[t >> 5] >> (t & 31)) & 1u;
        } else {
          const uint32_t lv = (a.bitmap[t >> 4] >> (2 * (t & 15))) & 3u;
          bw = (int)((a.cands >> (8 * lv)) & 255u);
        }
      }
    }
    const uint64_t hmask = ballot(act && hi);
    int64_t code_off = a.off_codes + t * a.sz_lo;
    if constexpr (MODE == 2) {
      uint32_t incl = (uint32_t)bw;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t o = (uint32_t)__shfl_up((int)incl, off, 64);
        if (lane >= off) incl += o;
      }
      code_off = a.off_codes + (int64_t)(G / 8) * ((int64_t)a.table[t0 >> 6] + (int64_t)(incl - (uint32_t)bw));
    } else if constexpr (MIXED) {
      const uint32_t hb = a.table[t0 >> 6] + lanes_below(hmask);
      code_off += (int64_t)hb * (a.sz_hi - a.sz_lo);
    } else {
      if (lane < a.map_words && a.bitmap) {
        // one width everywhere: the width map's words are constant and the
        // block table is closed-form (no b_hi tile in the two-width layout;
        // 64 times the width per run in the any-width layout)
        const int64_t blk = t0 >> 6;
        // entries past the last tile stay zero
        const int per_word = 64 / a.map_words;
        const int64_t left = a.tiles - t0 - (int64_t)lane * per_word;
        uint32_t fill = a.map_fill;
        if (left < per_word) fill = left <= 0 ? 0u : fill & ((1u << (left * (a.map_words >> 1))) - 1u);
        a.bitmap[a.map_words * blk + lane] = fill;
        if (lane == 0) a.table[blk] = (uint32_t)blk * a.table_step;
      }
    }
    const int b = MODE == 2 ? bw : (hi ? a.b_hi : a.b_lo);

    // ---- forward: P_d through the lane's fp32 row (a register array takes no
    // per-lane index), then H of Eq. (4) in registers
    const uint64_t fmask = ballot(act && flag);
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      if ((uint32_t)(fmask >> (32 * r)) != 0u) {
        __syncthreads();
        if (half == r && act && flag) {
          lds_write_tile<G, float>(row, v);
          const uint32_t x0 = lds_elem_bits<float>(row, 0), xd = lds_elem_bits<float>(row, piv);
          lds_elem_set<float>(row, 0, xd);
          lds_elem_set<float>(row, piv, x0);
          lds_read_tile<G, float>(row, v);
        }
      }
    }
    if (act && flag) fwht<G>(v);

    // ---- quantize, pack, dequantize
    bool scaled = false;
    if (act) scaled = quantize_stream<G, OUT, MODE == 2>(a, v, t, b, code_off, flag != 0);

    // ---- inverse and out: two rounds of 32 rebuilt tiles through LDS
    if constexpr (OUT != 0) {
      if (act && flag) fwht<G>(v);  // H^T = H
      // the 1/G where the dequantization did not take it
      if (ballot(act && flag && !scaled) != 0) {
        if (act && flag && !scaled) {
#pragma unroll
          for (int k = 0; k < G; ++k) v[k] = v[k] * (1.0f / G);
        }
      }
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int nr = min(max(n - r * RT, 0), RT);
        if (nr > 0) {
          __syncthreads();
          if (half == r && act) {
            lds_write_tile<G, TOut>(row, v);
            if (flag) {  // element d takes y_0, element 0 takes y_d
              const uint32_t y0 = lds_elem_bits<TOut>(row, 0), yd = lds_elem_bits<TOut>(row, piv);
              lds_elem_set<TOut>(row, piv, y0);
              lds_elem_set<TOut>(row, 0, yd);
            }
          }
          __syncthreads();
          rows_out<RO::kBytes, kStride>(st, a.y + (t0 + r * RT) * RO::kBytes, nr);
        }
      }
    }
  }
}

// One workgroup per group of 64 tiles. Against a persistent grid of the
// resident workgroups (each taking every gridDim.x-th group, with the next
// group prefetched), the hardware dispatcher then balances the load and no
// workgroup is left with an extra group at the end: 8192 x 8192 bf16 round
// trip 61.2 -> 58.1 us (66.5 -> 60.7 us in the first launches after an idle
// spell), 16384 x 4096 63.5 -> 60.6 us, 16384 x 5120 fp32 at tile 128 164.7
// -> 155.8 us, encode only 42.4 -> 40.5 us (one box, interleaved); one
// workgroup per two or three groups fell in between.
template <typename TIn, int OUT, int MODE>
static hipError_t launch_128(const EncArgs& a, hipStream_t st) {
  constexpr int NT = 64;
  const int64_t nwg = a.tiles > 0 ? (a.tiles + NT - 1) / NT : 1;
  hipLaunchKernelGGL((k_encode128<TIn, OUT, MODE>), dim3((unsigned)nwg), dim3(NT), 0, st, a);
  return hipGetLastError();
}

template <int G, typename TIn, int OUT, int MODE>
static hipError_t launch_one(const EncArgs& a, hipStream_t st) {
  if constexpr (G == 128) return launch_128<TIn, OUT, MODE>(a, st);
  constexpr int NT = 64;
  const int64_t nwg = a.tiles > 0 ? (a.tiles + NT - 1) / NT : 1;
  hipLaunchKernelGGL((k_encode<G, TIn, OUT, MODE>), dim3((unsigned)nwg), dim3(NT), 0, st, a);
  return hipGetLastError();
}

template <int G, typename TIn, int MODE>
static hipError_t dispatch_mode(const EncArgs& a, int out, hipStream_t st) {
  if (out == 1) return launch_one<G, TIn, 1, MODE>(a, st);
  if (out == 2) return launch_one<G, TIn, 2, MODE>(a, st);
  return launch_one<G, TIn, 0, MODE>(a, st);
}

template <int G, typename TIn>
static hipError_t dispatch_out(const EncArgs& a, int out, int mode, hipStream_t st) {
  if (mode == 2) return dispatch_mode<G, TIn, 2>(a, out, st);
  if (mode == 1) return dispatch_mode<G, TIn, 1>(a, out, st);
  return dispatch_mode<G, TIn, 0>(a, out, st);
}

hipError_t launch_encode(const Plan& pl, const void* x, void* payload, void* y, int y_dtype, void* ws,
                         hipStream_t st, int mode) {
  const bool mixed = mode != 0;
  EncArgs a;
  a.x = static_cast<const uint8_t*>(x);
  a.y = static_cast<uint8_t*>(y);
  a.payload = static_cast<uint8_t*>(payload);
  uint8_t* w = static_cast<uint8_t*>(ws);
  if (payload) {
    a.table = reinterpret_cast<uint32_t*>(a.payload + pl.off_table);
    a.bitmap = reinterpret_cast<uint32_t*>(a.payload + pl.off_bitmap);
  } else if (mixed) {
    a.table = reinterpret_cast<uint32_t*>(w + pl.ws_table);
    a.bitmap = reinterpret_cast<uint32_t*>(w + pl.ws_bitmap);
  } else {
    a.table = nullptr;
    a.bitmap = nullptr;
  }
  // the uniform-width kernel writes quantization-tile entropies: the entropy
  // area when allocation tiles are quantization tiles, else the sum area
  a.H = reinterpret_cast<float*>(w + (pl.kA > 1 ? pl.ws_LS : pl.ws_H));
  a.side_in = payload ? a.payload + pl.off_side : w + pl.ws_side;
  a.tiles = pl.tiles;
  a.off_side = pl.off_side;
  a.off_scale = pl.off_scale;
  a.off_zero = pl.off_zero;
  a.off_codes = pl.off_codes;
  a.b_lo = pl.b_lo;
  a.b_hi = pl.b_hi;
  a.map_words = 2;  // two-width layout: 1 bit per tile, none at b_hi
  a.map_fill = 0u;
  a.table_step = 0u;
  if (pl.allocator == TAH_ALLOC_GREEDY && mode == 0) {
    // any-width layout with every tile at level glevel: 2-bit map entries all
    // glevel, and the block table's running width sums grow by 64 widths a run
    const int c = pl.candidates[pl.glevel];
    a.b_lo = a.b_hi = c;
    a.map_words = 4;
    a.map_fill = (uint32_t)pl.glevel * 0x55555555u;
    a.table_step = 64u * (uint32_t)c;
  }
  a.sz_lo = pl.G * a.b_lo / 8;
  a.sz_hi = pl.G * a.b_hi / 8;
  a.cands = 0;
  for (int i = 0; i < pl.n_candidates; ++i) a.cands |= (uint32_t)pl.candidates[i] << (8 * i);
  a.wtotal = reinterpret_cast<const uint32_t*>(w + pl.ws_wtotal);
  a.code_end = pl.off_codes + pl.code_bytes;
  a.tau = pl.tau;
  make_header(pl, &a.hdr);
  make_pads(pl, &a.pads);
  const int out = y ? (y_dtype == TAH_DTYPE_F32 ? 1 : 2) : 0;
  const bool bf = pl.x_dtype == TAH_DTYPE_BF16;
  switch (pl.G) {
    case 32: return bf ? dispatch_out<32, bf16_t>(a, out, mode, st) : dispatch_out<32, float>(a, out, mode, st);
    case 64: return bf ? dispatch_out<64, bf16_t>(a, out, mode, st) : dispatch_out<64, float>(a, out, mode, st);
    case 128: return bf ? dispatch_out<128, bf16_t>(a, out, mode, st) : dispatch_out<128, float>(a, out, mode, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace tah
