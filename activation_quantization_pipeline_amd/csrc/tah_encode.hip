// Encode and fused encode+decode kernels of the TAH-Quant codec for gfx950.
//
// One workgroup takes NT consecutive tiles (NT lanes, one tile per lane):
//  1. stage:   the NT tiles (contiguous in HBM) are copied into padded LDS
//              rows with 16-byte coalesced loads;
//  2. phase A: lane i reads tile i from LDS and computes the outlier ratio of
//              Eq. (3) (top-2 magnitudes, pivot d, flag), and, for a uniform
//              allocation, the tile entropy of Eq. (1)-(2); with a mixed
//              allocation the width bit comes from the selection pass instead.
//              It fixes the tile's code-block offset (§3.4 packing order);
//  3. compact: tiles are regrouped by class (transformed or not x width) so
//              that whole wavefronts take the same branch: the Hadamard path
//              of §3.3 then runs only in the waves that hold flagged tiles;
//  4. phase B: each lane re-reads its assigned tile, applies the pivot swap
//              (P_d, done in LDS) and the register FWHT (Eq. 4) if flagged,
//              quantizes asymmetrically, packs the codes and stores code block,
//              scale and zero-point; the fused variant dequantizes from the
//              codes in registers, inverts the transform (H^T / G, undo swap)
//              and writes the tile back to LDS;
//  5. out:     the rebuilt tiles leave LDS with 16-byte coalesced stores.
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
  int64_t tiles;
  int64_t off_side, off_scale, off_zero, off_codes;
  int32_t b_lo, b_hi, sz_lo, sz_hi;
  float tau;
  Header hdr;
  PadRanges pads;
};

template <int G, typename T>
constexpr int tiles_per_wg() {
  return TileRow<G, T>::kBytes <= 128 ? 256 : (TileRow<G, T>::kBytes <= 256 ? 128 : 64);
}

// Rebuilt tile into its LDS row (T), then the pivot swap is undone in place.
template <int G, typename T>
__device__ __forceinline__ void write_y_row(uint8_t* row, const float (&v)[G], int flag, int piv) {
  lds_write_tile<G, T>(row, v);
  if (flag) {
    const uint32_t yd = lds_elem_bits<T>(row, piv);
    lds_elem_set<T>(row, piv, f32_to_elem_bits<T>(v[0]));
    lds_elem_set<T>(row, 0, yd);
  }
}

// Minimum waves per SIMD the register allocator must leave room for.
template <int G, typename T>
constexpr int kMinWaves() {
  return G <= 64 ? 3 : 1;
}

template <int G, int B>
__device__ __forceinline__ void store_codes(const uint32_t (&mq)[G], uint8_t* dst) {
  constexpr int W = G * B / 32;
  uint32_t w[W];
  pack_codes<G, B>(mq, w);
  // Every code block offset is a multiple of G*B/8 bytes past a 256-byte aligned base.
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

__device__ __forceinline__ uint32_t umed3(uint32_t a, uint32_t b, uint32_t c) {
  return max(min(a, b), min(max(a, b), c));
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
        const uint32_t xl = u[i] << 16, xh = u[i] & 0xffff0000u;
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

// OUT: 0 = no reconstruction, 1 = fp32, 2 = bf16.
// Persistent workgroups: group g of NT tiles is processed by workgroup
// g mod gridDim.x; while a group is being processed, the next group's tiles
// are already on their way from HBM into registers.
template <int G, typename TIn, int OUT, bool MIXED>
__global__ __launch_bounds__((tiles_per_wg<G, TIn>()), (kMinWaves<G, TIn>())) void k_encode(EncArgs a) {
  constexpr int NT = tiles_per_wg<G, TIn>();
  constexpr int NW = NT / 64;
  using RI = TileRow<G, TIn>;
  using TOut = typename std::conditional<OUT == 1, float, bf16_t>::type;
  using RO = TileRow<G, TOut>;
  constexpr int kRowMax = (OUT != 0 && RO::kStride > RI::kStride) ? RO::kStride : RI::kStride;
  // After compaction every LDS row is read and rewritten by the one lane that
  // owns it, so a rebuilt tile can go straight back into its own row when the
  // output row is not wider than the input row.
  constexpr bool kSameRow = RO::kStride == RI::kStride;

  __shared__ __attribute__((aligned(16))) uint8_t xs[NT * kRowMax];
  __shared__ uint32_t meta_off[NT];
  __shared__ uint8_t meta_side[NT];
  __shared__ uint8_t meta_hi[NT];
  __shared__ uint16_t perm[NT];
  __shared__ int cnt[NW][4];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  if (blockIdx.x == 0 && a.payload) {
    if (tid < 32) reinterpret_cast<uint32_t*>(a.payload)[tid] = a.hdr.w[tid];
    for (int r = 0; r < a.pads.n; ++r)
      for (int i = tid; i < a.pads.len[r]; i += NT) a.payload[a.pads.off[r] + i] = 0;
  }

  const int64_t ngroups = (a.tiles + NT - 1) / NT;
  int64_t g = blockIdx.x;
  GroupRegs<G, TIn> pre;
  if (g < ngroups) {
    const int64_t t0 = g * NT;
    group_load<G, TIn, NT>(a.x + t0 * RI::kBytes, (int)min<int64_t>(NT, a.tiles - t0), pre);
  }

  for (; g < ngroups; g += gridDim.x) {
    const int64_t t0 = g * NT;
    const int n = (int)min<int64_t>(NT, a.tiles - t0);
    group_to_lds<G, TIn, NT>(pre, xs, n);
    __syncthreads();
    {  // prefetch the next group of this workgroup
      const int64_t gn = g + gridDim.x;
      if (gn < ngroups) {
        const int64_t tn = gn * NT;
        group_load<G, TIn, NT>(a.x + tn * RI::kBytes, (int)min<int64_t>(NT, a.tiles - tn), pre);
      }
    }

    // ---------------- phase A: lane tid owns tile t0 + tid ----------------
    const bool act = tid < n;
    const int64_t t = t0 + tid;
    int flag = 0, piv = 0, hi = 0;
    if (act) {
      float v[G];
      float m1, m2, l1;
      int d;
      tile_stats<G, TIn>(xs + tid * RI::kStride, v, m1, m2, d, l1);
      flag = m1 > a.tau * (m2 + kRho);  // Eq. (3) without the division
      piv = d;
      if constexpr (!MIXED) {
        // Eq. (1)-(2): p_k = |a_k| / (L1 + eps), H = -sum p_k log2(p_k + sigma)
        const float r = 1.0f / (l1 + kEps);
        float acc = 0.0f;
#pragma unroll
        for (int k = 0; k < G; ++k) {
          const float p = fabsf(v[k]) * r;
          acc = __builtin_fmaf(p, log2s(p + kSigma), acc);
        }
        a.H[t] = 0.0f - acc;
      } else {
        hi = (a.bitmap[t >> 5] >> (t & 31)) & 1u;
      }
      if (a.payload) a.payload[a.off_side + t] = (uint8_t)((flag << 7) | piv);
    }

    // Code-block offsets: tile t starts at t*sz_lo + (b_hi tiles before t)*(sz_hi - sz_lo).
    const uint64_t hmask = ballot(act && hi);
    uint32_t rel_off = (uint32_t)tid * (uint32_t)a.sz_lo;
    int64_t wg_off = t0 * a.sz_lo;
    if constexpr (MIXED) {
      const uint32_t hb_wg = a.table[t0 >> 6];
      const uint32_t hb = (t0 + 64 * wave < a.tiles ? a.table[(t0 >> 6) + wave] : hb_wg) + lanes_below(hmask);
      rel_off += (hb - hb_wg) * (uint32_t)(a.sz_hi - a.sz_lo);
      wg_off += (int64_t)hb_wg * (a.sz_hi - a.sz_lo);
    } else {
      // uniform allocation: no tile has b_hi
      if (lane == 0 && a.bitmap && t0 + 64 * wave < a.tiles) {
        const int64_t blk = (t0 >> 6) + wave;
        a.bitmap[2 * blk] = 0u;
        a.bitmap[2 * blk + 1] = 0u;
        a.table[blk] = 0u;
      }
    }

    // ---------------- compaction by class ----------------
    const int cls = act ? (flag | (hi << 1)) : 4;
    const uint64_t b0 = ballot(cls == 0), b1 = ballot(cls == 1), b2 = ballot(cls == 2), b3 = ballot(cls == 3);
    if (lane == 0) {
      cnt[wave][0] = __popcll(b0);
      cnt[wave][1] = __popcll(b1);
      cnt[wave][2] = __popcll(b2);
      cnt[wave][3] = __popcll(b3);
    }
    meta_off[tid] = rel_off;
    meta_side[tid] = (uint8_t)((flag << 7) | piv);
    meta_hi[tid] = (uint8_t)hi;
    __syncthreads();
    if (act) {
      int dst = 0;
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int w = 0; w < NW; ++w) dst += (c < cls || (c == cls && w < wave)) ? cnt[w][c] : 0;
      const uint64_t mine = cls == 0 ? b0 : cls == 1 ? b1 : cls == 2 ? b2 : b3;
      dst += (int)lanes_below(mine);
      perm[dst] = (uint16_t)tid;
    }
    __syncthreads();

    // ---------------- phase B: lane tid takes tile j = perm[tid] ----------------
    float v[G];
    int j = 0;
    flag = 0;
    piv = 0;
    if (act) {
      j = perm[tid];
      const uint32_t side = meta_side[j];
      flag = side >> 7;
      piv = side & 127;
      hi = meta_hi[j];
      uint8_t* row = xs + j * RI::kStride;
      uint32_t xd = 0;
      if (flag) {  // pivot swap P_d (§3.3): slot d <- x_0 here, x_d goes to register 0
        const uint32_t x0 = lds_elem_bits<TIn>(row, 0);
        xd = lds_elem_bits<TIn>(row, piv);
        lds_elem_set<TIn>(row, piv, x0);
      }
      lds_read_tile<G, TIn>(row, v);
      if (flag) {
        v[0] = elem_bits_to_f32<TIn>(xd);
        fwht<G>(v);  // Eq. (4) without the 1/sqrt(G)
      }
      // asymmetric quantizer: zero-point lo, step s rounded up to bf16
      float lo = v[0], hv = v[0];
#pragma unroll
      for (int k = 1; k < G; ++k) {
        lo = fminf(lo, v[k]);
        hv = fmaxf(hv, v[k]);
      }
      lo = lo + 0.0f;
      hv = hv + 0.0f;
      const int b = hi ? a.b_hi : a.b_lo;
      const float L = (float)((1 << b) - 1);
      uint32_t sb = __float_as_uint((hv - lo) / L);
      if (sb & 0xffffu) sb = (sb & 0xffff0000u) + 0x10000u;
      float s = __uint_as_float(sb);
      if (!(s >= 0x1p-126f)) s = 0.0f;
      const float inv = s > 0.0f ? 1.0f / s : 0.0f;
      // q_k = round-half-even of the exact (y_k - lo) * inv: one fused rounding against 2^23
      uint32_t mq[G];
#pragma unroll
      for (int k = 0; k < G; ++k) mq[k] = __float_as_uint(__builtin_fmaf(v[k] - lo, inv, 0x1p23f));
      if (a.payload) {
        const int64_t tj = t0 + j;
        store_codes_b<G>(b, mq, a.payload + a.off_codes + wg_off + meta_off[j]);
        reinterpret_cast<uint16_t*>(a.payload + a.off_scale)[tj] = (uint16_t)(__float_as_uint(s) >> 16);
        reinterpret_cast<float*>(a.payload + a.off_zero)[tj] = lo;
      }
      if constexpr (OUT != 0) {
        // receiver side (Algorithm 1 line 5) from the codes held in registers
#pragma unroll
        for (int k = 0; k < G; ++k) v[k] = __builtin_fmaf(__uint_as_float(mq[k]) - 0x1p23f, s, lo);
        if (flag) {
          fwht<G>(v);
#pragma unroll
          for (int k = 0; k < G; ++k) v[k] = v[k] * (1.0f / G);
        }
        if constexpr (kSameRow) write_y_row<G, TOut>(xs + j * RO::kStride, v, flag, piv);
      }
    }

    if constexpr (OUT != 0) {
      if constexpr (!kSameRow) {
        // wider output rows overlap other lanes' input rows: wait for every read
        __syncthreads();
        if (act) write_y_row<G, TOut>(xs + j * RO::kStride, v, flag, piv);
      }
      __syncthreads();
      stage_out<G, TOut, NT>(xs, a.y + t0 * RO::kBytes, n);
    }
    __syncthreads();  // LDS is rewritten by the next group
  }
}

// Resident workgroups per CU of a kernel, from the runtime's occupancy query.
template <typename K>
static int wgs_per_cu(K kernel, int threads) {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, threads, 0) != hipSuccess || n < 1) n = 1;
  return n;
}

static int cu_count() {
  static int cus = 0;
  if (!cus) {
    int dev = 0;
    hipGetDevice(&dev);
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) cus = 256;
  }
  return cus;
}

template <int G, typename TIn, int OUT, bool MIXED>
static hipError_t launch_one(const EncArgs& a, hipStream_t st) {
  constexpr int NT = tiles_per_wg<G, TIn>();
  static const int per_cu = wgs_per_cu(k_encode<G, TIn, OUT, MIXED>, NT);
  const int64_t ngroups = a.tiles > 0 ? (a.tiles + NT - 1) / NT : 1;
  const int64_t resident = (int64_t)per_cu * cu_count();
  const int64_t nwg = ngroups < resident ? ngroups : resident;
  hipLaunchKernelGGL((k_encode<G, TIn, OUT, MIXED>), dim3((unsigned)nwg), dim3(NT), 0, st, a);
  return hipGetLastError();
}

template <int G, typename TIn>
static hipError_t dispatch_out(const EncArgs& a, int out, bool mixed, hipStream_t st) {
  if (mixed) {
    if (out == 1) return launch_one<G, TIn, 1, true>(a, st);
    if (out == 2) return launch_one<G, TIn, 2, true>(a, st);
    return launch_one<G, TIn, 0, true>(a, st);
  }
  if (out == 1) return launch_one<G, TIn, 1, false>(a, st);
  if (out == 2) return launch_one<G, TIn, 2, false>(a, st);
  return launch_one<G, TIn, 0, false>(a, st);
}

hipError_t launch_encode(const Plan& pl, const void* x, void* payload, void* y, int y_dtype, void* ws,
                         hipStream_t st, bool mixed) {
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
  a.H = reinterpret_cast<float*>(w + pl.ws_H);
  a.tiles = pl.tiles;
  a.off_side = pl.off_side;
  a.off_scale = pl.off_scale;
  a.off_zero = pl.off_zero;
  a.off_codes = pl.off_codes;
  a.b_lo = pl.b_lo;
  a.b_hi = pl.b_hi;
  a.sz_lo = pl.G * pl.b_lo / 8;
  a.sz_hi = pl.G * pl.b_hi / 8;
  a.tau = pl.tau;
  make_header(pl, &a.hdr);
  make_pads(pl, &a.pads);
  const int out = y ? (y_dtype == TAH_DTYPE_F32 ? 1 : 2) : 0;
  const bool bf = pl.x_dtype == TAH_DTYPE_BF16;
  switch (pl.G) {
    case 32: return bf ? dispatch_out<32, bf16_t>(a, out, mixed, st) : dispatch_out<32, float>(a, out, mixed, st);
    case 64: return bf ? dispatch_out<64, bf16_t>(a, out, mixed, st) : dispatch_out<64, float>(a, out, mixed, st);
    case 128: return bf ? dispatch_out<128, bf16_t>(a, out, mixed, st) : dispatch_out<128, float>(a, out, mixed, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace tah
