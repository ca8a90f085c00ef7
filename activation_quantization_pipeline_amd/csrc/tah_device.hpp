// Device building blocks of the TAH-Quant kernels for CDNA4 (gfx950, wave64).
//
// Layout decision: one lane owns one whole tile (G contiguous channels of one
// token). Tiles are staged through LDS so that HBM traffic stays fully
// coalesced (16 bytes per lane, contiguous per wave), and every per-tile step
// of the method — top-2 and pivot (Eq. 3), L1 norm and entropy (Eq. 1-2), the
// Hadamard butterflies (Eq. 4), min/max, codes and bit packing — then runs in
// the lane's own registers with no cross-lane traffic.
//
// The fp32 operation order of every step is fixed (stated at each routine),
// so the results are reproducible bit for bit. Build with -ffp-contract=off;
// every fused multiply-add below is an explicit fmaf.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace tah {

// ϱ of Eq. (3) (TAH-Quant §3.3): a small positive constant, 2^-40. The ε of
// Eq. (1) and ς of Eq. (2) only keep zeros finite; the entropy below handles
// zeros explicitly instead.
constexpr float kRho = 0x1p-40f;

typedef uint16_t bf16_t;

__device__ __forceinline__ float bf16_to_f32(uint32_t h16) { return __uint_as_float(h16 << 16); }

// fp32 -> bf16, round to nearest even (finite values).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// Two fp32 -> two bf16 (round to nearest even) in one v_cvt_pk_bf16_f32.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// Tables of the entropy's log2, j = 0..127 (the top 7 stored mantissa bits):
//   kLog2Tab[j]       = fp32(log2(1 + j/128) - 1)
//   kLog2Tab[128 + j] = fp32((log2(1 + (j+1)/128) - log2(1 + j/128)) / 2^16)
// each computed in double precision and rounded once to fp32.
__device__ const float kLog2Tab[256] = {
    -0x1p+0f, -0x1.fa406cp-1f, -0x1.f48c34p-1f, -0x1.eee32ep-1f,
    -0x1.e9452cp-1f, -0x1.e3b206p-1f, -0x1.de298ep-1f, -0x1.d8abap-1f,
    -0x1.d33812p-1f, -0x1.cdcebep-1f, -0x1.c86f7cp-1f, -0x1.c31a28p-1f,
    -0x1.bdce9ep-1f, -0x1.b88cbap-1f, -0x1.b35458p-1f, -0x1.ae2558p-1f,
    -0x1.a8ff98p-1f, -0x1.a3e2f4p-1f, -0x1.9ecf5p-1f, -0x1.99c48cp-1f,
    -0x1.94c288p-1f, -0x1.8fc924p-1f, -0x1.8ad846p-1f, -0x1.85efdp-1f,
    -0x1.810fa6p-1f, -0x1.7c37aap-1f, -0x1.7767c2p-1f, -0x1.729fd2p-1f,
    -0x1.6ddfc2p-1f, -0x1.692778p-1f, -0x1.6476dap-1f, -0x1.5fcdcep-1f,
    -0x1.5b2c3ep-1f, -0x1.56921p-1f, -0x1.51ff2ep-1f, -0x1.4d738p-1f,
    -0x1.48eef2p-1f, -0x1.44716ap-1f, -0x1.3ffad4p-1f, -0x1.3b8b1cp-1f,
    -0x1.37222cp-1f, -0x1.32bfeep-1f, -0x1.2e645p-1f, -0x1.2a0f3cp-1f,
    -0x1.25c0ap-1f, -0x1.217868p-1f, -0x1.1d3682p-1f, -0x1.18fadcp-1f,
    -0x1.14c56p-1f, -0x1.109602p-1f, -0x1.0c6caap-1f, -0x1.08494cp-1f,
    -0x1.042bd4p-1f, -0x1.001434p-1f, -0x1.f804aep-2f, -0x1.efec62p-2f,
    -0x1.e7df6p-2f, -0x1.dfdd8ap-2f, -0x1.d7e6cp-2f, -0x1.cffae6p-2f,
    -0x1.c819dcp-2f, -0x1.c04386p-2f, -0x1.b877c6p-2f, -0x1.b0b68p-2f,
    -0x1.a8ff98p-2f, -0x1.a152f2p-2f, -0x1.99b072p-2f, -0x1.9218p-2f,
    -0x1.8a898p-2f, -0x1.8304dap-2f, -0x1.7b89fp-2f, -0x1.7418acp-2f,
    -0x1.6cb0f6p-2f, -0x1.6552b4p-2f, -0x1.5dfddp-2f, -0x1.56b22ep-2f,
    -0x1.4f6fbcp-2f, -0x1.48365ep-2f, -0x1.410602p-2f, -0x1.39de8ep-2f,
    -0x1.32bfeep-2f, -0x1.2baa0cp-2f, -0x1.249cd2p-2f, -0x1.1d982cp-2f,
    -0x1.169c06p-2f, -0x1.0fa848p-2f, -0x1.08bcep-2f, -0x1.01d9bcp-2f,
    -0x1.f5fd8ap-3f, -0x1.e857d4p-3f, -0x1.dac22ep-3f, -0x1.cd3c72p-3f,
    -0x1.bfc67ap-3f, -0x1.b26024p-3f, -0x1.a5094cp-3f, -0x1.97c1ccp-3f,
    -0x1.8a898p-3f, -0x1.7d604ap-3f, -0x1.704604p-3f, -0x1.633a8cp-3f,
    -0x1.563dc2p-3f, -0x1.494f86p-3f, -0x1.3c6fb6p-3f, -0x1.2f9e32p-3f,
    -0x1.22dadcp-3f, -0x1.162594p-3f, -0x1.097e38p-3f, -0x1.f9c95ep-4f,
    -0x1.e0b1aep-4f, -0x1.c7b528p-4f, -0x1.aed392p-4f, -0x1.960cbp-4f,
    -0x1.7d604ap-4f, -0x1.64ce26p-4f, -0x1.4c561p-4f, -0x1.33f7cep-4f,
    -0x1.1bb32ap-4f, -0x1.0387fp-4f, -0x1.d6ebd2p-5f, -0x1.a6f9c4p-5f,
    -0x1.77394cp-5f, -0x1.47aa08p-5f, -0x1.184b8ep-5f, -0x1.d23afcp-6f,
    -0x1.743ee8p-6f, -0x1.16a21ep-6f, -0x1.72c7bap-7f, -0x1.720d9cp-8f,
    0x1.6fe50cp-23f, 0x1.6d0dc6p-23f, 0x1.6a41a4p-23f, 0x1.678068p-23f,
    0x1.64c9dp-23f, 0x1.621da2p-23f, 0x1.5f7b9ep-23f, 0x1.5ce38ep-23f,
    0x1.5a553ap-23f, 0x1.57d06ap-23f, 0x1.5554e8p-23f, 0x1.52e284p-23f,
    0x1.50790ap-23f, 0x1.4e184cp-23f, 0x1.4bc018p-23f, 0x1.49704p-23f,
    0x1.47289ap-23f, 0x1.44e8fcp-23f, 0x1.42b138p-23f, 0x1.408126p-23f,
    0x1.3e58ap-23f, 0x1.3c377ep-23f, 0x1.3a1d9cp-23f, 0x1.380ad2p-23f,
    0x1.35fefep-23f, 0x1.33f9fep-23f, 0x1.31fbbp-23f, 0x1.3003fp-23f,
    0x1.2e12a2p-23f, 0x1.2c27a4p-23f, 0x1.2a42d8p-23f, 0x1.286422p-23f,
    0x1.268b6p-23f, 0x1.24b87cp-23f, 0x1.22eb54p-23f, 0x1.2123d2p-23f,
    0x1.1f61dap-23f, 0x1.1da552p-23f, 0x1.1bee2p-23f, 0x1.1a3c2cp-23f,
    0x1.188f6p-23f, 0x1.16e7a2p-23f, 0x1.1544dep-23f, 0x1.13a6fcp-23f,
    0x1.120de6p-23f, 0x1.107986p-23f, 0x1.0ee9cap-23f, 0x1.0d5e9cp-23f,
    0x1.0bd7e8p-23f, 0x1.0a559cp-23f, 0x1.08d7a2p-23f, 0x1.075decp-23f,
    0x1.05e864p-23f, 0x1.0476fap-23f, 0x1.03099cp-23f, 0x1.01a03ap-23f,
    0x1.003ac2p-23f, 0x1.fdb24ap-24f, 0x1.faf6a6p-24f, 0x1.f8427ap-24f,
    0x1.f595a4p-24f, 0x1.f2f008p-24f, 0x1.f0518ap-24f, 0x1.edba0ep-24f,
    0x1.eb2976p-24f, 0x1.e89fa6p-24f, 0x1.e61c86p-24f, 0x1.e39ffap-24f,
    0x1.e129e8p-24f, 0x1.deba38p-24f, 0x1.dc50dp-24f, 0x1.d9ed9ap-24f,
    0x1.d7907cp-24f, 0x1.d5395ep-24f, 0x1.d2e82cp-24f, 0x1.d09cdp-24f,
    0x1.ce573p-24f, 0x1.cc173cp-24f, 0x1.c9dcdap-24f, 0x1.c7a7f8p-24f,
    0x1.c5788p-24f, 0x1.c34e6p-24f, 0x1.c12984p-24f, 0x1.bf09dap-24f,
    0x1.bcef4cp-24f, 0x1.bad9cap-24f, 0x1.b8c942p-24f, 0x1.b6bda2p-24f,
    0x1.b4b6d8p-24f, 0x1.b2b4d2p-24f, 0x1.b0b782p-24f, 0x1.aebed6p-24f,
    0x1.accabep-24f, 0x1.aadb28p-24f, 0x1.a8f008p-24f, 0x1.a7094cp-24f,
    0x1.a526e8p-24f, 0x1.a348cap-24f, 0x1.a16ee6p-24f, 0x1.9f992ap-24f,
    0x1.9dc78cp-24f, 0x1.9bf9fep-24f, 0x1.9a307p-24f, 0x1.986ad6p-24f,
    0x1.96a922p-24f, 0x1.94eb4ap-24f, 0x1.93313ep-24f, 0x1.917af4p-24f,
    0x1.8fc85ep-24f, 0x1.8e197p-24f, 0x1.8c6e22p-24f, 0x1.8ac662p-24f,
    0x1.89222ap-24f, 0x1.87816ep-24f, 0x1.85e42p-24f, 0x1.844a38p-24f,
    0x1.82b3aap-24f, 0x1.81206cp-24f, 0x1.7f9074p-24f, 0x1.7e03b6p-24f,
    0x1.7c7a2cp-24f, 0x1.7af3c8p-24f, 0x1.797082p-24f, 0x1.77f05p-24f,
    0x1.76732ap-24f, 0x1.74f904p-24f, 0x1.7381d8p-24f, 0x1.720d9cp-24f,
};

// Copy kLog2Tab into LDS (every lane of a 64-lane workgroup takes 4 entries).
__device__ __forceinline__ void load_log2_tab(float* lt) {
  const float4 v = reinterpret_cast<const float4*>(kLog2Tab)[threadIdx.x & 63];
  if (threadIdx.x < 64) reinterpret_cast<float4*>(lt)[threadIdx.x] = v;
}

// log2 of the entropy (TAH-Quant §3.2, Eq. 2 writes "log"; the base does not
// change the ranking). x = m 2^E with m in [0.5, 1) (frexp; E = 0 for x = 0),
// j = bits 16..22 of x, w = bits 0..15:
//   log2(x) = fmaf((float)w, D[j], (float)E + T[j]),   lt = {T, D} in LDS.
// log2_node is the same for x with w = 0 (every widened bf16 value, which
// sits on a node of the table): the fma would add an exact zero to a sum that
// is never -0, so it is left out, and the table offset j * 4 is one bit-field
// extract of bits 14..22 (bits 14 and 15 are zero).
__device__ __forceinline__ float log2_node(float x, const float* lt) {
  const uint32_t off = __builtin_amdgcn_ubfe(__float_as_uint(x), 14u, 9u);
  const float t = *reinterpret_cast<const float*>(reinterpret_cast<const uint8_t*>(lt) + off);
  return (float)__builtin_amdgcn_frexp_expf(x) + t;
}
__device__ __forceinline__ float log2_full(float x, const float* lt) {
  const uint32_t b = __float_as_uint(x);
  const uint32_t j = (b >> 16) & 127u;
  const float base = (float)__builtin_amdgcn_frexp_expf(x) + lt[j];
  return __builtin_fmaf((float)(b & 0xffffu), lt[128 + j], base);
}

// Tile entropy of Eq. (1)-(2) with the minus sign, written as
//   H = log2 L - (1/L) sum_k |a_k| log2 |a_k|,   L = sum_k |a_k|
// (equal to -sum p_k log2 p_k with p_k = |a_k| / L). fp32 order: S summed
// left to right with fmaf from 0, then log2(L) - S / L; L = 0 gives 0.
// NODE: the tile's values are widened bf16 (log2_node applies).
// S = sum_k |a_k| log2 |a_k| of one tile, fma-accumulated left to right from 0.
template <int G, bool NODE>
__device__ __forceinline__ float tile_logsum(const float (&v)[G], const float* lt) {
  float S = 0.0f;
#pragma unroll
  for (int k = 0; k < G; ++k) {
    const float lg = NODE ? log2_node(v[k], lt) : log2_full(fabsf(v[k]), lt);
    S = __builtin_fmaf(fabsf(v[k]), lg, S);
  }
  asm volatile("" : "+v"(S));  // the sum is complete here, ahead of the L = 0 test
  return S;
}

template <int G, bool NODE>
__device__ __forceinline__ float tile_entropy(const float (&v)[G], float l1, const float* lt) {
  const float S = tile_logsum<G, NODE>(v, lt);
  return l1 > 0.0f ? log2_full(l1, lt) - S / l1 : 0.0f;
}

// The same entropy from the two sums L = sum |a_k| and S = sum |a_k| log2 |a_k|.
__device__ __forceinline__ float entropy_from_sums(float l1, float S, const float* lt) {
  asm volatile("" : "+v"(S));
  return l1 > 0.0f ? log2_full(l1, lt) - S / l1 : 0.0f;
}

// Unnormalized Sylvester Walsh-Hadamard transform in registers, v <- H_G v
// (H_G[i][j] = (-1)^popcount(i & j)); stages h = 1, 2, ..., G/2, butterfly
// (a, b) -> (a + b, a - b). Fully unrolled: G log2 G adds, no data movement.
template <int G>
__device__ __forceinline__ void fwht(float (&v)[G]) {
#pragma unroll
  for (int h = 1; h < G; h <<= 1) {
#pragma unroll
    for (int j = 0; j < G; ++j) {
      if ((j & h) == 0) {
        float a = v[j], b = v[j + h];
        v[j] = a + b;
        v[j + h] = a - b;
      }
    }
  }
}

// Value of v in lane (lane xor M), M in {1, 2, 4, 8}: DPP quad permutes for
// 1 and 2, a bit-mode swizzle for 4 and 8. The partner lane must be active.
template <int M>
__device__ __forceinline__ float xor_lane(float v) {
  const int i = __float_as_int(v);
  if constexpr (M == 1) return __int_as_float(__builtin_amdgcn_mov_dpp(i, 0xB1, 0xF, 0xF, true));  // [1,0,3,2]
  else if constexpr (M == 2) return __int_as_float(__builtin_amdgcn_mov_dpp(i, 0x4E, 0xF, 0xF, true));  // [2,3,0,1]
  else return __int_as_float(__builtin_amdgcn_ds_swizzle(i, 0x1F | (M << 10)));  // and 0x1f, xor M
}

// The same transform as fwht<G> spread over the 16 lanes of an aligned group:
// lane r holds elements [r V, r V + V) of the tile (V = G / 16). Stages
// h < V are butterflies inside the lane; stage h = V M pairs lane r with
// r xor M. Every butterfly is the same single-rounded a + b / a - b as in
// fwht<G>, in the same stage order, so the results are identical.
template <int V>
__device__ __forceinline__ void fwht16(float (&y)[V], int r) {
#pragma unroll
  for (int h = 1; h < V; h <<= 1)
#pragma unroll
    for (int j = 0; j < V; ++j)
      if ((j & h) == 0) {
        const float a = y[j], b = y[j + h];
        y[j] = a + b;
        y[j + h] = a - b;
      }
  // lower lane: own + partner; upper lane: partner - own (fma with -1 rounds once)
  {
    const float sg = (r & 1) ? -1.0f : 1.0f;
#pragma unroll
    for (int i = 0; i < V; ++i) y[i] = __builtin_fmaf(y[i], sg, xor_lane<1>(y[i]));
  }
  {
    const float sg = (r & 2) ? -1.0f : 1.0f;
#pragma unroll
    for (int i = 0; i < V; ++i) y[i] = __builtin_fmaf(y[i], sg, xor_lane<2>(y[i]));
  }
  {
    const float sg = (r & 4) ? -1.0f : 1.0f;
#pragma unroll
    for (int i = 0; i < V; ++i) y[i] = __builtin_fmaf(y[i], sg, xor_lane<4>(y[i]));
  }
  {
    const float sg = (r & 8) ? -1.0f : 1.0f;
#pragma unroll
    for (int i = 0; i < V; ++i) y[i] = __builtin_fmaf(y[i], sg, xor_lane<8>(y[i]));
  }
}

__device__ __forceinline__ uint32_t umed3(uint32_t a, uint32_t b, uint32_t c) {
  return max(min(a, b), min(max(a, b), c));
}

// Statistics of a tile held in registers (Eq. 3 and Eq. 1): m1 = max |a_k|,
// d = the first index holding it, m2 = max |a_k| over k != d, l1 = sum |a_k|
// left to right from 0. NODE: widened bf16 values, whose low 16 bits are zero,
// so the magnitude bits and (G-1-k) share one 32-bit key and unsigned max /
// median give the top two magnitudes and the lowest index among ties.
template <int G, bool NODE>
__device__ __forceinline__ void tile_stats_regs(const float (&v)[G], float& m1, float& m2, int& d, float& l1) {
  if constexpr (NODE) {
    uint32_t k1 = 0u, k2 = 0u;
    float s = 0.0f;
#pragma unroll
    for (int k = 0; k < G; ++k) {
      const uint32_t key = (__float_as_uint(v[k]) & 0x7fff0000u) | (uint32_t)(G - 1 - k);
      s = s + fabsf(v[k]);
      k2 = umed3(k2, key, k1);
      k1 = max(k1, key);
    }
    m1 = __uint_as_float(k1 & 0xffff0000u);
    m2 = __uint_as_float(k2 & 0xffff0000u);
    d = G - 1 - (int)(k1 & 0xffffu);
    l1 = s;
  } else {
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

// Number of lanes below this one whose bit is set in mask.
__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

// Pack G codes of width B into G*B/32 little-endian dwords, code k at stream
// bits [kB, kB + B), least significant bit first. mq[k] holds the code in its
// low bits (higher bits are ignored): v_alignbit shifts the running word right
// and inserts the low bits of the next code at the top, so the codes of each
// output dword are inserted in stream order and bits of a code that belong to
// the previous dword fall out at the bottom.
template <int G, int B>
__device__ __forceinline__ void pack_codes(const uint32_t (&mq)[G], uint32_t (&w)[G * B / 32]) {
#pragma unroll
  for (int i = 0; i < G * B / 32; ++i) {
    const int lo_bit = 32 * i;
    const int k0 = lo_bit / B;
    const int k1 = (lo_bit + 31) / B;
    uint32_t acc = 0;
#pragma unroll
    for (int k = k0; k <= k1; ++k) {
      const int n = (k < k1) ? B : (lo_bit + 32 - k1 * B);
      acc = __builtin_amdgcn_alignbit(mq[k], acc, (uint32_t)n);
    }
    w[i] = acc;
  }
}

// Inverse of pack_codes: code k as an integer.
template <int G, int B>
__device__ __forceinline__ uint32_t unpack_code(const uint32_t (&w)[G * B / 32], int k) {
  const int bit = k * B;
  const int i = bit >> 5, off = bit & 31;
  if (off + B <= 32) return __builtin_amdgcn_ubfe(w[i], (uint32_t)off, (uint32_t)B);
  return __builtin_amdgcn_ubfe(__builtin_amdgcn_alignbit(w[i + 1], w[i], (uint32_t)off), 0u, (uint32_t)B);
}

// Element type traits for the staged tiles.
template <typename T>
struct Elem;
template <>
struct Elem<float> {
  static constexpr int kBytes = 4;
  static constexpr int kDtype = 0;
};
template <>
struct Elem<bf16_t> {
  static constexpr int kBytes = 2;
  static constexpr int kDtype = 1;
};

// LDS tile row: G elements plus 16 bytes of padding, so that 16-byte reads of
// consecutive lanes' tiles start 4 banks apart (conflict free).
template <int G, typename T>
struct TileRow {
  static constexpr int kBytes = G * Elem<T>::kBytes;
  static constexpr int kStride = kBytes + 16;
  static constexpr int kChunks = kBytes / 16;  // 16-byte chunks per tile
};

// Read a tile from LDS into fp32 registers (bf16 widens exactly).
template <int G, typename T>
__device__ __forceinline__ void lds_read_tile(const uint8_t* row, float (&v)[G]) {
  const uint4* p = reinterpret_cast<const uint4*>(row);
  if constexpr (Elem<T>::kBytes == 4) {
#pragma unroll
    for (int c = 0; c < G / 4; ++c) {
      uint4 q = p[c];
      v[4 * c + 0] = __uint_as_float(q.x);
      v[4 * c + 1] = __uint_as_float(q.y);
      v[4 * c + 2] = __uint_as_float(q.z);
      v[4 * c + 3] = __uint_as_float(q.w);
    }
  } else {
#pragma unroll
    for (int c = 0; c < G / 8; ++c) {
      uint4 q = p[c];
      const uint32_t u[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[8 * c + 2 * i] = __uint_as_float(u[i] << 16);
        v[8 * c + 2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
      }
    }
  }
}

// Write a tile of fp32 registers to LDS as T (bf16: round to nearest even).
template <int G, typename T>
__device__ __forceinline__ void lds_write_tile(uint8_t* row, const float (&v)[G]) {
  uint4* p = reinterpret_cast<uint4*>(row);
  if constexpr (Elem<T>::kBytes == 4) {
#pragma unroll
    for (int c = 0; c < G / 4; ++c)
      p[c] = make_uint4(__float_as_uint(v[4 * c]), __float_as_uint(v[4 * c + 1]), __float_as_uint(v[4 * c + 2]),
                        __float_as_uint(v[4 * c + 3]));
  } else {
#pragma unroll
    for (int c = 0; c < G / 8; ++c)
      p[c] = make_uint4(pack_bf16x2(v[8 * c], v[8 * c + 1]), pack_bf16x2(v[8 * c + 2], v[8 * c + 3]),
                        pack_bf16x2(v[8 * c + 4], v[8 * c + 5]), pack_bf16x2(v[8 * c + 6], v[8 * c + 7]));
  }
}

// One element of an LDS tile, as raw bits (bf16: 16 bits) and as fp32.
template <typename T>
__device__ __forceinline__ uint32_t lds_elem_bits(const uint8_t* row, int k) {
  if constexpr (Elem<T>::kBytes == 4) return reinterpret_cast<const uint32_t*>(row)[k];
  else return reinterpret_cast<const uint16_t*>(row)[k];
}
template <typename T>
__device__ __forceinline__ void lds_elem_set(uint8_t* row, int k, uint32_t bits) {
  if constexpr (Elem<T>::kBytes == 4) reinterpret_cast<uint32_t*>(row)[k] = bits;
  else reinterpret_cast<uint16_t*>(row)[k] = (uint16_t)bits;
}
template <typename T>
__device__ __forceinline__ float elem_bits_to_f32(uint32_t bits) {
  if constexpr (Elem<T>::kBytes == 4) return __uint_as_float(bits);
  else return __uint_as_float(bits << 16);
}
template <typename T>
__device__ __forceinline__ uint32_t f32_to_elem_bits(float f) {
  if constexpr (Elem<T>::kBytes == 4) return __float_as_uint(f);
  else return f32_to_bf16_rne(f);
}

// Elements [r V, r V + V) of an LDS tile row, as fp32 (bf16 widens exactly).
template <int V, typename T>
__device__ __forceinline__ void lds_read_part(const uint8_t* row, int r, float (&y)[V]) {
  if constexpr (Elem<T>::kBytes == 4) {
    const float* p = reinterpret_cast<const float*>(row) + r * V;
#pragma unroll
    for (int i = 0; i < V; ++i) y[i] = p[i];
  } else {
    const uint32_t* p = reinterpret_cast<const uint32_t*>(row) + r * (V / 2);
#pragma unroll
    for (int i = 0; i < V / 2; ++i) {
      const uint32_t u = p[i];
      y[2 * i] = __uint_as_float(u << 16);
      y[2 * i + 1] = __uint_as_float(u & 0xffff0000u);
    }
  }
}

// Elements [r V, r V + V) of an LDS tile row from fp32 (bf16: round to nearest even).
template <int V, typename T>
__device__ __forceinline__ void lds_write_part(uint8_t* row, int r, const float (&y)[V]) {
  if constexpr (Elem<T>::kBytes == 4) {
    float* p = reinterpret_cast<float*>(row) + r * V;
#pragma unroll
    for (int i = 0; i < V; ++i) p[i] = y[i];
  } else {
    uint32_t* p = reinterpret_cast<uint32_t*>(row) + r * (V / 2);
#pragma unroll
    for (int i = 0; i < V / 2; ++i) p[i] = pack_bf16x2(y[2 * i], y[2 * i + 1]);
  }
}

// Streaming accesses with the nontemporal hint: the tensor read by the encoder
// and the tensor written by the encoder and decoder are touched once per call.
// Measured on the 8192 x 8192 bf16 round trip: 67.2 -> 61.0 us, decode
// 39.0 -> 29.5 us. Not used for the statistics pass's reads (the encoder reads
// the same tensor right after it, from the cache) nor for the payload.
typedef uint32_t nt_u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_stream(const uint4* p) {
  const nt_u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const nt_u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void store_stream(uint4* p, const uint4 q) {
  nt_u32x4 v;
  v.x = q.x;
  v.y = q.y;
  v.z = q.z;
  v.w = q.w;
  __builtin_nontemporal_store(v, reinterpret_cast<nt_u32x4*>(p));
}

// A group of NT consecutive tiles held in registers on its way to LDS: thread
// i owns the 16-byte chunks i, i + NT, i + 2 NT, ... of the group, so every
// load instruction of the workgroup reads one contiguous, coalesced block.
template <int G, typename T>
struct GroupRegs {
  uint4 c[TileRow<G, T>::kChunks];
};

template <int G, typename T, int NT>
__device__ __forceinline__ void group_load(const uint8_t* __restrict__ src, int n_tiles, GroupRegs<G, T>& r) {
  using R = TileRow<G, T>;
  const uint4* s = reinterpret_cast<const uint4*>(src);
  // One straight-line path for full and partial groups (n_tiles >= 1): a chunk
  // past the end reloads the last one, which group_to_lds never stores.
  const int last = n_tiles * R::kChunks - 1;
#pragma unroll
  for (int i = 0; i < R::kChunks; ++i) r.c[i] = load_stream(&s[min((int)threadIdx.x + i * NT, last)]);
}

// Makes the compiler wait for the loads of r here (an empty asm that reads them).
template <int G, typename T>
__device__ __forceinline__ void group_wait(const GroupRegs<G, T>& r) {
#pragma unroll
  for (int i = 0; i < TileRow<G, T>::kChunks; ++i)
    asm volatile("" ::"v"(r.c[i].x), "v"(r.c[i].y), "v"(r.c[i].z), "v"(r.c[i].w));
}

template <int G, typename T, int NT>
__device__ __forceinline__ void group_to_lds(const GroupRegs<G, T>& r, uint8_t* lds, int n_tiles) {
  using R = TileRow<G, T>;
  static_assert(NT % R::kChunks == 0, "a pass of NT chunks covers whole tiles");
  const int nchunks = n_tiles * R::kChunks;
  // chunk threadIdx.x + i NT lands in row threadIdx.x / kChunks + i NT / kChunks
  uint8_t* base = lds + (threadIdx.x / R::kChunks) * R::kStride + (threadIdx.x % R::kChunks) * 16;
#pragma unroll
  for (int i = 0; i < R::kChunks; ++i) {
    if (n_tiles == NT || (int)threadIdx.x + i * NT < nchunks)
      *reinterpret_cast<uint4*>(base + i * (NT / R::kChunks) * R::kStride) = r.c[i];
  }
}

// Copy n_tiles contiguous tiles (global, 16-byte aligned) into padded LDS rows.
template <int G, typename T, int NT>
__device__ __forceinline__ void stage_in(const uint8_t* __restrict__ src, uint8_t* lds, int n_tiles) {
  using R = TileRow<G, T>;
  const int nchunks = n_tiles * R::kChunks;
  const uint4* s = reinterpret_cast<const uint4*>(src);
  if (n_tiles == NT) {
    constexpr int per = NT * R::kChunks / NT;  // chunks per thread
    uint4 buf[per];
#pragma unroll
    for (int i = 0; i < per; ++i) buf[i] = s[threadIdx.x + i * NT];
#pragma unroll
    for (int i = 0; i < per; ++i) {
      const int c = threadIdx.x + i * NT;
      *reinterpret_cast<uint4*>(lds + (c / R::kChunks) * R::kStride + (c % R::kChunks) * 16) = buf[i];
    }
  } else {
    for (int c = threadIdx.x; c < nchunks; c += NT)
      *reinterpret_cast<uint4*>(lds + (c / R::kChunks) * R::kStride + (c % R::kChunks) * 16) = s[c];
  }
}

// Copy n_tiles padded LDS rows out to contiguous global memory.
template <int G, typename T, int NT>
__device__ __forceinline__ void stage_out(const uint8_t* lds, uint8_t* __restrict__ dst, int n_tiles) {
  using R = TileRow<G, T>;
  static_assert(NT % R::kChunks == 0, "a pass of NT chunks covers whole tiles");
  const int nchunks = n_tiles * R::kChunks;
  const uint8_t* base = lds + (threadIdx.x / R::kChunks) * R::kStride + (threadIdx.x % R::kChunks) * 16;
  uint4* d = reinterpret_cast<uint4*>(dst) + threadIdx.x;
  // every LDS read first (rows past n_tiles hold stale data and are not
  // stored), so one wait covers them all instead of one per store
  uint4 buf[R::kChunks];
#pragma unroll
  for (int i = 0; i < R::kChunks; ++i) buf[i] = *reinterpret_cast<const uint4*>(base + i * (NT / R::kChunks) * R::kStride);
#pragma unroll
  for (int i = 0; i < R::kChunks; ++i) {
    if (n_tiles == NT || (int)threadIdx.x + i * NT < nchunks) store_stream(&d[i * NT], buf[i]);
  }
}

}  // namespace tah
