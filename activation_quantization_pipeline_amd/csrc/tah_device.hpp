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

// ε (Eq. 1), ς (Eq. 2), ϱ (Eq. 3) of TAH-Quant §3.2-3.3: small positive constants, 2^-40 each.
constexpr float kEps = 0x1p-40f;
constexpr float kSigma = 0x1p-40f;
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

// log2 for the entropy (TAH-Quant §3.2, Eq. 2 writes "log"; the base does not
// change the ranking). u = m 2^e, m in [0.5, 1): f = 2m - 1 in [0, 1) exactly,
// log2 u = (e - 1) + log2(1 + f), with log2(1 + f) replaced by the degree-5
// minimax polynomial f (c1 + f (c2 + f (c3 + f (c4 + f c5)))) (|error| < 1.5e-5
// on [0, 1]); the -1 is folded into the last Horner step. Valid for normal u > 0.
__device__ __forceinline__ float log2s(float u) {
  const float c1 = 0x1.7124acp+0f, c2 = -0x1.6b5948p-1f, c3 = 0x1.aba0f0p-2f, c4 = -0x1.91fd90p-3f,
              c5 = 0x1.7c0becp-5f;
  float m = __builtin_amdgcn_frexp_mantf(u);
  int e = __builtin_amdgcn_frexp_expf(u);
  float f = __builtin_fmaf(m, 2.0f, -1.0f);
  float t = c5;
  t = __builtin_fmaf(t, f, c4);
  t = __builtin_fmaf(t, f, c3);
  t = __builtin_fmaf(t, f, c2);
  t = __builtin_fmaf(t, f, c1);
  t = __builtin_fmaf(t, f, -1.0f);
  return (float)e + t;
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
  const int nchunks = n_tiles * R::kChunks;
  if (n_tiles == NT) {
#pragma unroll
    for (int i = 0; i < R::kChunks; ++i) r.c[i] = s[threadIdx.x + i * NT];
  } else {
#pragma unroll
    for (int i = 0; i < R::kChunks; ++i) {
      const int c = threadIdx.x + i * NT;
      r.c[i] = c < nchunks ? s[c] : make_uint4(0u, 0u, 0u, 0u);
    }
  }
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
#pragma unroll
  for (int i = 0; i < R::kChunks; ++i) {
    if (n_tiles == NT || (int)threadIdx.x + i * NT < nchunks)
      d[i * NT] = *reinterpret_cast<const uint4*>(base + i * (NT / R::kChunks) * R::kStride);
  }
}

}  // namespace tah
