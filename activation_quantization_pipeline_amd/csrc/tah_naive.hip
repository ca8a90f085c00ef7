// Backward compressor of TAH-Quant pipeline training for gfx950: the activation
// gradients sent back across the stage boundary (Algorithm 1, the backward pass) go
// through a simple b-bit fixed-point quantizer (§3.5), with the scaling of
// Appendix H, Eq. (24): g_hat = Q(c g) / c.
//   q = clamp(round_half_even(g * c_q), -2^(b-1), 2^(b-1) - 1),  c_q = c 2^(b-1)
//   g_hat = q / c_q
// Payload: a 256-byte header region, then the codes as b-bit two's complement,
// code i at stream bits [i b, i b + b), least significant bit first. One
// thread owns one group of 32 codes, which fills exactly b 32-bit words.
// The kernels are elementwise and bound by HBM: inputs and outputs go through
// padded LDS rows so that global memory is read and written with 16-byte
// coalesced accesses.
#include <math.h>
#include <string.h>

#include "tah_device.hpp"
#include "tah_internal.hpp"

namespace tah {

struct NaiveArgs {
  const uint8_t* in;  // gradients (encode) or payload (decode)
  uint8_t* out;       // payload (encode) or gradients (decode)
  int32_t* status;    // decode: device status word
  int64_t n, ngroups, total;
  int32_t bits;
  float cq;           // c 2^(b-1), exact
  uint32_t hdr[8];    // header bytes 0..31 (the rest of the 256 bytes is zero)
};

constexpr int kNaiveThreads = 256;  // groups per workgroup

// The B words of a packed group to dst (LDS, 4 B-aligned; 16-byte aligned
// when B is a multiple of 4).
template <int B>
__device__ __forceinline__ void pack_store(const uint32_t (&q)[32], uint32_t* dst) {
  uint32_t w[B];
  pack_codes<32, B>(q, w);
  if constexpr (B % 4 == 0) {
#pragma unroll
    for (int i = 0; i < B / 4; ++i)
      reinterpret_cast<uint4*>(dst)[i] = make_uint4(w[4 * i], w[4 * i + 1], w[4 * i + 2], w[4 * i + 3]);
  } else if constexpr (B % 2 == 0) {
#pragma unroll
    for (int i = 0; i < B / 2; ++i) reinterpret_cast<uint2*>(dst)[i] = make_uint2(w[2 * i], w[2 * i + 1]);
  } else {
#pragma unroll
    for (int i = 0; i < B; ++i) dst[i] = w[i];
  }
}

// Code k (two's complement, B bits) of a packed group, sign-extended.
template <int B>
__device__ __forceinline__ int32_t code_signed(const uint32_t (&w)[B], int k) {
  const int bit = k * B;
  const int i = bit >> 5, off = bit & 31;
  if (off + B <= 32) return __builtin_amdgcn_sbfe((int32_t)w[i], (uint32_t)off, (uint32_t)B);
  return __builtin_amdgcn_sbfe((int32_t)__builtin_amdgcn_alignbit(w[i + 1], w[i], (uint32_t)off), 0u, (uint32_t)B);
}

template <int B, typename TOut>
__device__ __forceinline__ void load_dequant_naive(const uint8_t* src, float cq, float (&v)[32]) {
  uint32_t w[B];
  if constexpr (B % 2 == 0) {
#pragma unroll
    for (int i = 0; i < B / 2; ++i) {
      const uint2 q = reinterpret_cast<const uint2*>(src)[i];
      w[2 * i] = q.x;
      w[2 * i + 1] = q.y;
    }
  } else {
#pragma unroll
    for (int i = 0; i < B; ++i) w[i] = reinterpret_cast<const uint32_t*>(src)[i];
  }
#pragma unroll
  for (int k = 0; k < 32; ++k) v[k] = (float)code_signed<B>(w, k) / cq;  // one IEEE division
}

// Copy the elements [e0, e0 + ne) (ne <= 256 * 32) of a row-major element
// stream into 256 padded LDS rows of 32 elements; the last partial 16-byte
// chunk is read element by element (never past the caller's buffer), missing
// elements are zero.
template <typename T, int kStride>
__device__ __forceinline__ void naive_stage_in(const uint8_t* src, int64_t ne, uint8_t* rows) {
  constexpr int EB = Elem<T>::kBytes;
  constexpr int kChunks = 32 * EB / 16;  // chunks per row
  const int64_t bytes = ne * EB;
  const int nchunks = (int)((bytes + 15) >> 4);
  for (int c = threadIdx.x; c < kNaiveThreads * kChunks; c += kNaiveThreads) {
    uint4 q = make_uint4(0u, 0u, 0u, 0u);
    const int64_t off = (int64_t)c * 16;
    if (off + 16 <= bytes) {
      q = load_stream(reinterpret_cast<const uint4*>(src + off));  // streamed once: nontemporal
    } else if (c < nchunks) {
      uint32_t wv[4] = {0u, 0u, 0u, 0u};
      for (int64_t b = off; b < bytes; b += EB) {  // the tail chunk, element by element
        const uint32_t e = EB == 4 ? *reinterpret_cast<const uint32_t*>(src + b)
                                   : (uint32_t)*reinterpret_cast<const uint16_t*>(src + b);
        const int k = (int)(b - off);
        wv[k >> 2] |= e << ((k & 3) * 8);
      }
      q = make_uint4(wv[0], wv[1], wv[2], wv[3]);
    }
    *reinterpret_cast<uint4*>(rows + (c / kChunks) * kStride + (c % kChunks) * 16) = q;
  }
}

template <typename T, int kStride>
__device__ __forceinline__ void naive_stage_out(const uint8_t* rows, uint8_t* dst, int64_t ne) {
  constexpr int EB = Elem<T>::kBytes;
  constexpr int kChunks = 32 * EB / 16;
  const int64_t bytes = ne * EB;
  const int nchunks = (int)((bytes + 15) >> 4);
  for (int c = threadIdx.x; c < nchunks; c += kNaiveThreads) {
    const uint4 q = *reinterpret_cast<const uint4*>(rows + (c / kChunks) * kStride + (c % kChunks) * 16);
    const int64_t off = (int64_t)c * 16;
    if (off + 16 <= bytes) {
      store_stream(reinterpret_cast<uint4*>(dst + off), q);  // streamed once: nontemporal
    } else {
      const uint32_t wv[4] = {q.x, q.y, q.z, q.w};
      for (int64_t b = off; b < bytes; b += EB) {  // the tail chunk, element by element
        const int k = (int)(b - off);
        const uint32_t e = wv[k >> 2] >> ((k & 3) * 8);
        if constexpr (EB == 4) *reinterpret_cast<uint32_t*>(dst + b) = e;
        else *reinterpret_cast<uint16_t*>(dst + b) = (uint16_t)e;
      }
    }
  }
}

template <typename TIn>
__global__ __launch_bounds__(kNaiveThreads) void k_naive_encode(NaiveArgs a) {
  constexpr int kStride = 32 * Elem<TIn>::kBytes + 16;
  __shared__ __attribute__((aligned(16))) uint8_t rows[kNaiveThreads * kStride];
  const int tid = threadIdx.x;
  if (blockIdx.x == 0) {  // header region and the zero pad after the last group
    if (tid < 64) reinterpret_cast<uint32_t*>(a.out)[tid] = tid < 8 ? a.hdr[tid] : 0u;
    for (int64_t i = 256 + a.ngroups * 4 * a.bits + tid; i < a.total; i += kNaiveThreads) a.out[i] = 0;
  }
  const int64_t gbase = (int64_t)blockIdx.x * kNaiveThreads;
  const int64_t e0 = gbase * 32;
  if (e0 >= a.n) return;
  const int64_t ne = a.n - e0 < (int64_t)kNaiveThreads * 32 ? a.n - e0 : (int64_t)kNaiveThreads * 32;
  naive_stage_in<TIn, kStride>(a.in + e0 * Elem<TIn>::kBytes, ne, rows);
  __syncthreads();
  const int64_t g = gbase + tid;
  const bool act = g < a.ngroups;
  float v[32];
  if (act) lds_read_tile<32, TIn>(rows + tid * kStride, v);
  const float lo = -(float)(1 << (a.bits - 1)), hi = (float)((1 << (a.bits - 1)) - 1);
  uint32_t q[32];
#pragma unroll
  for (int k = 0; k < 32; ++k) {
    const float r = __builtin_rintf(v[k] * a.cq);  // round half to even
    q[k] = (uint32_t)(int32_t)__builtin_amdgcn_fmed3f(lo, r, hi);
  }
  __syncthreads();  // every row read: the buffer now takes the packed groups
  // the workgroup's groups are contiguous in the payload: packed into LDS in
  // group order, then stored with 16-byte coalesced writes
  uint32_t* pw = reinterpret_cast<uint32_t*>(rows);
  if (act) {
    uint32_t* dst = pw + tid * a.bits;
    switch (a.bits) {
    case 2: pack_store<2>(q, dst); break;
    case 3: pack_store<3>(q, dst); break;
    case 4: pack_store<4>(q, dst); break;
    case 5: pack_store<5>(q, dst); break;
    case 6: pack_store<6>(q, dst); break;
    case 7: pack_store<7>(q, dst); break;
    case 8: pack_store<8>(q, dst); break;
    case 9: pack_store<9>(q, dst); break;
    case 10: pack_store<10>(q, dst); break;
    case 11: pack_store<11>(q, dst); break;
    case 12: pack_store<12>(q, dst); break;
    case 13: pack_store<13>(q, dst); break;
    case 14: pack_store<14>(q, dst); break;
    case 15: pack_store<15>(q, dst); break;
    default: pack_store<16>(q, dst); break;
    }
  }
  __syncthreads();
  const int64_t ng = a.ngroups - gbase < kNaiveThreads ? a.ngroups - gbase : kNaiveThreads;
  const int nw = (int)ng * a.bits;  // words of this workgroup's groups
  uint32_t* out = reinterpret_cast<uint32_t*>(a.out + 256 + gbase * 4 * a.bits);  // 16-byte aligned
  const int nq = nw >> 2;
  for (int i = tid; i < nq; i += kNaiveThreads) reinterpret_cast<uint4*>(out)[i] = reinterpret_cast<const uint4*>(pw)[i];
  for (int i = 4 * nq + tid; i < nw; i += kNaiveThreads) out[i] = pw[i];
}

template <typename TOut>
__global__ __launch_bounds__(kNaiveThreads) void k_naive_decode(NaiveArgs a) {
  constexpr int kStride = 32 * Elem<TOut>::kBytes + 16;
  __shared__ __attribute__((aligned(16))) uint8_t rows[kNaiveThreads * kStride];
  __shared__ int bad;
  const int tid = threadIdx.x;
  if (tid < 64) {  // header: all but the input-dtype byte and bytes 20..23
    bool mism = false;
    if (tid < 8 && tid != 5) {
      uint32_t got = reinterpret_cast<const uint32_t*>(a.in)[tid];
      uint32_t want = a.hdr[tid];
      if (tid == 1) {
        got &= 0xff00ffffu;
        want &= 0xff00ffffu;
      }
      mism = got != want;
    }
    const uint64_t m = ballot(mism);
    if (tid == 0) bad = m != 0;
  }
  __syncthreads();
  if (blockIdx.x == 0 && tid == 0) *a.status = bad ? (int32_t)TAH_ERR_BAD_PAYLOAD : (int32_t)TAH_OK;
  if (bad) return;
  const int64_t gbase = (int64_t)blockIdx.x * kNaiveThreads;
  const int64_t e0 = gbase * 32;
  if (e0 >= a.n) return;
  const int64_t g = gbase + tid;
  if (g < a.ngroups) {
    const uint8_t* src = a.in + 256 + g * 4 * a.bits;
    float v[32];
    switch (a.bits) {
      case 2: load_dequant_naive<2, TOut>(src, a.cq, v); break;
      case 3: load_dequant_naive<3, TOut>(src, a.cq, v); break;
      case 4: load_dequant_naive<4, TOut>(src, a.cq, v); break;
      case 5: load_dequant_naive<5, TOut>(src, a.cq, v); break;
      case 6: load_dequant_naive<6, TOut>(src, a.cq, v); break;
      case 7: load_dequant_naive<7, TOut>(src, a.cq, v); break;
      case 8: load_dequant_naive<8, TOut>(src, a.cq, v); break;
      case 9: load_dequant_naive<9, TOut>(src, a.cq, v); break;
      case 10: load_dequant_naive<10, TOut>(src, a.cq, v); break;
      case 11: load_dequant_naive<11, TOut>(src, a.cq, v); break;
      case 12: load_dequant_naive<12, TOut>(src, a.cq, v); break;
      case 13: load_dequant_naive<13, TOut>(src, a.cq, v); break;
      case 14: load_dequant_naive<14, TOut>(src, a.cq, v); break;
      case 15: load_dequant_naive<15, TOut>(src, a.cq, v); break;
      default: load_dequant_naive<16, TOut>(src, a.cq, v); break;
    }
    lds_write_tile<32, TOut>(rows + tid * kStride, v);
  }
  __syncthreads();
  const int64_t ne = a.n - e0 < (int64_t)kNaiveThreads * 32 ? a.n - e0 : (int64_t)kNaiveThreads * 32;
  naive_stage_out<TOut, kStride>(rows, a.out + e0 * Elem<TOut>::kBytes, ne);
}

static void naive_args(int64_t n, int bits, float c, int dtype, NaiveArgs* a) {
  a->n = n;
  a->ngroups = (n + 31) / 32;
  const int64_t code_bytes = a->ngroups * 4 * bits;
  a->total = ((256 + code_bytes) + 255) / 256 * 256;
  a->bits = bits;
  a->cq = ldexpf(c, bits - 1);
  uint8_t h[32];
  memset(h, 0, sizeof(h));
  const uint32_t magic = 0x4E484154u;  // "TAHN"
  const uint16_t ver = 1;
  const uint8_t dt = (uint8_t)dtype, b = (uint8_t)bits;
  memcpy(h + 0, &magic, 4);
  memcpy(h + 4, &ver, 2);
  memcpy(h + 6, &dt, 1);
  memcpy(h + 7, &b, 1);
  memcpy(h + 8, &n, 8);
  memcpy(h + 16, &c, 4);
  memcpy(h + 24, &a->total, 8);
  memcpy(a->hdr, h, 32);
}

int64_t naive_payload_bytes(int64_t n, int bits) {
  const int64_t groups = (n + 31) / 32;
  return ((256 + groups * 4 * bits) + 255) / 256 * 256;
}

hipError_t launch_naive_encode(const void* g, int g_dtype, int64_t n, int bits, float c, void* payload,
                               hipStream_t st) {
  NaiveArgs a;
  naive_args(n, bits, c, g_dtype, &a);
  a.in = static_cast<const uint8_t*>(g);
  a.out = static_cast<uint8_t*>(payload);
  a.status = nullptr;
  const int64_t nwg = a.ngroups > 0 ? (a.ngroups + kNaiveThreads - 1) / kNaiveThreads : 1;
  if (g_dtype == TAH_DTYPE_F32)
    hipLaunchKernelGGL(k_naive_encode<float>, dim3((unsigned)nwg), dim3(kNaiveThreads), 0, st, a);
  else
    hipLaunchKernelGGL(k_naive_encode<bf16_t>, dim3((unsigned)nwg), dim3(kNaiveThreads), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_naive_decode(const void* payload, int64_t n, int bits, float c, void* y, int y_dtype, void* ws,
                               hipStream_t st) {
  NaiveArgs a;
  naive_args(n, bits, c, 0, &a);
  a.in = static_cast<const uint8_t*>(payload);
  a.out = static_cast<uint8_t*>(y);
  a.status = static_cast<int32_t*>(ws);
  const int64_t nwg = a.ngroups > 0 ? (a.ngroups + kNaiveThreads - 1) / kNaiveThreads : 1;
  if (y_dtype == TAH_DTYPE_F32)
    hipLaunchKernelGGL(k_naive_decode<float>, dim3((unsigned)nwg), dim3(kNaiveThreads), 0, st, a);
  else
    hipLaunchKernelGGL(k_naive_decode<bf16_t>, dim3((unsigned)nwg), dim3(kNaiveThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace tah
