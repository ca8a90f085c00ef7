// The tile-local Hadamard transform of Eq. (4) (TAH-Quant §3.3), unnormalized,
// as a standalone operation with two implementations, kept to compare them:
//
//  BUTTERFLY  one lane per tile: rows staged through LDS, fwht<G> in registers
//             (G log2 G adds in the stage order the codec and its oracle use),
//             so its results are those of the codec bit for bit;
//  MFMA       the dense product the pages price at O(G^2) per tile (§3.4), on
//             the matrix cores: a wavefront takes 64 tiles (G = 64, bf16) as
//             the 64 x 64 matrix X and forms Y = X H with sixteen
//             v_mfma_f32_32x32x16_bf16 (H is symmetric with entries +-1, exact
//             in bf16; products are exact, sums are fp32). The hardware adds
//             the 64 products in its own order, so its results may differ from
//             the butterfly's in the last bits.
//
// The codec itself uses the butterfly (its codes must match the oracle bit for
// bit); this operation exists to measure the alternative.
#include "tah_device.hpp"
#include "tah_internal.hpp"

namespace tah {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

template <int G, typename TIn>
__global__ __launch_bounds__(64) void k_had_butterfly(const uint8_t* __restrict__ x, uint8_t* __restrict__ y,
                                                      int64_t tiles) {
  constexpr int NT = 64;
  using RI = TileRow<G, TIn>;
  using RO = TileRow<G, float>;
  __shared__ __attribute__((aligned(16))) uint8_t xs[NT * RI::kStride];
  __shared__ __attribute__((aligned(16))) uint8_t ys[NT * RO::kStride];
  const int lane = threadIdx.x;
  const int64_t ngroups = (tiles + NT - 1) / NT;
  for (int64_t g = blockIdx.x; g < ngroups; g += gridDim.x) {
    const int64_t t0 = g * NT;
    const int n = (int)min<int64_t>(NT, tiles - t0);
    stage_in<G, TIn, NT>(x + t0 * RI::kBytes, xs, n);
    __syncthreads();
    if (lane < n) {
      float v[G];
      lds_read_tile<G, TIn>(xs + lane * RI::kStride, v);
      fwht<G>(v);
      lds_write_tile<G, float>(ys + lane * RO::kStride, v);
    }
    __syncthreads();
    stage_out<G, float, NT>(ys, y + t0 * RO::kBytes, n);
    __syncthreads();
  }
}

// G = 64, bf16 tiles. Operand layouts of the 32x32x16 instruction (checked on
// the device): A row i = lane % 32 holds k = 8 (lane / 32) + e, e = 0..7; B
// column j = lane % 32 holds the same k; D register r of a lane is row
// 8 (r / 4) + 4 (lane / 32) + r % 4, column lane % 32.
__global__ __launch_bounds__(64) void k_had_mfma(const uint8_t* __restrict__ x, uint8_t* __restrict__ y,
                                                 int64_t tiles) {
  constexpr int G = 64, NT = 64;
  using RI = TileRow<G, bf16_t>;
  using RO = TileRow<G, float>;
  __shared__ __attribute__((aligned(16))) uint8_t xs[NT * RI::kStride];
  __shared__ __attribute__((aligned(16))) uint8_t ys[NT * RO::kStride];
  const int lane = threadIdx.x;
  const int lr = lane & 31, lh = lane >> 5;

  // H as the B operand: column block cb (32 columns), k step s (16 rows)
  bf16x8_t hb[2][4];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb)
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      uint16_t e8[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int k = 16 * s + 8 * lh + e, j = 32 * cb + lr;
        e8[e] = (__popc((unsigned)(k & j)) & 1) ? 0xBF80u : 0x3F80u;  // -1 / +1
      }
      hb[cb][s] = __builtin_bit_cast(bf16x8_t, e8);
    }

  const int64_t ngroups = (tiles + NT - 1) / NT;
  for (int64_t g = blockIdx.x; g < ngroups; g += gridDim.x) {
    const int64_t t0 = g * NT;
    const int n = (int)min<int64_t>(NT, tiles - t0);
    stage_in<G, bf16_t, NT>(x + t0 * RI::kBytes, xs, n);
    if (n < NT) {  // rows past the end are zero (their outputs are not stored)
      for (int i = lane; i < (NT - n) * (RI::kStride / 16); i += NT)
        reinterpret_cast<uint4*>(xs + n * RI::kStride)[i] = make_uint4(0, 0, 0, 0);
    }
    __syncthreads();
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        f32x16_t acc = {};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(xs + (32 * rb + lr) * RI::kStride + (16 * s + 8 * lh) * 2);
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, hb[cb][s], acc, 0, 0, 0);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int i = 32 * rb + 8 * (r / 4) + 4 * lh + (r % 4);
          reinterpret_cast<float*>(ys + i * RO::kStride)[32 * cb + lr] = acc[r];
        }
      }
    __syncthreads();
    stage_out<G, float, NT>(ys, y + t0 * RO::kBytes, n);
    __syncthreads();
  }
}

// One workgroup per group of 64 tiles for both kernels, as in the codec's
// encoder (against a persistent grid of the resident workgroups, 8192 x 8192
// bf16: butterfly 59.4 -> 57.8 us, matrix cores 59.9 -> 57.8 us, one box).
static int64_t had_grid(int64_t ngroups) { return ngroups; }

template <int G, typename TIn>
static hipError_t launch_butterfly(const void* x, float* y, int64_t tiles, hipStream_t st) {
  const int64_t ngroups = (tiles + 63) / 64;
  const int64_t nwg = had_grid(ngroups);
  hipLaunchKernelGGL((k_had_butterfly<G, TIn>), dim3((unsigned)nwg), dim3(64), 0, st,
                     static_cast<const uint8_t*>(x), reinterpret_cast<uint8_t*>(y), tiles);
  return hipGetLastError();
}

hipError_t launch_hadamard(const void* x, int x_dtype, int64_t tiles, int G, int method, float* y, hipStream_t st) {
  if (tiles == 0) return hipSuccess;
  if (method == 1) {
    const int64_t nwg = had_grid((tiles + 63) / 64);
    hipLaunchKernelGGL(k_had_mfma, dim3((unsigned)nwg), dim3(64), 0, st, static_cast<const uint8_t*>(x),
                       reinterpret_cast<uint8_t*>(y), tiles);
    return hipGetLastError();
  }
  const bool bf = x_dtype == TAH_DTYPE_BF16;
  switch (G) {
    case 32: return bf ? launch_butterfly<32, bf16_t>(x, y, tiles, st) : launch_butterfly<32, float>(x, y, tiles, st);
    case 64: return bf ? launch_butterfly<64, bf16_t>(x, y, tiles, st) : launch_butterfly<64, float>(x, y, tiles, st);
    case 128: return bf ? launch_butterfly<128, bf16_t>(x, y, tiles, st) : launch_butterfly<128, float>(x, y, tiles, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace tah
