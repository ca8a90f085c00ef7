// Block-wide scan shared by the select kernels of the library (top-p% and
// greedy): the per-64-tile counts or width sums of one sample, held in LDS,
// into the block table.
#pragma once

#include "tah_device.hpp"

namespace tah {

// Exclusive scan of the counts of LDS array rc (4 nr NT entries, zero past
// the n that matter) by the NT threads of a workgroup: dst[j] = base + the
// counts before j, for j < n, stored coalesced. Thread t owns the 4 nr
// consecutive counts from 4 nr t (nr 16-byte words, nr <= MAXQ); wsum holds
// NT / 64 words of LDS. Returns the base plus all counts, in every thread.
template <int NT, int MAXQ>
__device__ uint32_t lds_scan_store(uint32_t* rc, int nr, uint32_t base, uint32_t* dst, int64_t n, uint32_t* wsum) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint4* seg = reinterpret_cast<uint4*>(rc) + tid * nr;
  uint32_t c[4 * MAXQ];
#pragma unroll
  for (int q = 0; q < MAXQ; ++q) {
    const uint4 w4 = q < nr ? seg[q] : make_uint4(0u, 0u, 0u, 0u);
    c[4 * q] = w4.x;
    c[4 * q + 1] = w4.y;
    c[4 * q + 2] = w4.z;
    c[4 * q + 3] = w4.w;
  }
  uint32_t tot = 0u;
#pragma unroll
  for (int i = 0; i < 4 * MAXQ; ++i) tot += c[i];
  uint32_t incl = tot;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t o = __shfl_up(incl, off, 64);
    if (lane >= off) incl += o;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  uint32_t run = base + incl - tot, all = base;
  for (int w = 0; w < NT / 64; ++w) {
    if (w < wave) run += wsum[w];
    all += wsum[w];
  }
#pragma unroll
  for (int i = 0; i < 4 * MAXQ; ++i) {
    const uint32_t ci = c[i];
    c[i] = run;
    run += ci;
  }
#pragma unroll
  for (int q = 0; q < MAXQ; ++q)
    if (q < nr) seg[q] = make_uint4(c[4 * q], c[4 * q + 1], c[4 * q + 2], c[4 * q + 3]);
  __syncthreads();
  for (int64_t j = tid; j < n; j += NT) dst[j] = rc[j];
  return all;
}

// Sum of v over the wavefront, in every lane (every lane active): DPP and
// swizzle steps inside rows of 16 lanes, then the four rows read out.
__device__ __forceinline__ uint32_t wave_total(uint32_t v) {
  v += __float_as_uint(xor_lane<1>(__uint_as_float(v)));
  v += __float_as_uint(xor_lane<2>(__uint_as_float(v)));
  v += __float_as_uint(xor_lane<4>(__uint_as_float(v)));
  v += __float_as_uint(xor_lane<8>(__uint_as_float(v)));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 0) + (uint32_t)__builtin_amdgcn_readlane((int)v, 16) +
         (uint32_t)__builtin_amdgcn_readlane((int)v, 32) + (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
}

// Rank search by one wavefront (every lane active) in a histogram of NB bins
// (NB a multiple of 256; global or LDS memory, 16-byte aligned) whose total
// is below 2^32: the bin that holds rank r (1-based), the bins taken in
// descending order (desc) or ascending. Gives the bin, its count and the
// count of the bins before it in that order; false when r is 0 or exceeds
// the total. Each 1 KB slice j of the histogram is one coalesced 16-byte load
// per lane: lane l holds the four bins at order positions o = 256 j + 4 l + m
// (m = 0 .. 3), so the order walks the slices, then the lanes, then a lane's
// four bins.
template <int NB>
__device__ __forceinline__ bool find_rank(const uint32_t* h, bool desc, uint32_t r, uint32_t& bin, uint32_t& cnt,
                                          uint32_t& before) {
  constexpr int J = NB / 256;
  const int lane = threadIdx.x & 63;
  uint32_t c[J][4], t[J], T[J];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int o = 256 * j + 4 * lane;
    const uint4 q = *reinterpret_cast<const uint4*>(h + (desc ? NB - 4 - o : o));
    c[j][0] = desc ? q.w : q.x;
    c[j][1] = desc ? q.z : q.y;
    c[j][2] = desc ? q.y : q.z;
    c[j][3] = desc ? q.x : q.w;
    t[j] = c[j][0] + c[j][1] + c[j][2] + c[j][3];
  }
  // the slice holding rank r, and the count before it
#pragma unroll
  for (int j = 0; j < J; ++j) T[j] = wave_total(t[j]);
  uint32_t base = 0;
  int js = -1;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    if (js < 0) {
      if (r <= base + T[j]) js = j;
      else base += T[j];
    }
  }
  if (js < 0) return false;
  uint32_t v = 0, cj[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int j = 0; j < J; ++j)
    if (j == js) {
      v = t[j];
      cj[0] = c[j][0];
      cj[1] = c[j][1];
      cj[2] = c[j][2];
      cj[3] = c[j][3];
    }
  // the lane inside the slice: inclusive scan of the lanes' sums
  uint32_t incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t o = (uint32_t)__shfl_up((int)incl, off, 64);
    if (lane >= off) incl += o;
  }
  const uint32_t rr = r - base, excl = incl - v;
  const uint64_t hm = ballot(excl < rr && rr <= incl);
  if (hm == 0) return false;
  const int src = __ffsll((unsigned long long)hm) - 1;
  // the bin inside that lane
  uint32_t b4 = excl, ci = cj[3];
  int mi = 3;
  bool done = false;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (!done) {
      if (b4 + cj[i] >= rr) {
        mi = i;
        ci = cj[i];
        done = true;
      } else {
        b4 += cj[i];
      }
    }
  }
  const int o = 256 * js + 4 * src + __builtin_amdgcn_readlane(mi, src);
  bin = (uint32_t)(desc ? NB - 1 - o : o);
  cnt = (uint32_t)__builtin_amdgcn_readlane((int)ci, src);
  before = base + (uint32_t)__builtin_amdgcn_readlane((int)b4, src);
  return true;
}

}  // namespace tah
