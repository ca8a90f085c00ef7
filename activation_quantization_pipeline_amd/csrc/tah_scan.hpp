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

}  // namespace tah
