// Decode kernels of the TAH-Quant codec for gfx950 (Algorithm 1, the receiver's step: the
// receiving stage dequantizes). A workgroup is one wavefront and takes one
// group of 64 consecutive tiles. k_decode (tiles of up to 64 channels) gives
// each lane a tile; k_decode4 (128 channels, below) rebuilds the tiles by
// quads of lanes.
//  - the payload header is checked once against the expected one (shape,
//    params, section offsets); on a mismatch the status word is set and
//    nothing is written;
//  - a group's code region (contiguous in the payload, located by the block
//    table and the width map) arrives by 16-byte coalesced loads; k_decode
//    also keeps a software pipeline for a grid smaller than the number of
//    groups (metadata two groups ahead, the region one group ahead), idle
//    under the launch below, which gives every group a workgroup;
//  - processing: the region goes to LDS, each lane reads its code block,
//    unpacks and dequantizes (fmaf(q, s, lo)); flagged tiles get H^T / G and
//    the swap undone (§3.3) by 16-lane groups through fp32 LDS slots (which
//    reuse the region's buffer once every code is read); rows are written to
//    LDS and leave it with 16-byte coalesced stores at the top of the next
//    iteration.
#include <type_traits>

#include "tah_device.hpp"
#include "tah_internal.hpp"

namespace tah {

struct DecArgs {
  const uint8_t* payload;
  uint8_t* y;
  int32_t* status;
  int64_t tiles, len;
  int64_t off_table, off_bitmap, off_side, off_scale, off_zero, off_codes;
  int32_t b_lo, b_hi, sz_lo, sz_hi;
  uint32_t cands;  // candidate widths, one byte each (any-width layout)
  Header expect;
};

// The G codes of width B at src (LDS, 4-byte aligned; 8-byte aligned for
// G >= 64), dequantized: v_k = fmaf(q_k, s, lo).
template <int G, int B>
__device__ __forceinline__ void load_dequant(const uint8_t* src, float s, float lo, float (&v)[G]) {
  constexpr int W = G * B / 32;
  uint32_t w[W];
  if constexpr (G >= 64) {
#pragma unroll
    for (int i = 0; i < W / 2; ++i) {
      const uint2 q = reinterpret_cast<const uint2*>(src)[i];
      w[2 * i] = q.x;
      w[2 * i + 1] = q.y;
    }
  } else {
#pragma unroll
    for (int i = 0; i < W; ++i) w[i] = reinterpret_cast<const uint32_t*>(src)[i];
  }
#pragma unroll
  for (int k = 0; k < G; ++k) v[k] = __builtin_fmaf((float)unpack_code<G, B>(w, k), s, lo);
}

template <int G>
__device__ __forceinline__ void load_dequant_b(int b, const uint8_t* src, float s, float lo, float (&v)[G]) {
  switch (b) {
    case 1: load_dequant<G, 1>(src, s, lo, v); break;
    case 2: load_dequant<G, 2>(src, s, lo, v); break;
    case 3: load_dequant<G, 3>(src, s, lo, v); break;
    case 4: load_dequant<G, 4>(src, s, lo, v); break;
    case 5: load_dequant<G, 5>(src, s, lo, v); break;
    case 6: load_dequant<G, 6>(src, s, lo, v); break;
    case 7: load_dequant<G, 7>(src, s, lo, v); break;
    default: load_dequant<G, 8>(src, s, lo, v); break;
  }
}

// A group's metadata: per lane (side byte, bf16 scale, zero-point) and per
// group (block-table entry, the two words of the 1-bit width map); with the
// 2-bit level map, bm0 is instead the word that holds the lane's own level.
struct DecMeta {
  uint32_t side, scale, tab, bm0, bm1;
  float zero;
};

// Code width of a lane's tile under the 2-bit level map (a level past the
// candidates, only in a corrupt payload, reads as c_1 so every access stays
// inside the region buffer).
__device__ __forceinline__ int level_width(const DecArgs& a, const DecMeta& m, int lane) {
  const uint32_t lv = (m.bm0 >> (2 * (lane & 15))) & 3u;
  const int w = (int)((a.cands >> (8 * lv)) & 255u);
  return w != 0 ? w : a.b_lo;
}

template <int NT, bool MULTI>
__device__ __forceinline__ void load_meta(const DecArgs& a, int64_t g, DecMeta& m) {
  const int64_t t0 = g * NT;
  const int64_t t = t0 + threadIdx.x;
  const int64_t tc = t < a.tiles ? t : a.tiles - 1;  // inactive lanes read a valid tile
  m.side = a.payload[a.off_side + tc];
  m.scale = reinterpret_cast<const uint16_t*>(a.payload + a.off_scale)[tc];
  m.zero = reinterpret_cast<const float*>(a.payload + a.off_zero)[tc];
  const int64_t blk = t0 >> 6;
  const uint32_t* map = reinterpret_cast<const uint32_t*>(a.payload + a.off_bitmap);
  m.tab = reinterpret_cast<const uint32_t*>(a.payload + a.off_table)[blk];
  if constexpr (MULTI) {
    m.bm0 = map[4 * blk + (threadIdx.x >> 4)];  // 16 tiles per word
    m.bm1 = 0u;
  } else {
    m.bm0 = map[2 * blk];
    m.bm1 = map[2 * blk + 1];
  }
}

// The code region of a group: first byte and length (the group's blocks are
// contiguous: b_lo blocks and b_hi blocks in tile order, or blocks of any
// candidate width located by the width-sum table, G/8 bytes per unit).
template <int NT, bool MULTI>
__device__ __forceinline__ void region_of(const DecArgs& a, int64_t g, const DecMeta& m, int64_t& rs, int& rlen) {
  const int64_t t0 = g * NT;
  const int n = (int)((a.tiles - t0) < NT ? (a.tiles - t0) : NT);
  if constexpr (MULTI) {
    const int lane = threadIdx.x;
    int w = lane < n ? level_width(a, m, lane) : 0;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) w += __shfl_xor(w, off, 64);
    const int unit = a.sz_lo / a.b_lo;  // G/8
    rs = a.off_codes + (int64_t)unit * (int64_t)m.tab;
    rlen = unit * w;
  } else {
    const uint64_t bm = ((uint64_t)m.bm1 << 32) | m.bm0;
    const uint64_t valid = n >= 64 ? ~0ull : ((1ull << n) - 1ull);
    rs = a.off_codes + t0 * a.sz_lo + (int64_t)m.tab * (a.sz_hi - a.sz_lo);
    rlen = n * a.sz_lo + __popcll(bm & valid) * (a.sz_hi - a.sz_lo);
  }
}

// Region bytes of a group go through registers in 16-byte chunks: the region
// holds at most NT * G * MAXB / 8 bytes (codes of at most MAXB bits), plus one
// chunk of misalignment. (A native 4 x u32 vector, not the uint4 struct:
// struct copies become memcpy and keep the array in scratch memory.)
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int G, int NT, int MAXB>
struct RegionRegs {
  static constexpr int kChunks = (NT * G * MAXB / 8 + 16 + 16 * NT - 1) / (16 * NT);
  u32x4 c[kChunks];
};

template <int G, int NT, int MAXB>
__device__ __forceinline__ void load_region(const DecArgs& a, int64_t rs, int rlen, RegionRegs<G, NT, MAXB>& r) {
  const int64_t base = rs & ~(int64_t)15;
  const int nchunks = (int)((rs - base + rlen + 15) >> 4);
  const int64_t last = (a.len >> 4) - 1;  // the payload's last whole chunk (bounds on a corrupt table)
#pragma unroll
  for (int i = 0; i < RegionRegs<G, NT, MAXB>::kChunks; ++i) {
    const int c = (int)threadIdx.x + i * NT;
    int64_t q = (base >> 4) + (c < nchunks ? c : 0);
    q = q < last ? q : last;
    q = q > 0 ? q : 0;
    r.c[i] = reinterpret_cast<const u32x4*>(a.payload)[q];
  }
}

// MAXB: the widest code the payload can hold (4 or 8 bits), which sizes the
// code region in LDS and in registers; fewer LDS bytes per workgroup let more
// workgroups share a compute unit. MULTI: the 2-bit level map of the greedy
// allocator instead of the 1-bit width map.
template <int G, typename TOut, int MAXB, bool MULTI>
__global__ __launch_bounds__(64) void k_decode(DecArgs a) {
  constexpr int NT = 64;
  constexpr int V = G / 16;     // elements per lane in a 16-lane transform group
  constexpr int kCoop = 8;      // flagged tiles per round
  constexpr int kSlot = G + 4;  // fp32 slot stride
  using RO = TileRow<G, TOut>;
  using RR = RegionRegs<G, NT, MAXB>;
  __shared__ __attribute__((aligned(16))) uint8_t ys[NT * RO::kStride];
  // The code region, and once every lane has unpacked its codes, the fp32
  // slots of the flagged tiles' transforms (the region is not read again
  // before the next group is written there).
  __shared__ __attribute__((aligned(16))) u32x4 region[NT * RR::kChunks];
  static_assert(sizeof(region) >= sizeof(float) * kCoop * kSlot, "the slots fit in the region buffer");
  float* ts = reinterpret_cast<float*>(region);
  __shared__ uint32_t flist[NT];

  const int lane = threadIdx.x;
  const int q4 = lane >> 4, r16 = lane & 15;

  {  // header
    bool mism = false;
    if (lane < 32) {
      uint32_t got = reinterpret_cast<const uint32_t*>(a.payload)[lane];
      uint32_t want = a.expect.w[lane];
      if (lane == 1) {  // byte 6 records the encoder's input dtype: 0 or 1
        mism = ((got >> 16) & 0xffu) > 1u;
        got &= 0xff00ffffu;
        want &= 0xff00ffffu;
      }
      mism = mism || got != want;
    }
    const bool bad = ballot(mism) != 0;
    if (blockIdx.x == 0 && lane == 0) *a.status = bad ? (int32_t)TAH_ERR_BAD_PAYLOAD : (int32_t)TAH_OK;
    if (bad) return;
  }

  const int64_t ngroups = (a.tiles + NT - 1) / NT;
  const int64_t step = gridDim.x;
  int64_t g = blockIdx.x;
  if (g >= ngroups) return;

  DecMeta mc, mn;  // metadata of the next group (its region is loading) and of the one after
  RR rr;
  int64_t rs_c;
  int rlen_c;
  load_meta<NT, MULTI>(a, g, mc);
  region_of<NT, MULTI>(a, g, mc, rs_c, rlen_c);
  load_region<G, NT>(a, rs_c, rlen_c, rr);
  if (g + step < ngroups) load_meta<NT, MULTI>(a, g + step, mn);

  int64_t prev_t0 = -1;
  int prev_n = 0;
  for (; g < ngroups; g += step) {
    const int64_t t0 = g * NT;
    const int n = (int)((a.tiles - t0) < NT ? (a.tiles - t0) : NT);
    if (prev_t0 >= 0) stage_out<G, TOut, NT>(ys, a.y + prev_t0 * RO::kBytes, prev_n);
#pragma unroll
    for (int i = 0; i < RR::kChunks; ++i) region[lane + i * NT] = rr.c[i];
    const DecMeta m = mc;
    const int64_t rs = rs_c;
    // the next group's region, and the metadata two groups ahead
    if (g + step < ngroups) {
      mc = mn;
      region_of<NT, MULTI>(a, g + step, mc, rs_c, rlen_c);
      load_region<G, NT>(a, rs_c, rlen_c, rr);
      if (g + 2 * step < ngroups) load_meta<NT, MULTI>(a, g + 2 * step, mn);
    } else {
#pragma unroll
      for (int i = 0; i < RR::kChunks; ++i) rr.c[i] = u32x4{0u, 0u, 0u, 0u};  // last group: the old contents are dead
    }
    __syncthreads();

    // ---------------- dequantize: lane owns tile t0 + lane ----------------
    const bool act = lane < n;
    const uint64_t bm = ((uint64_t)m.bm1 << 32) | m.bm0;
    const int hi = act ? (int)((bm >> lane) & 1u) : 0;
    const int flag = act ? (int)(m.side >> 7) : 0;
    const int piv = (int)(m.side & (G - 1));  // a corrupt pivot must not index outside the tile
    int b, sz, lane_off;
    if constexpr (MULTI) {
      const int unit = a.sz_lo / a.b_lo;  // G/8
      b = act ? level_width(a, m, lane) : 0;
      int incl = b;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int o = __shfl_up(incl, off, 64);
        if (lane >= off) incl += o;
      }
      sz = unit * b;
      lane_off = unit * (incl - b);
    } else {
      b = hi ? a.b_hi : a.b_lo;
      sz = hi ? a.sz_hi : a.sz_lo;
      lane_off = lane * a.sz_lo + (int)lanes_below(bm) * (a.sz_hi - a.sz_lo);
    }
    float v[G];
    if (act) {
      int off = (int)(rs & 15) + lane_off;
      const int cap = RR::kChunks * NT * 16 - sz;
      off = off < cap ? off : 0;  // stays inside the region buffer on a corrupt table
      const float s = __uint_as_float(m.scale << 16);
      load_dequant_b<G>(b, reinterpret_cast<const uint8_t*>(region) + off, s, m.zero, v);
    }
    const uint64_t fmask = ballot(act && flag);
    const int nf = (int)__popcll(fmask);
    const int slot = (int)lanes_below(fmask);
    if (act && !flag) lds_write_tile<G, TOut>(ys + lane * RO::kStride, v);
    if (nf != 0) {
      __syncthreads();  // every code read from the region before a slot overwrites it
      if (act && flag) flist[slot] = (uint32_t)lane | ((uint32_t)piv << 8);
      // rounds of kCoop flagged tiles: owners fill the slots, 16-lane groups
      // apply H^T / G and undo the swap into the tile's row
      for (int j_lo = 0; j_lo < nf; j_lo += kCoop) {
        const int j_hi = nf < j_lo + kCoop ? nf : j_lo + kCoop;
        if (act && flag && slot >= j_lo && slot < j_hi)
          lds_write_tile<G, float>(reinterpret_cast<uint8_t*>(ts + (slot - j_lo) * kSlot), v);
        __syncthreads();
        for (int j0 = j_lo; j0 < j_hi; j0 += 4) {
          const int j = j0 + q4;
          if (j < j_hi) {
            const uint32_t e = flist[j];
            uint8_t* row = ys + (e & 255u) * RO::kStride;
            float y[V];
            lds_read_part<V, float>(reinterpret_cast<const uint8_t*>(ts + (j - j_lo) * kSlot), r16, y);
            fwht16<V>(y, r16);
#pragma unroll
            for (int i = 0; i < V; ++i) y[i] = y[i] * (1.0f / G);
            lds_write_part<V, TOut>(row, r16, y);
            if (r16 == 0) {  // element d takes y_0, element 0 takes y_d
              const int d = (int)(e >> 8);
              const uint32_t yd = lds_elem_bits<TOut>(row, d);
              lds_elem_set<TOut>(row, d, f32_to_elem_bits<TOut>(y[0]));
              lds_elem_set<TOut>(row, 0, yd);
            }
          }
        }
        __syncthreads();
      }
    }
    prev_t0 = t0;
    prev_n = n;
    __syncthreads();  // rows and region are read by other lanes next
  }
  if (prev_t0 >= 0) stage_out<G, TOut, NT>(ys, a.y + prev_t0 * RO::kBytes, prev_n);
}

// The unnormalized Sylvester transform of a tile spread over an aligned
// quad of lanes, lane r holding elements [r V, r V + V): the stages h < V
// inside the lane, then h = V (partner lane r xor 1) and h = 2V (r xor 2).
// Every butterfly is the single-rounded a + b / a - b of fwht<G> in the same
// stage order (the upper lane forms partner - own with one fma), so the
// result is that of fwht<4 V>.
template <int V>
__device__ __forceinline__ void fwht_quad(float (&y)[V], int r) {
#pragma unroll
  for (int h = 1; h < V; h <<= 1)
#pragma unroll
    for (int j = 0; j < V; ++j)
      if ((j & h) == 0) {
        const float a = y[j], b = y[j + h];
        y[j] = a + b;
        y[j + h] = a - b;
      }
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
}

// Tiles of 128 channels: the same group, region and metadata as k_decode, but
// each tile is rebuilt by a quad of lanes, sixteen tiles per pass: lane r of
// a quad takes elements 32 r ... 32 r + 31 (its codes are the 4-byte-aligned
// words r b ... r b + b - 1 of the code block, unpacked as a 32-element
// block), dequantizes them, a flagged tile applies H^T / G with fwht_quad and
// the quad undoes the pivot swap with two shuffles; the pass's sixteen rows
// then leave through LDS with 16-byte coalesced stores. A lane holds 32
// values instead of a whole tile: about 80 VGPRs and 15-19 KB of LDS per
// workgroup instead of all 512 registers and 39-43 KB.
template <int G, typename TOut, int MAXB, bool MULTI>
__global__ __launch_bounds__(64) void k_decode4(DecArgs a) {
  constexpr int NT = 64;
  constexpr int V = G / 4;  // elements per lane of a quad
  constexpr int TP = NT / 4;  // tiles per pass
  constexpr int RB = G * Elem<TOut>::kBytes;  // output row bytes
  using RR = RegionRegs<G, NT, MAXB>;
  __shared__ __attribute__((aligned(16))) u32x4 region[NT * RR::kChunks];
  __shared__ __attribute__((aligned(16))) uint8_t ys[TP * RB];
  __shared__ uint32_t m_off[NT], m_bfp[NT];
  __shared__ float m_s[NT], m_lo[NT];

  const int lane = threadIdx.x;
  const int64_t ngroups = (a.tiles + NT - 1) / NT;
  const int64_t g = blockIdx.x;
  // the group's metadata first: its loads are in flight during the header check
  DecMeta m;
  if (g < ngroups) load_meta<NT, MULTI>(a, g, m);
  {  // header
    bool mism = false;
    if (lane < 32) {
      uint32_t got = reinterpret_cast<const uint32_t*>(a.payload)[lane];
      uint32_t want = a.expect.w[lane];
      if (lane == 1) {  // byte 6 records the encoder's input dtype: 0 or 1
        mism = ((got >> 16) & 0xffu) > 1u;
        got &= 0xff00ffffu;
        want &= 0xff00ffffu;
      }
      mism = mism || got != want;
    }
    const bool bad = ballot(mism) != 0;
    if (blockIdx.x == 0 && lane == 0) *a.status = bad ? (int32_t)TAH_ERR_BAD_PAYLOAD : (int32_t)TAH_OK;
    if (bad) return;
  }
  if (g >= ngroups) return;
  const int64_t t0 = g * NT;
  const int n = (int)((a.tiles - t0) < NT ? (a.tiles - t0) : NT);
  int64_t rs;
  int rlen;
  region_of<NT, MULTI>(a, g, m, rs, rlen);
  {
    RR rr;
    load_region<G, NT>(a, rs, rlen, rr);
#pragma unroll
    for (int i = 0; i < RR::kChunks; ++i) region[lane + i * NT] = rr.c[i];
  }

  // ---------------- per tile (lane owns tile t0 + lane): width, offset ----------------
  {
    const bool act = lane < n;
    const uint64_t bm = ((uint64_t)m.bm1 << 32) | m.bm0;
    const int hi = act ? (int)((bm >> lane) & 1u) : 0;
    const int flag = act ? (int)(m.side >> 7) : 0;
    const int piv = (int)(m.side & (G - 1));  // a corrupt pivot must not index outside the tile
    int b, sz, lane_off;
    if constexpr (MULTI) {
      const int unit = a.sz_lo / a.b_lo;  // G/8
      b = act ? level_width(a, m, lane) : 0;
      int incl = b;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int o = __shfl_up(incl, off, 64);
        if (lane >= off) incl += o;
      }
      sz = unit * b;
      lane_off = unit * (incl - b);
    } else {
      b = hi ? a.b_hi : a.b_lo;
      sz = hi ? a.sz_hi : a.sz_lo;
      lane_off = lane * a.sz_lo + (int)lanes_below(bm) * (a.sz_hi - a.sz_lo);
    }
    int off = (int)(rs & 15) + lane_off;
    const int cap = RR::kChunks * NT * 16 - sz;
    off = off < cap ? off : 0;  // stays inside the region buffer on a corrupt table
    m_off[lane] = (uint32_t)off;
    m_bfp[lane] = (uint32_t)b | ((uint32_t)flag << 8) | ((uint32_t)piv << 16);
    m_s[lane] = __uint_as_float(m.scale << 16);
    m_lo[lane] = m.zero;
  }
  __syncthreads();

  // ---------------- quads, sixteen tiles per pass ----------------
  const int q = lane >> 2, r = lane & 3, qb = lane & ~3;
  for (int j0 = 0; j0 < n; j0 += TP) {
    const int j = j0 + q;
    if (j < n) {  // a whole quad takes a tile or none
      const uint32_t e = m_bfp[j];
      const int b = (int)(e & 255u), flag = (int)((e >> 8) & 1u), piv = (int)(e >> 16);
      float y[V];
      // block offsets are multiples of G/8 = 16 bytes, so this lane's V b
      // bits start on a 4-byte boundary
      load_dequant_b<V>(b, reinterpret_cast<const uint8_t*>(region) + m_off[j] + r * (V * b / 8), m_s[j],
                        m_lo[j], y);
      if (flag) {  // the same for the quad's four lanes
        fwht_quad<V>(y, r);
#pragma unroll
        for (int i = 0; i < V; ++i) y[i] = y[i] * (1.0f / G);
        // element d takes y_0, element 0 takes y_d
        const int dl = piv / V, ds = piv % V;
        float mine = y[0];
#pragma unroll
        for (int i = 1; i < V; ++i) mine = ds == i ? y[i] : mine;
        const float y0 = __shfl(y[0], qb, 64);
        const float yd = __shfl(mine, qb + dl, 64);
        if (r == 0) y[0] = yd;
        if (r == dl) {
#pragma unroll
          for (int i = 0; i < V; ++i) y[i] = ds == i ? y0 : y[i];
        }
      }
      lds_write_part<V, TOut>(ys + q * RB, r, y);
    }
    __syncthreads();
    // the pass's rows out: 16-byte chunks, consecutive lanes on consecutive chunks
    const int nrow = n - j0 < TP ? n - j0 : TP;
    const int nch = nrow * (RB / 16);
    uint4* dst = reinterpret_cast<uint4*>(a.y + (t0 + j0) * (int64_t)RB);
#pragma unroll
    for (int i = 0; i < TP * RB / 16 / NT; ++i) {
      const int c = lane + i * NT;
      if (c < nch) store_stream(dst + c, reinterpret_cast<const uint4*>(ys)[c]);
    }
    __syncthreads();  // the rows are rewritten by the next pass
  }
}

// One workgroup per group (8192 x 8192 bf16 decode 29.9 -> 27.2 us, the
// 80/20 one 31.8 -> 30.2 us against a persistent grid of the resident
// workgroups, one box, interleaved). Tiles of 128 channels take k_decode4.
template <int G, typename TOut, int MAXB, bool MULTI>
static hipError_t launch_dec_b(const DecArgs& a, hipStream_t st) {
  const int64_t nwg = a.tiles > 0 ? (a.tiles + 63) / 64 : 1;
  if constexpr (G > 64)
    hipLaunchKernelGGL((k_decode4<G, TOut, MAXB, MULTI>), dim3((unsigned)nwg), dim3(64), 0, st, a);
  else
    hipLaunchKernelGGL((k_decode<G, TOut, MAXB, MULTI>), dim3((unsigned)nwg), dim3(64), 0, st, a);
  return hipGetLastError();
}

template <int G, typename TOut>
static hipError_t launch_dec_t(const DecArgs& a, bool multi, hipStream_t st) {
  if (multi) return a.b_hi <= 4 ? launch_dec_b<G, TOut, 4, true>(a, st) : launch_dec_b<G, TOut, 8, true>(a, st);
  return a.b_hi <= 4 ? launch_dec_b<G, TOut, 4, false>(a, st) : launch_dec_b<G, TOut, 8, false>(a, st);
}

hipError_t launch_decode(const Plan& pl, const void* payload, void* y, int y_dtype, void* ws, hipStream_t st) {
  DecArgs a;
  a.payload = static_cast<const uint8_t*>(payload);
  a.y = static_cast<uint8_t*>(y);
  a.status = reinterpret_cast<int32_t*>(static_cast<uint8_t*>(ws) + pl.ws_status);
  a.tiles = pl.tiles;
  a.len = pl.total;
  a.off_table = pl.off_table;
  a.off_bitmap = pl.off_bitmap;
  a.off_side = pl.off_side;
  a.off_scale = pl.off_scale;
  a.off_zero = pl.off_zero;
  a.off_codes = pl.off_codes;
  a.b_lo = pl.b_lo;
  a.b_hi = pl.b_hi;
  a.sz_lo = pl.G * pl.b_lo / 8;
  a.sz_hi = pl.G * pl.b_hi / 8;
  a.cands = 0;
  for (int i = 0; i < pl.n_candidates; ++i) a.cands |= (uint32_t)pl.candidates[i] << (8 * i);
  make_header(pl, &a.expect);
  const bool f32 = y_dtype == TAH_DTYPE_F32, multi = pl.mode == 2;
  switch (pl.G) {
    case 32: return f32 ? launch_dec_t<32, float>(a, multi, st) : launch_dec_t<32, bf16_t>(a, multi, st);
    case 64: return f32 ? launch_dec_t<64, float>(a, multi, st) : launch_dec_t<64, bf16_t>(a, multi, st);
    case 128: return f32 ? launch_dec_t<128, float>(a, multi, st) : launch_dec_t<128, bf16_t>(a, multi, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace tah
