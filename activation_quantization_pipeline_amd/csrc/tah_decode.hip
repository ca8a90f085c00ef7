// Decode kernel of the TAH-Quant codec for gfx950 (Algorithm 1, line 5: the
// receiving stage dequantizes). One workgroup rebuilds NT consecutive tiles:
//  - the payload header is checked against the expected one (shape, params,
//    section offsets); on a mismatch the status word is set and nothing is written;
//  - phase A, lane i: side byte (flag, pivot), width bit, scale, zero-point and
//    the code-block offset of tile i (block table + popcount of the width map);
//  - tiles are regrouped by (flag, width) so that whole wavefronts take the
//    same branch;
//  - phase B: each lane loads its code block, unpacks, dequantizes
//    (fmaf(q, s, lo)), applies H^T / G and undoes the pivot swap on flagged
//    tiles (§3.3), and writes the tile to LDS;
//  - the tiles leave LDS with 16-byte coalesced stores.
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
  Header expect;
};

template <int G, typename TOut>
constexpr int dec_tiles_per_wg() {
  return TileRow<G, TOut>::kBytes <= 128 ? 256 : (TileRow<G, TOut>::kBytes <= 256 ? 128 : 64);
}

template <int G, int B>
__device__ __forceinline__ void load_dequant(const uint8_t* src, float s, float lo, float (&v)[G]) {
  constexpr int W = G * B / 32;
  uint32_t w[W];
  if constexpr (G >= 128) {
#pragma unroll
    for (int i = 0; i < W / 4; ++i) {
      const uint4 q = reinterpret_cast<const uint4*>(src)[i];
      w[4 * i] = q.x;
      w[4 * i + 1] = q.y;
      w[4 * i + 2] = q.z;
      w[4 * i + 3] = q.w;
    }
  } else if constexpr (G >= 64) {
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

template <int G, typename TOut>
__global__ __launch_bounds__((dec_tiles_per_wg<G, TOut>())) void k_decode(DecArgs a) {
  constexpr int NT = dec_tiles_per_wg<G, TOut>();
  constexpr int NW = NT / 64;
  using RO = TileRow<G, TOut>;
  __shared__ __attribute__((aligned(16))) uint8_t ys[NT * RO::kStride];
  __shared__ uint32_t meta_off[NT];
  __shared__ uint32_t meta_scale[NT];
  __shared__ float meta_lo[NT];
  __shared__ uint8_t meta_side[NT];
  __shared__ uint8_t meta_hi[NT];
  __shared__ uint16_t perm[NT];
  __shared__ int cnt[NW][4];
  __shared__ int bad;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid < 64) {
    bool mism = false;
    if (tid < 32) {
      uint32_t got = reinterpret_cast<const uint32_t*>(a.payload)[tid];
      uint32_t want = a.expect.w[tid];
      if (tid == 1) {  // byte 6 records the encoder's input dtype: 0 or 1
        mism = ((got >> 16) & 0xffu) > 1u;
        got &= 0xff00ffffu;
        want &= 0xff00ffffu;
      }
      mism = mism || got != want;
    }
    const uint64_t m = ballot(mism);
    if (tid == 0) bad = m != 0;
  }
  __syncthreads();
  if (blockIdx.x == 0 && tid == 0) *a.status = bad ? (int32_t)TAH_ERR_BAD_PAYLOAD : (int32_t)TAH_OK;
  if (bad) return;

  const int64_t t0 = (int64_t)blockIdx.x * NT;
  const int n = (int)((a.tiles - t0) < NT ? (a.tiles - t0) : NT);
  if (n <= 0) return;
  const bool act = tid < n;
  const int64_t t = t0 + tid;
  const uint32_t* table = reinterpret_cast<const uint32_t*>(a.payload + a.off_table);
  const uint32_t* bitmap = reinterpret_cast<const uint32_t*>(a.payload + a.off_bitmap);

  // ---------------- phase A ----------------
  int flag = 0, hi = 0;
  uint32_t side = 0;
  if (act) {
    side = a.payload[a.off_side + t];
    flag = side >> 7;
    hi = (bitmap[t >> 5] >> (t & 31)) & 1u;
    meta_scale[tid] = reinterpret_cast<const uint16_t*>(a.payload + a.off_scale)[t];
    meta_lo[tid] = reinterpret_cast<const float*>(a.payload + a.off_zero)[t];
  }
  const uint64_t hmask = ballot(act && hi);
  const int64_t blk_wave = (t0 >> 6) + wave;
  const uint32_t hb_wg = table[t0 >> 6];
  const uint32_t hb = (act ? table[blk_wave] : hb_wg) + lanes_below(hmask);
  const int64_t wg_off = t0 * a.sz_lo + (int64_t)hb_wg * (a.sz_hi - a.sz_lo);
  meta_off[tid] = (uint32_t)tid * (uint32_t)a.sz_lo + (hb - hb_wg) * (uint32_t)(a.sz_hi - a.sz_lo);
  meta_side[tid] = (uint8_t)side;
  meta_hi[tid] = (uint8_t)hi;

  // plain tiles first, transformed tiles as one run rotated to wave (block mod NW)
  // so that the Hadamard work spreads over the CU's SIMDs
  const int cls = act ? ((flag << 1) | hi) : 4;
  const uint64_t b0 = ballot(cls == 0), b1 = ballot(cls == 1), b2 = ballot(cls == 2), b3 = ballot(cls == 3);
  if (lane == 0) {
    cnt[wave][0] = __popcll(b0);
    cnt[wave][1] = __popcll(b1);
    cnt[wave][2] = __popcll(b2);
    cnt[wave][3] = __popcll(b3);
  }
  __syncthreads();
  if (act) {
    int dst = 0;
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int w = 0; w < NW; ++w) dst += (c < cls || (c == cls && w < wave)) ? cnt[w][c] : 0;
    const uint64_t mine = cls == 0 ? b0 : cls == 1 ? b1 : cls == 2 ? b2 : b3;
    dst += (int)lanes_below(mine);
    int plain = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) plain += cnt[w][0] + cnt[w][1];
    const int start = (int)(blockIdx.x % NW) * 64;
    dst = (dst + n + start - plain) % n;
    perm[dst] = (uint16_t)tid;
  }
  __syncthreads();

  // ---------------- phase B ----------------
  if (act) {
    const int j = perm[tid];
    const uint32_t sj = meta_side[j];
    const int fj = sj >> 7;
    const int d = sj & (G - 1);  // a corrupt pivot must not index outside the tile
    const int b = meta_hi[j] ? a.b_hi : a.b_lo;
    const int sz = meta_hi[j] ? a.sz_hi : a.sz_lo;
    int64_t off = a.off_codes + wg_off + meta_off[j];
    if (off + sz > a.len) off = a.off_codes;  // stays in bounds on a corrupt table
    const float s = __uint_as_float(meta_scale[j] << 16);
    const float lo = meta_lo[j];
    float v[G];
    load_dequant_b<G>(b, a.payload + off, s, lo, v);
    if (fj) {
      fwht<G>(v);
#pragma unroll
      for (int k = 0; k < G; ++k) v[k] = v[k] * (1.0f / G);
    }
    uint8_t* row = ys + j * RO::kStride;
    lds_write_tile<G, TOut>(row, v);
    if (fj) {
      const uint32_t yd = lds_elem_bits<TOut>(row, d);
      lds_elem_set<TOut>(row, d, f32_to_elem_bits<TOut>(v[0]));
      lds_elem_set<TOut>(row, 0, yd);
    }
  }
  __syncthreads();
  stage_out<G, TOut, NT>(ys, a.y + t0 * RO::kBytes, n);
}

template <int G, typename TOut>
static hipError_t launch_dec_t(const DecArgs& a, hipStream_t st) {
  constexpr int NT = dec_tiles_per_wg<G, TOut>();
  const int64_t nwg = a.tiles > 0 ? (a.tiles + NT - 1) / NT : 1;
  hipLaunchKernelGGL((k_decode<G, TOut>), dim3((unsigned)nwg), dim3(NT), 0, st, a);
  return hipGetLastError();
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
  make_header(pl, &a.expect);
  const bool f32 = y_dtype == TAH_DTYPE_F32;
  switch (pl.G) {
    case 32: return f32 ? launch_dec_t<32, float>(a, st) : launch_dec_t<32, bf16_t>(a, st);
    case 64: return f32 ? launch_dec_t<64, float>(a, st) : launch_dec_t<64, bf16_t>(a, st);
    case 128: return f32 ? launch_dec_t<128, float>(a, st) : launch_dec_t<128, bf16_t>(a, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace tah
