// Internal declarations of the MI355X TAH-Quant library: the per-call plan
// (shape, width pair, payload and workspace layout) and the kernel launchers.
// Nothing here is part of the C ABI (include/tah.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/tah.h"

namespace tah {

// Histogram digits of the per-sample radix select (see tah_select.hip).
constexpr int kDigitBits = 11;
constexpr int kBins = 1 << kDigitBits;
constexpr int kMaxPasses = 6;
// Candidates for breaking ties at the threshold, listed by the last entropy
// pass: (key, tile index) pairs, at most kCandPerChunk per histogram workgroup
// and kMaxCand per sample.
constexpr int kCandPerChunk = 512;
constexpr int64_t kMaxCand = 4096;
// The largest samples selected by one workgroup with the keys in LDS.
constexpr int64_t kLdsSelect = 4096;
// Two-width layouts whose width map and block table the select's last two
// launches write (no marking or scan launch): at most this many runs of 64
// tiles per sample, whose counts the resolve workgroup scans in LDS.
constexpr int64_t kFoldMaxRuns = 16384;

struct SelectPass {
  int32_t kind;   // 0: entropy key digit, 1: tile-index digit among tied entropies
  int32_t shift;  // lowest bit of the digit
  int32_t width;  // digit width in bits
  int32_t last_h; // 1 on the last entropy pass
};

// One digit of the greedy allocator's select over 64-bit (key, index) composites.
struct GPass {
  int32_t shift, width;
};

struct Plan {
  int64_t tokens, hidden, S, nsamples, M, tiles, nblocks;
  int32_t G, log2G, b_lo, b_hi;
  // allocation tiles (§3.2): A = kA * G channels, atiles in all, N per sample
  int64_t A, kA, atiles, N;
  int64_t k;  // allocation tiles per sample with b_hi
  // width layout of the encoder: 0 one width, 1 two widths (top-p% select),
  // 2 any candidate per tile (greedy allocator, 2-bit level map)
  int32_t allocator, mode;
  // greedy allocator: R bits per sample above c_1; nl upgrades per tile with
  // constants lam and costs cost; the select runs over composites of 32 key
  // bits and ib index bits unless every tile takes the same level (glevel >= 0)
  int64_t R;
  int32_t nl, ib, glevel, ngpasses, ngidx;
  float lam[3];
  int32_t cost[3];
  GPass gpasses[kMaxPasses];  // the three digits of the 32-bit key
  GPass gidx[3];              // the digits of the upgrade index (inside one workgroup per sample)
  int32_t x_dtype;
  float tau, budget;
  int32_t n_candidates;
  uint8_t candidates[4];
  // payload layout
  int64_t off_table, off_bitmap, off_side, off_scale, off_zero, off_codes, code_bytes, total;
  // workspace layout
  int64_t ws_status, ws_state, ws_hist, ws_H, ws_LS, ws_blockcnt, ws_table, ws_bitmap, ws_cand, ws_wtotal, ws_side,
      ws_total;
  // two-width layout built without the marking and scan launches: the last
  // entropy pass writes the width map's sure bits and the count of each run
  // of 64 tiles, the resolve kernel adds the tiles decided at the threshold
  // and scans the counts into the block table
  int32_t fold;
  int64_t ncand, cand_stride;  // capacity of a sample's candidate list; its uint32 words
  int32_t npasses;
  SelectPass passes[kMaxPasses];
};

// Per-sample state of the greedy allocator's select: the composite prefix
// found so far and the bit position (1-based, by weight) still to place in it.
struct GState {
  uint64_t prefix;
  int64_t r;
};

// Per-sample selection state, device resident.
struct SampleState {
  uint32_t key;     // orderable entropy key prefix; the k-th largest key once the entropy passes end
  uint32_t upos;    // tile-index prefix among tied keys; the last selected tied index at the end
  int64_t r;        // rank still to place (1-based) inside the current prefix
  int32_t tie_all;  // 1: every tile with the threshold key is selected
  int32_t pad;
};

struct Header {
  uint32_t w[32];  // the 128 header bytes
};

struct PadRanges {
  int64_t off[8];
  int32_t len[8];
  int32_t n;
};

// Launchers (return hipSuccess or the launch error).
// mode: the width layout (Plan::mode), 0 when the tensor is empty
hipError_t launch_encode(const Plan& pl, const void* x, void* payload, void* y, int y_dtype, void* ws,
                         hipStream_t st, int mode);
// Entropy of every allocation tile into h_out (pl.atiles values); side (may
// be null) receives every quantization tile's side byte (Eq. 3).
hipError_t launch_stats(const Plan& pl, const void* x, float* h_out, void* ws, bool init_select, uint8_t* side,
                        hipStream_t st);
hipError_t launch_select(const Plan& pl, void* payload, void* ws, hipStream_t st);
// Greedy allocator (tah_greedy.hip): levels, width sums, block table.
hipError_t launch_greedy(const Plan& pl, void* payload, void* ws, hipStream_t st);
// Exclusive scan of per-64-tile counts into the block table; total (may be
// null) receives the sum of all counts.
hipError_t launch_table(const uint32_t* cnt, uint32_t* table, uint32_t* total, int64_t nblocks, hipStream_t st);
hipError_t launch_decode(const Plan& pl, const void* payload, void* y, int y_dtype, void* ws, hipStream_t st);

// Backward compressor (tah_naive.hip).
int64_t naive_payload_bytes(int64_t n, int bits);
hipError_t launch_naive_encode(const void* g, int g_dtype, int64_t n, int bits, float c, void* payload,
                               hipStream_t st);
hipError_t launch_naive_decode(const void* payload, int64_t n, int bits, float c, void* y, int y_dtype, void* ws,
                               hipStream_t st);

// Tile-local Hadamard transform alone (tah_hadamard.hip); method 0 butterfly, 1 MFMA.
hipError_t launch_hadamard(const void* x, int x_dtype, int64_t tiles, int G, int method, float* y, hipStream_t st);

void make_header(const Plan& pl, Header* h);
void make_pads(const Plan& pl, PadRanges* pr);

}  // namespace tah
