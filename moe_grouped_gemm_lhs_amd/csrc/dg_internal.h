// dg_internal.h -- shared between the host library (dg_host.cpp) and the kernels
// (dg_kernels.hip).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dg {

constexpr int kBlockK = 128;       // depth of one scaled K block
constexpr int kAlignM = 128;       // contiguous-layout row alignment
// Stream-K instances run at most this many workgroups.
constexpr int kStreamGrid = 256;
// Stream-K workspace: one 8-byte record per (shared tile, wave) for up to kStreamGrid
// shared tiles of 8 waves (arrival count and completed parts), then two fp32 partial
// tiles per workgroup, stored bit-inverted (a zero word means "not written yet").  All
// of it must be zero filled before the first call, and every call leaves it zero filled.
constexpr int kArrivalBytes = kStreamGrid * 8 * 8;
// Bound on a contributor's polls for the other partials of its part of a shared tile
// (about a microsecond each); when it runs out the contributor leaves the part to the
// last contributor to arrive, which never waits.  The host may lower it per call
// (DG_HELPER_POLLS, for tests of that hand-over).
constexpr int kHelperPolls = 2000;

// Workgroups of a dense stream-K launch over `tiles` output tiles of `nkb` K blocks on
// a grid of at most `g` (min(CUs, kStreamGrid)): whole tiles dealt out evenly when that
// keeps at least 70% of the grid, so that no tile is shared and nothing is reduced;
// otherwise at least 8 iterations per workgroup, where a shared tile's hand-off costs
// more than the shorter loop saves; never more workgroups than iterations.
inline long stream_grid(long tiles, long nkb, long g) {
  const long work = tiles * nkb;
  if (work <= g) return work;
  for (long k = 1; k <= tiles; ++k) {
    if (tiles % k != 0 || tiles / k > g) continue;
    if (10 * (tiles / k) >= 7 * g) return tiles / k;
    break;
  }
  return work / 8 < g ? (work / 8 > 0 ? work / 8 : 1) : g;
}

// Instance modes.
constexpr int kModeTiled = 0;    // one output tile per work item
constexpr int kModeStream = 2;   // persistent stream-K over (tile, K block) iterations

enum Kind : int { kDense = 0, kContiguous = 1, kMasked = 2 };
enum Fmt : int { kFmtE4M3 = 0, kFmtE5M2 = 1 };

// Everything a kernel needs to know about one call.
struct GemmArgs {
  const uint8_t* A;
  const float* sA;
  const uint8_t* B;
  const float* sB;
  uint16_t* C;
  const int32_t* group_idx;   // contiguous only
  const int32_t* masked_m;    // masked only
  float* partial;             // stream-K fp32 partial tiles (workspace), or nullptr
  int* arrivals;              // stream-K arrival counters per shared tile (workspace)
  int helper_polls;           // stream-K: bound on an owner's polls (kHelperPolls)
  int rows;                   // dense M, contiguous M_total, masked cap
  int N, K, G;
  int nkb;                    // K / 128
  int nnb;                    // ceil(N / 128)
  int tiles_m;                // row tiles per group (masked) or overall
  int tiles_n;
  int num_tiles;              // tiles_m * tiles_n (* G for masked)
  int band;                   // row-tiles per raster band (tile order)
};

// One build-time kernel instance.
struct Instance {
  const char* name;
  int kind;          // Kind this instance serves
  int bm, bn;        // output tile
  int mode;          // kModeTiled or kModeStream
  int threads;       // workgroup size
  int fmt_a, fmt_b;  // operand formats (kFmtE4M3 / kFmtE5M2)
  // grid size for a call (0 = nothing to launch)
  int (*grid)(const GemmArgs& a, int num_cus);
  void (*launch)(const GemmArgs& a, int grid, hipStream_t stream);
};

// Table of all instances compiled into the library (defined in dg_kernels.hip).
const Instance* instances(int* count);

// fp8 block quantisation launch (defined in dg_quant.hip); arguments already validated.
void launch_quantize(int block128x128, int fmt, int bf16, const void* X, uint8_t* Q, float* S,
                     int64_t rows, int64_t K, int num_cus, hipStream_t stream);

// The library-owned split-K workspace of the current device (defined in
// dg_noalloc.hip): its capacity in bytes, and its address (looked up, and zeroed unless
// `stream` is capturing, on the first call for a device).
size_t scratch_capacity();
hipError_t scratch_for_current_device(void** out, hipStream_t stream);

// Byte-matrix transposition (defined in dg_quant.hip); arguments already validated.
void launch_transpose_u8(const uint8_t* X, uint8_t* Y, int64_t rows, int64_t cols,
                         hipStream_t stream);

}  // namespace dg
