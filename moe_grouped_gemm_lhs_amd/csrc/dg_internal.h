// dg_internal.h -- shared between the host library (dg_host.cpp) and the kernels
// (dg_kernels.hip).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dg {

constexpr int kBlockK = 128;       // depth of one scaled K block
constexpr int kAlignM = 128;       // contiguous-layout row alignment
// Stream-K workspace layout: arrival counters in a fixed header at offset 0 (every call
// leaves them zero, whatever its shape), fp32 partial tiles after it.
constexpr int kCounterSlots = 16384;
// Stream-K instances run at most this many workgroups (their workspace holds two
// partial tiles per workgroup).
constexpr int kStreamGrid = 256;

// Instance modes.
constexpr int kModeTiled = 0;    // one output tile per work item
constexpr int kModeStream = 2;   // persistent stream-K over (tile, K block) iterations

constexpr size_t kCounterBytes = kCounterSlots * sizeof(uint32_t);

enum Kind : int { kDense = 0, kContiguous = 1, kMasked = 2 };

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
  uint32_t* counters;         // stream-K arrival counters (workspace), or nullptr
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
  // grid size for a call (0 = nothing to launch)
  int (*grid)(const GemmArgs& a, int num_cus);
  void (*launch)(const GemmArgs& a, int grid, hipStream_t stream);
};

// Table of all instances compiled into the library (defined in dg_kernels.hip).
const Instance* instances(int* count);

}  // namespace dg
