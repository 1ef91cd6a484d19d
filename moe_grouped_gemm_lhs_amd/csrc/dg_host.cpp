// dg_host.cpp -- host side of libdg: argument validation, kernel-instance selection and
// launch for the three calls declared in include/dg.h.
//
// Validation is pure host code that touches no device state, so every error code
// except DG_ERR_DEVICE / DG_ERR_HIP can be produced on a machine without a GPU.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>

#include "dg.h"
#include "dg_internal.h"

namespace {

using dg::GemmArgs;
using dg::Instance;

constexpr int kMaxDevices = 64;

struct DeviceInfo {
  int checked;
  int ok;
  int num_cus;
};
DeviceInfo g_dev[kMaxDevices];
std::mutex g_dev_mu;

int log_enabled() {
  static const int v = [] {
    const char* e = getenv("DG_LOG");
    return (e && *e && strcmp(e, "0") != 0) ? 1 : 0;
  }();
  return v;
}

// Current device must be gfx950; caches the CU count.
dg_status check_device(int* num_cus) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return DG_ERR_DEVICE;
  }
  std::lock_guard<std::mutex> lk(g_dev_mu);
  DeviceInfo& d = g_dev[dev];
  if (!d.checked) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
      (void)hipGetLastError();
      return DG_ERR_DEVICE;
    }
    d.ok = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    d.num_cus = prop.multiProcessorCount;
    d.checked = 1;
  }
  if (!d.ok) return DG_ERR_DEVICE;
  *num_cus = d.num_cus;
  return DG_OK;
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Shape rules shared by every call.  rows_or_cap = M, M_total or cap.
constexpr int64_t kMaxK = (int64_t)1 << 22;

dg_status check_shape(int kind, int64_t rows_or_cap, int64_t N, int64_t K, int64_t G) {
  if (K <= 0 || K % dg::kBlockK != 0) return DG_ERR_SHAPE;
  if (rows_or_cap < 0 || N < 0 || G < 1) return DG_ERR_SHAPE;
  // 32-bit row, column and tile indices inside the kernels
  if (G > INT32_MAX || rows_or_cap > INT32_MAX || N > INT32_MAX || K > INT32_MAX)
    return DG_ERR_SHAPE;
  // 32-bit byte offsets inside a tile's rows of A and B (up to 256 rows of K bytes)
  if (K > kMaxK) return DG_ERR_SHAPE;
  // 32-bit tile indices, counted for the smallest tile (64 x 64)
  const int64_t groups = kind == dg::kMasked ? G : 1;
  if ((rows_or_cap + 63) / 64 * ((N + 63) / 64) > INT32_MAX / groups) return DG_ERR_SHAPE;
  if (kind == dg::kMasked && rows_or_cap * G > INT32_MAX) return DG_ERR_SHAPE;
  return DG_OK;
}

// The instance of that name built for these operand formats.
const Instance* find_instance(const char* name, int fa = dg::kFmtE4M3, int fb = dg::kFmtE4M3) {
  int n = 0;
  const Instance* all = dg::instances(&n);
  for (int i = 0; i < n; ++i)
    if (strcmp(all[i].name, name) == 0 && all[i].fmt_a == fa && all[i].fmt_b == fb)
      return &all[i];
  return nullptr;
}

bool valid_format(int f) { return f == DG_FP8_E4M3 || f == DG_FP8_E5M2; }

constexpr int kAssumedCUs = 256;   // MI355X; selection is host-only and device-free

// Relative time of a tiled launch: full rounds of tiles over the CUs times the tile's
// area, divided by how efficiently that tile shape runs (bigger tiles re-read less).
double tile_cost(int64_t rows, int64_t N, int64_t groups, int bm, int bn, double eff) {
  const int64_t tiles = cdiv(rows, bm) * cdiv(N, bn) * groups;
  const int64_t rounds = cdiv(tiles, kAssumedCUs);
  return (double)rounds * bm * bn / eff;
}

// A dense stream-K instance holds every row in one tile; the masked one schedules at
// most 64 groups (one per lane of a wave).
bool stream_fits(const Instance* in, int64_t rows, int64_t N, int64_t G) {
  if (in->mode != dg::kModeStream) return true;
  if (in->kind == dg::kMasked) return G <= 64;
  return rows <= in->bm;
}

// Instance selection: the heuristic that maps a problem to a build-time instance.
// DG_FORCE_INSTANCE=<name> overrides it when the named instance serves the call kind.
// Every tile shape is built for all four operand-format pairs, so the choice of shape
// does not depend on the formats; `fa` / `fb` only pick that shape's build.
const Instance* select_instance(int kind, int64_t rows_or_cap, int64_t N, int64_t K,
                                int64_t G, int fa = dg::kFmtE4M3, int fb = dg::kFmtE4M3) {
  const char* forced = getenv("DG_FORCE_INSTANCE");
  if (forced && *forced) {
    const Instance* f = find_instance(forced, fa, fb);
    if (f && f->kind == kind && stream_fits(f, rows_or_cap, N, G)) return f;
  }
  const char* name = nullptr;
  const int64_t groups = kind == dg::kMasked ? G : 1;
  switch (kind) {
    case dg::kDense:
      // decode-shaped (all rows in one tile): persistent stream-K over the column tiles
      // and K blocks
      if (rows_or_cap <= 128) {
        // 128-column tiles (half the re-reads of A per byte of B) unless their grid would
        // leave more than a quarter of the CUs idle; 64-column tiles then (twice the
        // tiles; measured: 64x24576x1536 17.5 -> 12.1 us and 128x4096x7168 18.9 -> 17.4
        // us with 128 columns; 2112x7168 and 7168x2048 keep 64)
        const int64_t tiles128 = cdiv(N, 128), nkb = K / dg::kBlockK;
        const int64_t grid128 = dg::stream_grid(tiles128, nkb, kAssumedCUs);
        const bool wide = 4 * grid128 >= 3 * kAssumedCUs;
        // ranges of 16 K blocks or more per workgroup: the 4-wave build of the 128-column
        // tile (128x7168x16384: 44.0 -> 39.7 us; it loses 2-7% on shorter ranges)
        const bool long_range = tiles128 * nkb >= 16 * grid128;
        if (rows_or_cap <= 64)
          name = !wide ? "dense_64x64_stream"
                       : long_range ? "dense_64x128_stream_4w" : "dense_64x128_stream";
        else
          name = !wide ? "dense_128x64_stream"
                       : long_range ? "dense_128x128_stream_4w" : "dense_128x128_stream";
        break;
      }
      /* fall through */
    case dg::kContiguous:
    case dg::kMasked: {
      const char* pre = kind == dg::kDense ? "dense" : kind == dg::kContiguous ? "contig" : "masked";
      // eff: measured throughput per unit of tile area, relative to 256x256.  The 256x224
      // tile does less MFMA work per K block for about the same fixed costs (0.88); the
      // contiguous form's 256x224 build also copies from every wave (0.75).
      // The dense 256x160 tile (for N near 2048: one round of tiles) runs at 0.80.
      const double eff224 = kind == dg::kContiguous ? 0.75 : 0.88;
      struct Opt { const char* suffix; int bm, bn; double eff; } opts[] = {
          {"256x256", 256, 256, 1.0}, {"256x224", 256, 224, eff224}, {"256x160", 256, 160, 0.80},
          {"128x128", 128, 128, 0.6}};
      double best = 1e300;
      char buf[64];   // per call: concurrent calls from several host threads are fine
      for (const Opt& o : opts) {
        snprintf(buf, sizeof(buf), "%s_%s", pre, o.suffix);
        if (!find_instance(buf, fa, fb)) continue;
        const double c = tile_cost(rows_or_cap, N, groups, o.bm, o.bn, o.eff);
        if (c < best) {
          best = c;
          name = find_instance(buf, fa, fb)->name;
        }
      }
      const int64_t tiles128 = cdiv(N, 128) * G;
      if (kind == dg::kMasked && rows_or_cap <= 128 && G <= 64 && tiles128 < kAssumedCUs) {
        // every group fits one 128-row tile but the tiles are fewer than the CUs: split-K
        // over the groups' column tiles and K blocks (scheduled on the device from
        // masked_m) spreads the work over every CU (with a tile per CU or more, the tiled
        // kernel is faster: no hand-off)
        const int64_t nkb = K / dg::kBlockK;
        name = tiles128 * nkb >= 16 * kAssumedCUs ? "masked_128x128_stream" : "masked_128x64_stream";
      } else if (kind == dg::kMasked && rows_or_cap <= 64) {
        name = "masked_64x128";      // more than 64 groups of at most 64 rows
      }
      break;
    }
    default:
      return nullptr;
  }
  return name ? find_instance(name, fa, fb) : nullptr;
}

// false if the tile count does not fit the kernels' 32-bit tile indices
bool fill_tiles(GemmArgs& a, const Instance* in, int kind) {
  a.nkb = a.K / dg::kBlockK;
  a.nnb = (int)cdiv(a.N, dg::kBlockK);
  a.tiles_m = (int)cdiv(a.rows, in->bm);
  a.tiles_n = (int)cdiv(a.N, in->bn);
  const int64_t tiles = (int64_t)a.tiles_m * a.tiles_n * (kind == dg::kMasked ? a.G : 1);
  a.num_tiles = tiles > INT32_MAX ? 0 : (int)tiles;
  a.band = a.tiles_m < 4 ? a.tiles_m : 4;
  return tiles <= INT32_MAX;
}

size_t workspace_for(const Instance* in, const GemmArgs& a) {
  if (!in) return 0;
  if (in->mode == dg::kModeStream)   // arrival counters, two partial tiles per workgroup
    return dg::kArrivalBytes + (size_t)dg::kStreamGrid * 2 * in->bm * in->bn * sizeof(float);
  return 0;
}

dg_status run(int kind, int fa, int fb, GemmArgs& a, void* workspace, size_t workspace_bytes,
              void* stream) {
  const Instance* in = select_instance(kind, a.rows, a.N, a.K, a.G, fa, fb);
  if (!in) return DG_ERR_SHAPE;
  if (!fill_tiles(a, in, kind)) return DG_ERR_SHAPE;
  const size_t ws = workspace_for(in, a);
  if (ws > 0) {
    if (!workspace || workspace_bytes < ws || !aligned(workspace, 16)) return DG_ERR_WORKSPACE;
    a.arrivals = (int*)workspace;
    a.partial = (float*)((uint8_t*)workspace + dg::kArrivalBytes);
    // DG_HELPER_POLLS=<n>: a smaller bound on the owners' polls, so that tests can make
    // every part of a shared tile fall to its last contributor
    a.helper_polls = dg::kHelperPolls;
    if (const char* e = getenv("DG_HELPER_POLLS")) {
      char* end = nullptr;
      const long v = strtol(e, &end, 10);
      if (end != e && v >= 0 && v < dg::kHelperPolls) a.helper_polls = (int)v;
    }
  }
  if (in->mode == dg::kModeStream && !a.partial)
    return DG_ERR_WORKSPACE;
  int num_cus = 0;
  dg_status st = check_device(&num_cus);
  if (st != DG_OK) return st;
  const int grid = in->grid(a, num_cus);
  if (log_enabled())
    fprintf(stderr, "[dg] kind=%d fmt=%d/%d rows=%d N=%d K=%d G=%d -> %s grid=%d\n", kind, fa,
            fb, a.rows, a.N, a.K, a.G, in->name, grid);
  if (grid <= 0) return DG_OK;
  (void)hipGetLastError();
  in->launch(a, grid, (hipStream_t)stream);
  if (hipGetLastError() != hipSuccess) return DG_ERR_HIP;
  return DG_OK;
}

}  // namespace

extern "C" {

int dg_get_m_alignment_for_contiguous_layout(void) { return dg::kAlignM; }

const char* dg_status_string(dg_status s) {
  switch (s) {
    case DG_OK: return "DG_OK";
    case DG_ERR_NULL: return "DG_ERR_NULL";
    case DG_ERR_SHAPE: return "DG_ERR_SHAPE";
    case DG_ERR_ALIGN: return "DG_ERR_ALIGN";
    case DG_ERR_WORKSPACE: return "DG_ERR_WORKSPACE";
    case DG_ERR_DEVICE: return "DG_ERR_DEVICE";
    case DG_ERR_HIP: return "DG_ERR_HIP";
    case DG_ERR_FORMAT: return "DG_ERR_FORMAT";
    default: return "DG_ERR_UNKNOWN";
  }
}

size_t dg_workspace_bytes(int kind, int64_t rows_or_cap, int64_t N, int64_t K, int64_t G) {
  if (kind < dg::kDense || kind > dg::kMasked) return 0;
  if (kind == dg::kDense) G = 1;
  if (check_shape(kind, rows_or_cap, N, K, G) != DG_OK) return 0;
  if (rows_or_cap == 0 || N == 0) return 0;
  const Instance* in = select_instance(kind, rows_or_cap, N, K, G);
  if (!in) return 0;
  GemmArgs a{};
  a.rows = (int)rows_or_cap;
  a.N = (int)N;
  a.K = (int)K;
  a.G = (int)G;
  if (!fill_tiles(a, in, kind)) return 0;
  return workspace_for(in, a);
}

const char* dg_instance_name(int kind, int64_t rows_or_cap, int64_t N, int64_t K, int64_t G) {
  if (kind < dg::kDense || kind > dg::kMasked) return "none";
  if (kind == dg::kDense) G = 1;
  if (check_shape(kind, rows_or_cap, N, K, G) != DG_OK)
    return "none";
  if (rows_or_cap == 0 || N == 0) return "none";
  const Instance* in = select_instance(kind, rows_or_cap, N, K, G);
  return in ? in->name : "none";
}

dg_status dg_gemm_fp8_nt_ex(const uint8_t* A, int a_format, const float* sA, const uint8_t* B,
                            int b_format, const float* sB, uint16_t* C, int64_t M, int64_t N,
                            int64_t K, void* workspace, size_t workspace_bytes, void* stream) {
  dg_status st = check_shape(dg::kDense, M, N, K, 1);
  if (st != DG_OK) return st;
  if (!valid_format(a_format) || !valid_format(b_format)) return DG_ERR_FORMAT;
  if (M == 0 || N == 0) return DG_OK;
  if (!A || !sA || !B || !sB || !C) return DG_ERR_NULL;
  if (!aligned(A, 16) || !aligned(B, 16) || !aligned(C, 16) || !aligned(sA, 4) ||
      !aligned(sB, 4))
    return DG_ERR_ALIGN;
  GemmArgs a{};
  a.A = A; a.sA = sA; a.B = B; a.sB = sB; a.C = C;
  a.rows = (int)M; a.N = (int)N; a.K = (int)K; a.G = 1;
  return run(dg::kDense, a_format, b_format, a, workspace, workspace_bytes, stream);
}

dg_status dg_gemm_fp8_nt(const uint8_t* A, const float* sA, const uint8_t* B, const float* sB,
                         uint16_t* C, int64_t M, int64_t N, int64_t K, void* workspace,
                         size_t workspace_bytes, void* stream) {
  return dg_gemm_fp8_nt_ex(A, DG_FP8_E4M3, sA, B, DG_FP8_E4M3, sB, C, M, N, K, workspace,
                           workspace_bytes, stream);
}

dg_status dg_gemm_fp8_nt_noalloc(const uint8_t* A, const float* sA, const uint8_t* B,
                                 const float* sB, uint16_t* C, int64_t M, int64_t N, int64_t K,
                                 void* stream) {
  dg_status st = check_shape(dg::kDense, M, N, K, 1);
  if (st != DG_OK) return st;
  if (M == 0 || N == 0) return DG_OK;
  if (!A || !sA || !B || !sB || !C) return DG_ERR_NULL;
  if (!aligned(A, 16) || !aligned(B, 16) || !aligned(C, 16) || !aligned(sA, 4) ||
      !aligned(sB, 4))
    return DG_ERR_ALIGN;
  const size_t need = dg_workspace_bytes(dg::kDense, M, N, K, 1);
  if (need > dg::scratch_capacity()) return DG_ERR_WORKSPACE;
  void* ws = nullptr;
  if (need > 0) {
    int num_cus = 0;
    st = check_device(&num_cus);
    if (st != DG_OK) return st;
    if (dg::scratch_for_current_device(&ws, (hipStream_t)stream) != hipSuccess) {
      (void)hipGetLastError();
      return DG_ERR_HIP;
    }
  }
  GemmArgs a{};
  a.A = A; a.sA = sA; a.B = B; a.sB = sB; a.C = C;
  a.rows = (int)M; a.N = (int)N; a.K = (int)K; a.G = 1;
  return run(dg::kDense, DG_FP8_E4M3, DG_FP8_E4M3, a, ws, need, stream);
}

dg_status dg_grouped_gemm_fp8_contiguous_ex(const uint8_t* A, int a_format, const float* sA,
                                            const uint8_t* B, int b_format, const float* sB,
                                            const int32_t* group_idx, uint16_t* C,
                                            int64_t M_total, int64_t N, int64_t K, int64_t G,
                                            void* workspace, size_t workspace_bytes,
                                            void* stream) {
  dg_status st = check_shape(dg::kContiguous, M_total, N, K, G);
  if (st != DG_OK) return st;
  if (!valid_format(a_format) || !valid_format(b_format)) return DG_ERR_FORMAT;
  if (M_total == 0 || N == 0) return DG_OK;
  if (!A || !sA || !B || !sB || !group_idx || !C) return DG_ERR_NULL;
  if (!aligned(A, 16) || !aligned(B, 16) || !aligned(C, 16) || !aligned(sA, 4) ||
      !aligned(sB, 4) || !aligned(group_idx, 4))
    return DG_ERR_ALIGN;
  GemmArgs a{};
  a.A = A; a.sA = sA; a.B = B; a.sB = sB; a.C = C; a.group_idx = group_idx;
  a.rows = (int)M_total; a.N = (int)N; a.K = (int)K; a.G = (int)G;
  return run(dg::kContiguous, a_format, b_format, a, workspace, workspace_bytes, stream);
}

dg_status dg_grouped_gemm_fp8_contiguous(const uint8_t* A, const float* sA, const uint8_t* B,
                                         const float* sB, const int32_t* group_idx,
                                         uint16_t* C, int64_t M_total, int64_t N, int64_t K,
                                         int64_t G, void* workspace, size_t workspace_bytes,
                                         void* stream) {
  return dg_grouped_gemm_fp8_contiguous_ex(A, DG_FP8_E4M3, sA, B, DG_FP8_E4M3, sB, group_idx,
                                           C, M_total, N, K, G, workspace, workspace_bytes,
                                           stream);
}

dg_status dg_grouped_gemm_fp8_masked_ex(const uint8_t* A, int a_format, const float* sA,
                                        const uint8_t* B, int b_format, const float* sB,
                                        const int32_t* masked_m, uint16_t* C, int64_t G,
                                        int64_t cap, int64_t N, int64_t K, void* workspace,
                                        size_t workspace_bytes, void* stream) {
  dg_status st = check_shape(dg::kMasked, cap, N, K, G);
  if (st != DG_OK) return st;
  if (!valid_format(a_format) || !valid_format(b_format)) return DG_ERR_FORMAT;
  if (cap == 0 || N == 0) return DG_OK;
  if (!A || !sA || !B || !sB || !masked_m || !C) return DG_ERR_NULL;
  if (!aligned(A, 16) || !aligned(B, 16) || !aligned(C, 16) || !aligned(sA, 4) ||
      !aligned(sB, 4) || !aligned(masked_m, 4))
    return DG_ERR_ALIGN;
  GemmArgs a{};
  a.A = A; a.sA = sA; a.B = B; a.sB = sB; a.C = C; a.masked_m = masked_m;
  a.rows = (int)cap; a.N = (int)N; a.K = (int)K; a.G = (int)G;
  return run(dg::kMasked, a_format, b_format, a, workspace, workspace_bytes, stream);
}

dg_status dg_grouped_gemm_fp8_masked(const uint8_t* A, const float* sA, const uint8_t* B,
                                     const float* sB, const int32_t* masked_m, uint16_t* C,
                                     int64_t G, int64_t cap, int64_t N, int64_t K,
                                     void* workspace, size_t workspace_bytes, void* stream) {
  return dg_grouped_gemm_fp8_masked_ex(A, DG_FP8_E4M3, sA, B, DG_FP8_E4M3, sB, masked_m, C, G,
                                       cap, N, K, workspace, workspace_bytes, stream);
}

static dg_status quantize(int block128x128, const void* X, int x_dtype, uint8_t* Q, float* S,
                          int64_t rows, int64_t K, int format, void* stream) {
  if (rows < 0 || K <= 0 || K % dg::kBlockK != 0 || rows > INT32_MAX || K > INT32_MAX)
    return DG_ERR_SHAPE;
  if (rows * (K / dg::kBlockK) > (int64_t)INT32_MAX * 4) return DG_ERR_SHAPE;   // grid
  if (!valid_format(format) || (x_dtype != DG_IN_F32 && x_dtype != DG_IN_BF16))
    return DG_ERR_FORMAT;
  if (rows == 0) return DG_OK;
  if (!X || !Q || !S) return DG_ERR_NULL;
  if (!aligned(X, 16) || !aligned(Q, 8) || !aligned(S, 4))
    return DG_ERR_ALIGN;
  int num_cus = 0;
  const dg_status st = check_device(&num_cus);
  if (st != DG_OK) return st;
  (void)hipGetLastError();
  dg::launch_quantize(block128x128, format, x_dtype == DG_IN_BF16, X, Q, S, rows, K, num_cus,
                      (hipStream_t)stream);
  return hipGetLastError() == hipSuccess ? DG_OK : DG_ERR_HIP;
}

dg_status dg_quantize_fp8_1x128(const void* X, int x_dtype, uint8_t* Q, float* S, int64_t rows,
                                int64_t K, int format, void* stream) {
  return quantize(0, X, x_dtype, Q, S, rows, K, format, stream);
}

dg_status dg_quantize_fp8_128x128(const void* X, int x_dtype, uint8_t* Q, float* S,
                                  int64_t rows, int64_t K, int format, void* stream) {
  return quantize(1, X, x_dtype, Q, S, rows, K, format, stream);
}

dg_status dg_transpose_fp8(const uint8_t* X, uint8_t* Y, int64_t rows, int64_t cols,
                           void* stream) {
  if (rows < 0 || cols < 0 || rows % 16 != 0 || cols % 16 != 0) return DG_ERR_SHAPE;
  if (((rows + 63) / 64) * ((cols + 63) / 64) > INT32_MAX) return DG_ERR_SHAPE;
  if (rows == 0 || cols == 0) return DG_OK;
  if (!X || !Y) return DG_ERR_NULL;
  if (!aligned(X, 16) || !aligned(Y, 16)) return DG_ERR_ALIGN;
  int num_cus = 0;
  const dg_status st = check_device(&num_cus);
  if (st != DG_OK) return st;
  (void)hipGetLastError();
  dg::launch_transpose_u8(X, Y, rows, cols, (hipStream_t)stream);
  return hipGetLastError() == hipSuccess ? DG_OK : DG_ERR_HIP;
}

}  // extern "C"
