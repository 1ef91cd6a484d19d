// dg_kernels.hip -- FP8 (e4m3fn) block-scaled NT GEMM kernels for gfx950 (CDNA4).
//
// One templated tile body serves the three forms (dense, contiguous-grouped,
// masked-grouped); the tile scheduler and the epilogue's row predicate differ.
// For each output tile and each 128-deep K block kb:
//   1. the e4m3 bytes of A[m0:m0+BM, kb] and B_g[n0:n0+BN, kb], the scales
//      sA[m0:m0+BM, kb] and the few sB_g[nb, kb] the tile needs are copied global -> LDS
//      with direct-to-LDS buffer loads (buffer_load_dwordx4 / _dword ... lds), STAGES blocks
//      ahead, so that HBM/L2 traffic for later blocks overlaps the math of this one;
//   2. each 16x16 sub-tile's fp32 block partial comes from one
//      v_mfma_f32_16x16x128_f8f6f4 started from zero;
//   3. the partial is promoted on the VALU, acc += partial * (sA[m,kb] * sB[n/128,kb]),
//      into a separate fp32 register accumulator: the two-level accumulation of the
//      DeepGEMM pages (turtlesai.it summary, technical paragraph; chattools.cn, core
//      design ideas).  MFMA issue and the promotion of the partial from two steps
//      earlier are interleaved by hand (scheduler fences), so the matrix pipe stays
//      busy while the VALU works and only three partials are alive at a time;
//   4. after the last K block the accumulator is rounded to bf16 (nearest-even) and
//      stored, predicated on the rows the form may write.
//
// MFMA operand layout.  v_mfma_f32_16x16x128_f8f6f4 takes 32 bytes per lane for each
// operand: lane l supplies row l%16 of the first operand and column l%16 of the second,
// lane group q = l/16 a quarter of the 128-deep block.  Which K positions a (q, byte)
// slot holds does not matter for a dot product as long as both operands use the same
// assignment; here lane group q takes 16-byte chunks q and q+4 of the row's block.  B is
// passed as the first operand and A as the second, so the result lane l holds is
// C[m = l%16][n = 4(l/16) .. 4(l/16)+3]: one row and four consecutive columns.  Hence a
// lane needs one sA value per 16-row sub-tile, and stores four bf16 at once.
//
// LDS layout of a staged operand: 128 bytes per row = 8 chunks of 16 bytes; chunk c of
// row r sits in slot c ^ (r & 7), so the eight lanes that read the same chunk of eight
// consecutive rows hit eight different bank groups.  A direct-to-LDS instruction writes
// 64 lanes x 16 bytes = 8 rows x 128 bytes contiguously; each lane fetches the global
// chunk that belongs in its slot.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dg_internal.h"

namespace dg {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

// Format codes of the f8f6f4 MFMA operands: 0 = E4M3, 1 = E5M2 (the values of
// DG_FP8_E4M3 / DG_FP8_E5M2).  FA is the format of the instruction's first operand,
// FB of its second; the scale operands are 0 (no hardware block scaling).
template <int FA, int FB>
__device__ __forceinline__ v4f mfma_fp8_16x16x128(const v8i& a, const v8i& b) {
  const v4f zero = {0.f, 0.f, 0.f, 0.f};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, zero, FA, FB, 0, 0, 0, 0);
}

// s_waitcnt with only the vector-memory counter constrained (expcnt/lgkmcnt untouched).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// s_waitcnt lgkmcnt(0): this wave's LDS accesses are complete (vmcnt untouched).
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// Wait until at most `ahead` stages (PER loads each) of this wave are still in flight.
template <int PER, int A>
__device__ __forceinline__ void wait_stages_ahead(int ahead) {
  if constexpr (A <= 0) {
    wait_vmcnt<0>();
  } else {
    if (ahead >= A)
      wait_vmcnt<A * PER>();
    else
      wait_stages_ahead<PER, A - 1>(ahead);
  }
}

// The same for a kernel instance's copies: PER_STAGE per stage for the waves that also
// copy scales, PER_N for the other copy waves; waves that copy nothing do not wait (the
// barrier that follows orders them after the copy waves' waits).  `wave` is uniform.
template <class C, int A>
__device__ __forceinline__ void wait_stage_copies(int wave, int ahead) {
  if (wave < C::S_WAVES)
    wait_stages_ahead<C::PER_STAGE, A>(ahead);
  else if (wave < C::CW)
    wait_stages_ahead<C::PER_N, A>(ahead);
}

// The tiled kernel's wait: besides `ahead` later stages of copies, `epis` tile epilogues
// of NST stores each may have been issued after the awaited copies (vmcnt counts loads
// and stores together, and they retire in issue order).
template <int PER, int EXTRA, int A>
__device__ __forceinline__ void wait_ahead_plus(int ahead) {
  if constexpr (A <= 0) {
    wait_vmcnt<EXTRA>();
  } else {
    if (ahead >= A)
      wait_vmcnt<A * PER + EXTRA>();
    else
      wait_ahead_plus<PER, EXTRA, A - 1>(ahead);
  }
}
template <int PER, int NST, int A, int E, int PF>
__device__ __forceinline__ void wait_ahead_epi(int ahead, int epis) {
  if constexpr (E <= 0) {
    wait_ahead_plus<PER, PF, A>(ahead);
  } else {
    if (epis >= E)
      wait_ahead_plus<PER, E * NST + PF, A>(ahead);
    else
      wait_ahead_epi<PER, NST, A, E - 1, PF>(ahead, epis);
  }
}
// A wave that issues an L2 prefetch after each stage's copies (waves below C::PF_WAVES)
// counts PER + 1 loads per stage, and the awaited stage's own prefetch may stay in
// flight: it retires after that stage's copies.
template <class C, int NST, int PER>
__device__ __forceinline__ void wait_copies_pf(int wave, int ahead, int epis) {
  if (wave < C::PF_WAVES)
    wait_ahead_epi<PER + 1, NST, C::STAGES - 2, C::STAGES - 1, 1>(ahead, epis);
  else
    wait_ahead_epi<PER, NST, C::STAGES - 2, C::STAGES - 1, 0>(ahead, epis);
}
template <class C, int NST>
__device__ __forceinline__ void wait_copies_epi(int wave, int ahead, int epis) {
  if (wave < 0) return;   // a compute-only wave: it has no copies to wait for
  if (wave < C::S_WAVES)
    wait_copies_pf<C, NST, C::PER_STAGE>(wave, ahead, epis);
  else if (wave < C::CW)
    wait_copies_pf<C, NST, C::PER_N>(wave, ahead, epis);
}

// Buffer resource over `bytes` bytes from `base` (raw, stride 0): a load at an offset
// past the end returns zeros without touching memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_over(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}

// Direct-to-LDS buffer loads: 16 (or 4) bytes per lane at byte offset `off`, the wave's
// 64 lanes landing contiguously at `lds`.  AUX is the cache policy (0: default,
// 2: non-temporal, for operands that are read once and would only evict reused data).
template <int AUX = 0>
__device__ __forceinline__ void copy16(__amdgpu_buffer_rsrc_t r, int off, void* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 16, off, 0, 0, AUX);
}
__device__ __forceinline__ void copy4(__amdgpu_buffer_rsrc_t r, int off, void* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 4, off, 0, 0, 0);
}
// The same with the offset split into a per-lane part (one VGPR shared by a run of
// copies) and a uniform part in the instruction's scalar offset: no address arithmetic
// on the VALU per copy.
template <int AUX = 0>
__device__ __forceinline__ void copy16s(__amdgpu_buffer_rsrc_t r, int voff, int soff, void* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 16, voff, soff, 0, AUX);
}

// bf16 rounding (nearest, ties to even) by the hardware's packed conversion
// (v_cvt_pk_bf16_f32): bit-identical to the software rounding on finite values, ties,
// denormals and overflow to infinity (4M-value check on gfx950); NaN stays a NaN.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16x2_rne(float a, float b) {
  const bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ uint16_t bf16_rne(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Read-only int32 metadata at a workgroup-uniform index, through the scalar cache (the
// constant address space): the load counts on lgkmcnt, so waiting for it never waits for
// the vector-memory copies and stores in flight.
typedef const __attribute__((address_space(4))) int32_t scalar_i32;
__device__ __forceinline__ int load_uniform(const int32_t* p, long i) {
  return ((scalar_i32*)p)[i];
}

// Split-K partials are stored bit-inverted, so that an all-zero word marks a slot not
// yet written (the workspace's partial slots start zero filled and every call leaves
// them so).  The only value whose inverse is zero, the NaN with every bit set, is first
// replaced by another NaN.
__device__ __forceinline__ v4i encode_partial(v4f v) {
  v4i u = __builtin_bit_cast(v4i, v);
#pragma unroll
  for (int e = 0; e < 4; ++e) u[e] = ~(u[e] == -1 ? (int)0xFFC00000u : u[e]);
  return u;
}
__device__ __forceinline__ v4f decode_partial(v4i u) { return __builtin_bit_cast(v4f, ~u); }

// Cache policy of loads that poll for another workgroup's partials: sc1 (device
// coherent) plus the intrinsic's volatile bit, so that each poll stays inside its loop.
constexpr int kPollAux = (int)0x80000010u;

// One MFMA operand fragment from LDS (32 bytes per lane: chunks q and q+4 of the lane's
// row, at their swizzled slots), given the lane's pointers to those two chunks in the
// operand's first 16-row block: rows r and r + 16k share r & 7 and so the same slots,
// hence block b sits at a constant offset (an LDS-read immediate).
__device__ __forceinline__ v8i read_frag_block(const uint8_t* lo, const uint8_t* hi, int b) {
  const v4i l = *(const v4i*)(lo + b * 16 * kBlockK);
  const v4i h = *(const v4i*)(hi + b * 16 * kBlockK);
  return (v8i){l.x, l.y, l.z, l.w, h.x, h.y, h.z, h.w};
}

// Workgroup barrier without the memory fence of __syncthreads(): that fence waits for
// every outstanding vector-memory operation, i.e. it would drain the direct-to-LDS loads
// of all the stages that are meant to stay in flight.  Each wave instead waits for its
// own loads of the stage it is about to read (wait_stages_ahead) before the barrier.
// The empty asm statements keep the compiler from moving memory accesses across.
__device__ __forceinline__ void stage_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Compile-time shape of one kernel instance.
// B_NT: B blocks are read by exactly one workgroup (decode shapes), so they are loaded
// non-temporal.  FMT_A / FMT_B: operand formats (0: E4M3, 1: E5M2).
// CW_: how many waves issue the stage copies (0: all).
// XW_: copy-only waves after the compute waves (0: none).  With XW_ > 0 the XW_ extra
// waves issue every copy and never compute, and the compute waves issue none: a wave's
// MFMAs then never queue behind its own copies in the CU's address unit, which all
// copying waves share.  A wave's copies queue in the CU's
// address unit behind the other waves' (one 1 KB copy per 16 clocks at most), and a wave
// cannot start its MFMAs until its own copies are issued; with two waves per SIMD, giving
// all copies to the first wave of each SIMD lets the second start computing at once.
template <int BM_, int BN_, int WAVES_M_, int WAVES_N_, int STAGES_, bool B_NT_ = false,
          int FMT_A_ = 0, int FMT_B_ = 0, int CW_ = 0, int PFD_ = 0, int XW_ = 0>
struct Cfg {
  static constexpr int BM = BM_, BN = BN_, WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
  static constexpr int STAGES = STAGES_;
  static constexpr bool B_NT = B_NT_;
  static constexpr int FMT_A = FMT_A_, FMT_B = FMT_B_;
  static constexpr int W = WAVES_M * WAVES_N;    // compute waves: 0 .. W-1
  static constexpr int XW = XW_;
  static constexpr int CW = XW_ ? XW_ : (CW_ ? CW_ : W);   // copy waves: CW0 .. CW0+CW-1
  static constexpr int CW0 = XW_ ? W : 0;
  static constexpr int NT = 64 * (W + XW_);
  static constexpr int WM = BM / WAVES_M;       // rows per wave
  static constexpr int WN = BN / WAVES_N;       // columns per wave
  static constexpr int TI = WM / 16;            // 16-row sub-tiles per wave
  static constexpr int TJ = WN / 16;            // 16-column sub-tiles per wave
  // 1 KB direct loads (8 rows) per copy wave per stage; when the 8-row blocks do not
  // split evenly over the copy waves, the last loads fill padding rows that are never read
  static constexpr int A_DMA = (BM / 8 + CW - 1) / CW;
  static constexpr int B_DMA = (BN / 8 + CW - 1) / CW;
  static constexpr int A_BYTES = A_DMA * CW * 8 * kBlockK;
  static constexpr int B_BYTES = B_DMA * CW * 8 * kBlockK;
  static constexpr int NBV = (BN + 127) / 128 + 1;   // sB blocks a tile can touch
  // scale slots: sA for BM rows, then the tile's sB values, 64 per 4-byte-per-lane copy;
  // the first S_WAVES waves issue S_PER such copies each per stage
  static constexpr int S_COPIES = (BM + NBV + 63) / 64;
  static constexpr int S_WAVES = S_COPIES < CW ? S_COPIES : CW;
  static constexpr int S_PER = (S_COPIES + CW - 1) / CW;
  static constexpr int S_FLOATS = 64 * S_PER * S_WAVES;
  static constexpr int STAGE_BYTES = A_BYTES + B_BYTES + 4 * S_FLOATS;
  // copies per stage of a copy wave without / with scale copies
  static constexpr int PER_N = A_DMA + B_DMA;
  static constexpr int PER_STAGE = PER_N + S_PER;
  // L2 prefetch PFD K blocks ahead of each stage's copies (0: none), one load each by
  // waves 0 (A rows) and 1 (B rows)
  static constexpr int PFD = PFD_;
  static constexpr int PF_WAVES = PFD_ > 0 ? 2 : 0;
  // LDS after the stages: the prefetch scratch slot, then (contiguous form) two slots of
  // the tile rows' group indices, one per work item in flight
  static constexpr int PF_OFF = STAGES * STAGE_BYTES;
  static constexpr int GI_OFF = PF_OFF + (PFD_ > 0 ? 256 : 0);
  static constexpr int LDS_BYTES = GI_OFF + 2 * BM * 4;
  // every wave's columns fall inside one 128-column scale block
  static constexpr bool ONE_NB =
      (128 % WN == 0) && ((BN % 128 == 0) || (128 % BN == 0));
  static_assert(BM % (16 * WAVES_M) == 0 && BN % (16 * WAVES_N) == 0, "tile shape");
  static_assert(BM % 8 == 0 && BN % 8 == 0, "direct-load blocks");
  static_assert(BM + NBV <= S_FLOATS && S_WAVES <= CW && CW <= W, "scale slots");
  static_assert(PER_N >= 1, "every wave copies operand bytes");
  static_assert(STAGES >= 2 && (STAGES - 2) * PER_STAGE < 64, "pipeline depth");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
  static_assert(PFD_ == 0 || (S_WAVES >= 2 && BM <= 512 && BN <= 256), "prefetch waves");
};

// Where one output tile lives, and which rows of it may be computed.
struct TileRef {
  int ok;        // 0: nothing to do
  int g;         // group of the first 128-row block (contiguous) / group (masked)
  int g2;        // contiguous only: group of the second 128-row block, or -1
  int m0;        // first row of the tile inside the group's row range
  int row_base;  // global row (A, sA, C) of the group's row 0
  int rows;      // rows of this tile that exist (>= 1 when ok)
  int n0;
  int lead0, lead1;  // contiguous only: group index of each 128-row block's first row
};

template <int KIND, class C>
__device__ __forceinline__ TileRef locate_tile(const GemmArgs& p, int t) {
  TileRef r;
  r.ok = 1;
  r.g2 = -1;
  r.lead0 = r.lead1 = -1;
  int tm, tn;
  if (KIND == kMasked) {
    const int per_g = p.tiles_m * p.tiles_n;
    r.g = t / per_g;
    t -= r.g * per_g;
  } else {
    r.g = 0;
  }
  // grouped raster: bands of `band` row-tiles, column-major inside a band, so that
  // tiles that run together share A rows and B columns
  const int band = p.band;
  const int per_band = band * p.tiles_n;
  const int b = t / per_band;
  const int in_band = t - b * per_band;
  const int rows_in_band = min(band, p.tiles_m - b * band);
  tm = b * band + in_band % rows_in_band;
  tn = in_band / rows_in_band;
  r.m0 = tm * C::BM;
  r.n0 = tn * C::BN;
  if (KIND == kMasked) {
    int valid = load_uniform(p.masked_m, r.g);
    valid = valid < 0 ? 0 : (valid > p.rows ? p.rows : valid);
    r.row_base = r.g * p.rows;
    r.rows = min(C::BM, valid - r.m0);
    r.ok = r.m0 < valid;
  } else {
    r.row_base = 0;
    r.rows = min(C::BM, p.rows - r.m0);
    if (KIND == kContiguous) {
      // the tile holds one or two 128-row blocks; each block's leading index names
      // the only group its rows may be written with
      r.lead0 = load_uniform(p.group_idx, r.m0);
      r.lead1 = C::BM > kAlignM && r.rows > kAlignM ? load_uniform(p.group_idx, r.m0 + kAlignM)
                                                     : -1;
      r.g = r.lead0;
      r.g2 = r.lead1;
      if (r.g2 == r.g || r.g2 < 0 || r.g2 >= p.G) r.g2 = -1;
      if (r.g < 0 || r.g >= p.G) {
        r.g = r.g2;
        r.g2 = -1;
      }
      r.ok = r.g >= 0;
    }
  }
  r.g = uniform(r.g);
  r.g2 = uniform(r.g2);
  r.ok = uniform(r.ok);
  return r;
}

// Per (tile, group) values the staging and the math need.
struct TileCtx {
  const uint8_t* A;
  const float* sA;
  const uint8_t* Bg;
  const float* sBg;
  int K, nkb, nnb, N;
  int a_row0;    // global row of the tile's first row
  int rows;      // rows of the tile that exist
  int n0;
  int nb_first;  // sB block of column n0
  int wave, lane, wm, wn, q, l16;
  int cw;        // index among the copy waves (negative: a wave that issues no copies)
  int gslot;     // contiguous form: the LDS slot of this item's group indices
};

// Direct-to-LDS copy of K block kb of the tile into stage `st`.  The copies go through
// buffer resources that span only the tile's valid rows of A and columns of B (and their
// scales): a lane whose offset falls past the end reads zeros without touching memory,
// so the rows and columns past the matrix edge need no clamping and their (never
// stored) outputs come from zeros.  Every offset is a per-lane VGPR term plus a uniform
// term, all in the range-checked vector offset.  FRESH (the tiled kernel, whose loops
// keep more state live): the offsets are rebuilt at every call instead of kept in
// registers across calls.
template <class C, bool FRESH = false, bool GI = false>
__device__ __forceinline__ void issue_stage(uint8_t* __restrict__ st, const TileCtx& c, int kb,
                                            uint8_t* base = nullptr,
                                            const int32_t* gidx = nullptr) {
  if (c.cw < 0 || c.cw >= C::CW) return;   // not a copy wave
  if (GI && kb == 0 && c.cw == 0) {
    // contiguous form, with the item's first K block: its rows' group indices into the
    // item's LDS slot, for the epilogue's row checks (rows past the tile's valid ones
    // read zeros; the epilogue never stores them)
    const __amdgpu_buffer_rsrc_t rg = buffer_over(gidx + c.a_row0, c.rows * 4);
    uint8_t* gl = base + C::GI_OFF + c.gslot * (C::BM * 4);
#pragma unroll
    for (int it = 0; it < C::BM / 64; ++it) copy4(rg, (it * 64 + c.lane) * 4, gl + it * 256);
  }
  const int sub = c.lane >> 3;             // row inside the 8-row block
  const int ch = (c.lane & 7) ^ sub;       // global chunk for this lane's slot
  const int K = c.K;
  const __amdgpu_buffer_rsrc_t ra = buffer_over(c.A + (size_t)c.a_row0 * K, c.rows * K);
  const __amdgpu_buffer_rsrc_t rb =
      buffer_over(c.Bg + (size_t)c.n0 * K, min(C::BN, c.N - c.n0) * K);
  const int lane_off = sub * K + ch * 16;
  if constexpr (FRESH) {
    // The uniform parts are advanced copy by copy from starting values the compiler
    // cannot see through, so it keeps no per-copy offsets or LDS addresses live from
    // one call to the next (one per-lane term and a few scalars per call instead).
    int ua = c.cw * (C::A_DMA * 8) * K + kb * kBlockK, da = c.cw * C::A_DMA * 1024;
    int ub = c.cw * (C::B_DMA * 8) * K + kb * kBlockK, db = C::A_BYTES + c.cw * C::B_DMA * 1024;
    asm volatile("" : "+s"(ua), "+s"(da), "+s"(ub), "+s"(db));
#pragma unroll
    for (int it = 0; it < C::A_DMA; ++it, ua += 8 * K)
      copy16s<0>(ra, lane_off, ua, st + da + it * 1024);
#pragma unroll
    for (int it = 0; it < C::B_DMA; ++it, ub += 8 * K)
      copy16s<C::B_NT ? 2 : 0>(rb, lane_off, ub, st + db + it * 1024);
  } else {
#pragma unroll
    for (int it = 0; it < C::A_DMA; ++it) {
      const int cb = c.cw * C::A_DMA + it;
      copy16<0>(ra, lane_off + (cb * 8 * K + kb * kBlockK), st + cb * 1024);
    }
#pragma unroll
    for (int it = 0; it < C::B_DMA; ++it) {
      const int cb = c.cw * C::B_DMA + it;
      copy16<C::B_NT ? 2 : 0>(rb, lane_off + (cb * 8 * K + kb * kBlockK),
                              st + C::A_BYTES + cb * 1024);
    }
  }
  if (c.cw < C::S_WAVES) {
    // slot s < BM: sA of row s; slot BM + j: sB of column block nb_first + j (the slots
    // after the tile's NBV blocks, and any padding slots, are filled but never read)
    const __amdgpu_buffer_rsrc_t rsa =
        buffer_over(c.sA + (size_t)c.a_row0 * c.nkb, c.rows * c.nkb * 4);
    // sB: only the NBV blocks the tile can touch, so that the other lanes of its copy
    // (one sB row each, a line apiece) fetch nothing
    const __amdgpu_buffer_rsrc_t rsb = buffer_over(
        c.sBg + (size_t)c.nb_first * c.nkb, min(C::NBV, c.nnb - c.nb_first) * c.nkb * 4);
    int sl = c.lane;
    if (FRESH) asm volatile("" : "+v"(sl));
    const int s_off = sl * c.nkb * 4 + kb * 4;
#pragma unroll
    for (int it = 0; it < C::S_PER; ++it) {
      const int slot = c.cw * C::S_PER + it;
      uint8_t* dst = st + C::A_BYTES + C::B_BYTES + slot * 256;
      if (slot * 64 < C::BM)
        copy4(rsa, s_off + slot * 64 * c.nkb * 4, dst);
      else
        copy4(rsb, s_off + (slot * 64 - C::BM) * c.nkb * 4, dst);
    }
  }
  if (C::PF_WAVES > 0 && c.cw < C::PF_WAVES) {
    // The lines of K block kb + PFD that this workgroup brings into the L2 for its XCD.
    // The 32 workgroups of an XCD run 32 consecutive tiles, 4 row tiles by 8 column tiles
    // (4-row-tile bands, column-major), so each A row tile is read by 8 of them and each
    // B column tile by 4: each touches 1/8 of its A rows (wave 0) and 1/4 of its B rows
    // (wave 1), one 4-byte load per row into a slot that is never read, and every line of
    // that block is fetched once, PFD - 1 steps before the copies that read it.  Lanes
    // without a row, and blocks past the last, use an offset outside the resource, which
    // fetches nothing.
    const int kp = kb + C::PFD;
    const int tn = c.n0 / C::BN, tm = c.a_row0 / C::BM;
    int row = -1;
    if (c.cw == 0 && c.lane < C::BM / 8) row = (tn & 7) * (C::BM / 8) + c.lane;
    if (c.cw == 1 && c.lane < C::BN / 4) row = (tm & 3) * (C::BN / 4) + c.lane;
    const int off = kp < c.nkb && row >= 0 ? row * K + kp * kBlockK : 0x7FFFFFF0;
    copy4(c.cw == 1 ? rb : ra, off, base + C::PF_OFF);
  }
}

// MFMA block partials of one staged K block, promoted into acc.
template <class C>
__device__ __forceinline__ void compute_stage(const uint8_t* __restrict__ st, const TileCtx& c,
                                              v4f (&acc)[C::TI][C::TJ]) {
  constexpr int TI = C::TI, TJ = C::TJ, WM = C::WM, WN = C::WN;
  const uint8_t* As = st;
  const uint8_t* Bs = st + C::A_BYTES;
  const float* Ss = (const float*)(st + C::A_BYTES + C::B_BYTES);
  const int q = c.q, l16 = c.l16;

  // lane pointers to chunks q and q+4 of this lane's row in the wave's first 16-row
  // block of A and of B
  const int lo = l16 * kBlockK + ((q ^ (l16 & 7)) << 4);
  const int hi = l16 * kBlockK + (((q + 4) ^ (l16 & 7)) << 4);
  const uint8_t* a_lo = As + c.wm * WM * kBlockK + lo;
  const uint8_t* a_hi = As + c.wm * WM * kBlockK + hi;
  const uint8_t* b_lo = Bs + c.wn * WN * kBlockK + lo;
  const uint8_t* b_hi = Bs + c.wn * WN * kBlockK + hi;
  v8i af[TI];
  float sa[TI];
#pragma unroll
  for (int i = 0; i < TI; ++i) {
    af[i] = read_frag_block(a_lo, a_hi, i);
    sa[i] = Ss[c.wm * WM + 16 * i + l16];
  }
  float sb[TJ];
#pragma unroll
  for (int j = 0; j < TJ; ++j) {
    const int nb = min((c.n0 + c.wn * WN + 16 * j) / kBlockK, c.nnb - 1);
    sb[j] = Ss[C::BM + nb - c.nb_first];
  }
  float s_i[TI];
  if (C::ONE_NB) {
#pragma unroll
    for (int i = 0; i < TI; ++i) s_i[i] = sa[i] * sb[0];
  }
  v8i bf[2];
  bf[0] = read_frag_block(b_lo, b_hi, 0);
  __builtin_amdgcn_sched_barrier(0);

  // software pipeline: MFMA for step t, promotion of step t-2
  constexpr int T = TI * TJ;
  v4f part[T];
#pragma unroll
  for (int t = 0; t < T + 2; ++t) {
    if (t < T) {
      const int j = t / TI, i = t % TI;
      if (i == 0 && j + 1 < TJ) bf[(j + 1) & 1] = read_frag_block(b_lo, b_hi, j + 1);
      part[t] = mfma_fp8_16x16x128<C::FMT_B, C::FMT_A>(bf[j & 1], af[i]);   // B first
    }
    // keep the promotion behind this step's MFMA: moved ahead of it, it would read a
    // partial whose MFMA was issued just one MFMA earlier and stall for its latency
    __builtin_amdgcn_sched_barrier(0);
    if (t >= 2) {
      const int u = t - 2;
      const int j = u / TI, i = u % TI;
      const float sc = C::ONE_NB ? s_i[i] : sa[i] * sb[j];
      acc[i][j] = __builtin_elementwise_fma(part[u], (v4f){sc, sc, sc, sc}, acc[i][j]);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// One K-block step: start the copy of a later block into `next`, then multiply the block
// staged in `cur`.  The two stage pointers are restrict-qualified so that the compiler
// knows the reads of `cur` cannot see the copy into `next` and does not wait for it;
// every copy and every read of the K loop goes through this one call site (the
// prologue too), so they all carry the same pair of alias scopes.
template <class C>
__device__ __forceinline__ void kb_step(uint8_t* __restrict__ next, const uint8_t* __restrict__ cur,
                                        const TileCtx& cn, bool issue, int kb_next,
                                        const TileCtx& cc, bool compute,
                                        v4f (&acc)[C::TI][C::TJ]) {
  if (issue) issue_stage<C>(next, cn, kb_next);
  if (compute) compute_stage<C>(cur, cc, acc);
}

// bf16 (round-to-nearest-even) store of one wave's accumulator sub-tiles; rows at or past
// `rows` and columns at or past N are not written.
template <class C>
__device__ __forceinline__ void store_tile_bf16(const v4f (&acc)[C::TI][C::TJ], uint16_t* C_out,
                                                int N, int row0, int rows, int n0, int wm, int wn,
                                                int q, int l16) {
#pragma unroll
  for (int i = 0; i < C::TI; ++i) {
    const int ml = wm * C::WM + 16 * i + l16;
    if (ml >= rows) continue;
    uint16_t* crow = C_out + (size_t)(row0 + ml) * N;
#pragma unroll
    for (int j = 0; j < C::TJ; ++j) {
      const int n = n0 + wn * C::WN + 16 * j + 4 * q;
      const v4f v = acc[i][j];
      if (((N & 3) == 0) && n + 3 < N) {
        const uint32_t lo = bf16x2_rne(v[0], v[1]);
        const uint32_t hi = bf16x2_rne(v[2], v[3]);
        *(uint2*)(crow + n) = make_uint2(lo, hi);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (n + e < N) crow[n + e] = bf16_rne(v[e]);
      }
    }
  }
}

// ------------------------------------------------------------------------------------
// The tiled kernel's epilogue.
// Offset past every tile's output range: a buffer store there is dropped.
constexpr int kPastTile = 0x7FFFFF00;

// The finished tile an epilogue writes.
struct TileOut {
  int a_row0;        // global row of the tile's first row
  int rows;          // rows that exist
  int n0;
  int g;             // contiguous: the group whose rows are written
  int lead0, lead1;  // contiguous: group index of each 128-row block's first row
};

// The epilogue stores from registers: no LDS and no barrier.  Lane (l16, q) of
// a wave holds columns 4q .. 4q+3 of row l16 of every 16x16 fragment.  For fragments j
// and j+1, one v_permlane16_swap per packed bf16 word exchanges the odd 16-lane groups of
// fragment j with the even ones of fragment j+1, after which lane (l16, q) holds the 8
// consecutive columns 16(j + (q & 1)) + 8(q >> 1) .. +7 of its row: one 16-byte store, a
// store instruction covering 16 rows x 64 bytes.  An odd last fragment is stored 8 bytes
// per lane.  Fast form (N a multiple of 8): a fixed count of buffer stores per wave
// (direct_stores), chunks outside the tile's rows or columns dropped by an offset
// past the buffer's range; otherwise element-wise stores and a full wait at the end.
// Contiguous form: a row is stored only if it and its 128-row block's first row name the
// tile's group; the rows' group indices come from the LDS slot the tile's first K block
// filled (one 4-byte read per lane and fragment row).
template <class C>
constexpr int direct_stores() {
  return C::TI * ((C::TJ + 1) / 2);
}

template <int KIND, class C>
__device__ __forceinline__ bool store_tile_direct(const v4f (&acc)[C::TI][C::TJ],
                                                  const GemmArgs& p, const TileOut& o, int wm,
                                                  int wn, int lane, const int32_t* gl) {
  const int N = p.N;
  const bool fast = (N & 7) == 0 && (long)C::BM * N * 2 < (long)kPastTile;
  int ln = lane;
  asm volatile("" : "+v"(ln));           // lane terms computed here, not kept live
  const int l16 = ln & 15, q = ln >> 4;
  const int row_w = C::WM * wm + l16;    // this lane's row in the tile, first fragment row
  const int col_w = o.n0 + C::WN * wn;   // the wave's first column
  if (fast) {
    const __amdgpu_buffer_rsrc_t rc = buffer_over(p.C + (size_t)o.a_row0 * N, o.rows * N * 2);
    const int col_pair = col_w + 16 * (q & 1) + 8 * (q >> 1);   // + 16 j for pair (j, j+1)
    const int col_one = col_w + 4 * q;                         // + 16 j, odd last fragment
#pragma unroll
    for (int i = 0; i < C::TI; ++i) {
      const int r = row_w + 16 * i;
      bool row_ok = r < o.rows;
      if (KIND == kContiguous) {
        // a row is written if it and its 128-row block's first row name the group (the
        // rows' group indices were copied into LDS with the tile's first K block)
        const int lead = r < kAlignM ? o.lead0 : o.lead1;
        row_ok = row_ok && lead == o.g && gl[min(r, C::BM - 1)] == o.g;
      }
      const int row_off = r * N;
#pragma unroll
      for (int j = 0; j + 1 < C::TJ; j += 2) {
        const v4f a = acc[i][j], b = acc[i][j + 1];
        const uint32_t a0 = bf16x2_rne(a[0], a[1]), a1 = bf16x2_rne(a[2], a[3]);
        const uint32_t b0 = bf16x2_rne(b[0], b[1]), b1 = bf16x2_rne(b[2], b[3]);
        const auto s0 = __builtin_amdgcn_permlane16_swap(a0, b0, false, false);
        const auto s1 = __builtin_amdgcn_permlane16_swap(a1, b1, false, false);
        const v4i v = {(int)s0[0], (int)s1[0], (int)s0[1], (int)s1[1]};
        const int col = col_pair + 16 * j;
        __builtin_amdgcn_raw_buffer_store_b128(v, rc,
                                               row_ok && col < N ? (row_off + col) * 2 : kPastTile,
                                               0, 0);
      }
      if constexpr (C::TJ % 2 == 1) {
        const v4f a = acc[i][C::TJ - 1];
        typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
        const u32x2 v = {bf16x2_rne(a[0], a[1]), bf16x2_rne(a[2], a[3])};
        const int col = col_one + 16 * (C::TJ - 1);
        __builtin_amdgcn_raw_buffer_store_b64(v, rc,
                                              row_ok && col < N ? (row_off + col) * 2 : kPastTile,
                                              0, 0);
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < C::TI; ++i) {
      const int r = row_w + 16 * i;
      if (r >= o.rows) continue;
      if (KIND == kContiguous) {
        const int lead = r < kAlignM ? o.lead0 : o.lead1;
        if (lead != o.g || gl[r] != o.g) continue;
      }
      uint16_t* crow = p.C + (size_t)(o.a_row0 + r) * N;
#pragma unroll
      for (int j = 0; j < C::TJ; ++j) {
        const int n = col_w + 16 * j + 4 * q;
        const v4f v = acc[i][j];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (n + e < N) crow[n + e] = bf16_rne(v[e]);
      }
    }
    wait_vmcnt<0>();
  }
  return fast;
}

// A workgroup's work items: items slot, slot + G, ... of the work list that have rows
// to compute.  The list is the tiles in raster order; the contiguous form runs a tile once
// per group present in it (pass 0 and 1).
struct Work {
  int t;
  int pass;
  TileRef tr;
};

// Where the contiguous form's second passes go.  Run right after their first pass, by
// the same workgroup, they pile on the few workgroups that drew a tile straddling two
// groups (the random-size workload: 8 tiles for most workgroups, 9 or 10 for some).
// Instead, when it pays and is cheap to set up, the second passes are appended to the
// work list (pass-0 tiles first, then the second passes, row tile by row tile), where the
// striding hands them to the workgroups that drew one tile fewer.  Each wave counts the
// straddling row tiles with a vector scan of the group indices at kernel start (nothing
// is in flight then); taking an appended item (at most kMaxAppended per workgroup) scans
// again for its row tile.
constexpr int kMaxAppended = 4;
constexpr int kMaxScanRowTiles = 4096;

// Does row tile r hold two 128-row blocks led by two different valid groups?
template <class C>
__device__ __forceinline__ bool straddles(const GemmArgs& p, int r) {
  const int m0 = r * C::BM;
  if (r >= p.tiles_m || m0 + kAlignM >= p.rows) return false;
  const int l0 = p.group_idx[m0], l1 = p.group_idx[m0 + kAlignM];
  return l0 >= 0 && l0 < p.G && l1 >= 0 && l1 < p.G && l0 != l1;
}

// With s < 0: the number of straddling row tiles; else the s-th of them.
template <class C>
__device__ __forceinline__ int straddle_scan(const GemmArgs& p, int s, int lane) {
  int count = 0;
  for (int r0 = 0; r0 < p.tiles_m; r0 += 64) {
    const bool st = straddles<C>(p, r0 + lane);
    const uint64_t m = __builtin_amdgcn_ballot_w64(st);
    const int n = (int)__builtin_popcountll(m);
    if (s >= count && s < count + n) {
      const int below = (int)__builtin_amdgcn_mbcnt_hi((unsigned)(m >> 32),
                                                      __builtin_amdgcn_mbcnt_lo((unsigned)m, 0));
      const uint64_t hit = __builtin_amdgcn_ballot_w64(st && below == s - count);
      return r0 + (int)__builtin_ctzll(hit);
    }
    count += n;
  }
  return s < 0 ? count : 0;
}

// The work list's length: the tiles, plus the appended second passes when there are
// some and at most kMaxAppended per workgroup (else each runs after its first pass).
template <int KIND, class C>
__device__ __forceinline__ int work_total(const GemmArgs& p, int G, int lane) {
  if (KIND != kContiguous || C::BM <= kAlignM || p.tiles_m > kMaxScanRowTiles)
    return p.num_tiles;
  const long extra = (long)straddle_scan<C>(p, -1, lane) * p.tiles_n;
  return extra > (long)kMaxAppended * G ? p.num_tiles : p.num_tiles + (int)extra;
}

// The second pass of row tile rt, column tile tn (its tile straddles two groups).
template <class C>
__device__ __forceinline__ TileRef second_pass(const GemmArgs& p, int rt, int tn) {
  TileRef r;
  r.ok = 1;
  r.g2 = -1;
  r.m0 = rt * C::BM;
  r.n0 = tn * C::BN;
  r.row_base = 0;
  r.rows = min(C::BM, p.rows - r.m0);
  r.lead0 = load_uniform(p.group_idx, r.m0);
  r.lead1 = load_uniform(p.group_idx, r.m0 + kAlignM);
  r.g = uniform(r.lead1);
  return r;
}

// APP: the second passes are appended (the list is `total` > num_tiles items long).
template <int KIND, class C, bool APP>
__device__ __forceinline__ void next_work(const GemmArgs& p, Work& w, int G, int total,
                                          int lane) {
  if (KIND == kContiguous && !APP && w.pass == 0 && w.tr.g2 >= 0) {
    w.pass = 1;
    return;
  }
  w.pass = 0;
  for (w.t += G; w.t < total; w.t += G) {
    if (APP && w.t >= p.num_tiles) {
      const int e = w.t - p.num_tiles;
      w.tr = second_pass<C>(p, uniform(straddle_scan<C>(p, e / p.tiles_n, lane)),
                            e - (e / p.tiles_n) * p.tiles_n);
      return;
    }
    w.tr = locate_tile<KIND, C>(p, w.t);
    if (APP) w.tr.g2 = -1;   // its second pass comes later
    if (w.tr.ok) return;
  }
}

__device__ __forceinline__ void work_ctx(TileCtx& c, const GemmArgs& p, const Work& w) {
  const int g = w.pass == 0 ? w.tr.g : w.tr.g2;
  c.Bg = p.B + (size_t)g * p.N * p.K;
  c.sBg = p.sB + (size_t)g * p.nnb * p.nkb;
  c.a_row0 = w.tr.row_base + w.tr.m0;
  c.rows = w.tr.rows;
  c.n0 = w.tr.n0;
  c.nb_first = w.tr.n0 / kBlockK;
}

// The tiled kernel's walk over a workgroup's items.  Every LDS access goes through one
// of two restrict-qualified views of the stage buffer: `cp` for the copies, `rd` for the
// math and the epilogue.  At any time the two touch different stages (the waits and
// barriers order their reuse), and the restrict scopes let the compiler see that a read
// of a stage does not depend on the copies in flight into the others.
template <int KIND, class C, bool APP>
__device__ __forceinline__ void tile_walk(uint8_t* __restrict__ cp, uint8_t* __restrict__ rd,
                                         const GemmArgs& p, TileCtx c, int G, int slot,
                                         int nwork) {
  constexpr int TI = C::TI, TJ = C::TJ;
  constexpr int STAGES = C::STAGES;
  constexpr int NST = direct_stores<C>();   // epilogue stores per wave
  static_assert((STAGES - 2) * (C::PER_STAGE + 1) + 1 + (STAGES - 1) * NST < 64, "vmcnt range");
  // copy-only waves: they store nothing, so their waits never count epilogue stores
  constexpr bool SPEC = C::XW > 0;
  const int nkb = p.nkb;
  const int wave = c.wave;
  const int cw = c.cw;
  const bool computes = !SPEC || wave < C::W;
  constexpr bool GI = KIND == kContiguous;

  // w: the item being multiplied; wx: the next one, whose first K blocks are copied
  // during w's last steps (when every item has at least STAGES-1 K blocks; otherwise
  // each item fills and drains its own pipeline)
  Work w = {slot - G, 1, {}};
  w.tr.g2 = -1;
  next_work<KIND, C, APP>(p, w, G, nwork, c.lane);
  if (w.t >= nwork) return;
  work_ctx(c, p, w);
  Work wx = w;
  next_work<KIND, C, APP>(p, wx, G, nwork, c.lane);
  TileCtx cx = c;
  cx.gslot = c.gslot ^ 1;
  if (wx.t < nwork) work_ctx(cx, p, wx);
  const bool cross = nkb >= STAGES - 1;

  v4f acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) acc[i][j] = (v4f){0.f, 0.f, 0.f, 0.f};

  // Step kb of an item waits for its K block, starts the copy of the block STAGES-1
  // steps later (in this item or the next) and multiplies.  `stored`: the previous
  // item's epilogue used the fast form; its stores were issued after the copies of this
  // item's first STAGES-1 blocks, so those steps' waits count them.
  bool fill = true, stored = false;
  int sn = 0, sc = 0;
  for (;;) {
    const bool more = cross && wx.t < nwork;
    const int epi_n = stored && !SPEC ? 1 : 0;
    if (fill) {
      for (int f = 0; f < STAGES - 1 && f < nkb; ++f) {
        issue_stage<C, true, GI>(cp + sn * C::STAGE_BYTES, c, f, cp, p.group_idx);
        sn = sn + 1 == STAGES ? 0 : sn + 1;
      }
    }
    int kb = 0;
    // copies of this item's later blocks
    for (; kb + STAGES - 1 < nkb; ++kb) {
      wait_copies_epi<C, NST>(cw, STAGES - 2, kb <= STAGES - 2 ? epi_n : 0);
      stage_barrier();
      issue_stage<C, true, GI>(cp + sn * C::STAGE_BYTES, c, kb + STAGES - 1, cp, p.group_idx);
      sn = sn + 1 == STAGES ? 0 : sn + 1;
      if (computes) compute_stage<C>(rd + sc * C::STAGE_BYTES, c, acc);
      sc = sc + 1 == STAGES ? 0 : sc + 1;
    }
    // the last STAGES-1 steps: copies of the next item's first blocks, then the epilogue
    bool fast = false;
    for (; kb < nkb; ++kb) {
      wait_copies_epi<C, NST>(cw, more ? STAGES - 2 : min(STAGES - 2, nkb - 1 - kb),
                              kb <= STAGES - 2 ? epi_n : 0);
      stage_barrier();
      if (more) {
        issue_stage<C, true, GI>(cp + sn * C::STAGE_BYTES, cx, kb + STAGES - 1 - nkb, cp,
                                 p.group_idx);
        sn = sn + 1 == STAGES ? 0 : sn + 1;
      }
      if (computes) compute_stage<C>(rd + sc * C::STAGE_BYTES, c, acc);
      if (kb == nkb - 1 && computes) {
        TileOut o;
        o.a_row0 = c.a_row0;
        o.rows = c.rows;
        o.n0 = c.n0;
        o.g = w.pass == 0 ? w.tr.g : w.tr.g2;
        o.lead0 = w.tr.lead0;
        o.lead1 = w.tr.lead1;
        fast = store_tile_direct<KIND, C>(acc, p, o, c.wm, c.wn, c.lane,
                                          (const int32_t*)(rd + C::GI_OFF + c.gslot * (C::BM * 4)));
      }
      sc = sc + 1 == STAGES ? 0 : sc + 1;
    }
    if (wx.t >= nwork) break;
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < TJ; ++j) acc[i][j] = (v4f){0.f, 0.f, 0.f, 0.f};
    stored = fast && cross;
    fill = !cross;
    w = wx;
    c = cx;
    cx.gslot = c.gslot ^ 1;
    next_work<KIND, C, APP>(p, wx, G, nwork, c.lane);
    if (wx.t < nwork) work_ctx(cx, p, wx);
  }
}

// ------------------------------------------------------------------------------------
// The tiled kernel.  Each workgroup walks its work items (persistent: blockIdx strides
// over the tile list) with one copy pipeline through all of them: the copies of the next
// item's first K blocks are in flight while the current item finishes and stores its
// tile, and the epilogue's stores are counted in the waits instead of being drained.
template <int KIND, class C>
__global__ void __launch_bounds__(C::NT)
gemm_fp8_kernel(GemmArgs p) {
  // The kernel's only LDS variable: a second one would make the compiler tag LDS
  // accesses with per-variable alias scopes, dropping the restrict scopes that keep it
  // from waiting on in-flight stage copies.
  __shared__ __attribute__((aligned(1024))) uint8_t smem[C::LDS_BYTES];

  const int tid = threadIdx.x;
  TileCtx c;
  c.A = p.A;
  c.sA = p.sA;
  c.K = p.K;
  c.nkb = p.nkb;
  c.nnb = p.nnb;
  c.N = p.N;
  c.lane = tid & 63;
  c.wave = uniform(tid >> 6);
  c.cw = c.wave - C::CW0;
  c.gslot = 0;
  c.wm = c.wave / C::WAVES_N;
  c.wn = c.wave - c.wm * C::WAVES_N;
  c.q = c.lane >> 4;
  c.l16 = c.lane & 15;

  // XCD-aware order: workgroups are dispatched round-robin over the 8 XCDs, so give
  // each XCD a contiguous run of work items (neighbouring tiles share its L2).
  const int G = gridDim.x;
  const int xcd_runs = (G % 8 == 0) ? 8 : 1;
  const int slot = (blockIdx.x % xcd_runs) * (G / xcd_runs) + blockIdx.x / xcd_runs;
  // two compiled walks: one that takes appended second passes, one with none of that
  // code on the path of the (usual) lists without them
  const int nwork = work_total<KIND, C>(p, G, c.lane);
  if constexpr (KIND == kContiguous) {
    if (nwork > p.num_tiles) {
      tile_walk<KIND, C, true>(smem, smem, p, c, G, slot, nwork);
      return;
    }
  }
  tile_walk<KIND, C, false>(smem, smem, p, c, G, slot, nwork);
}

// ------------------------------------------------------------------------------------
// Stream-K kernel for short, wide problems (dense, all rows in one tile: the decode
// shapes).  The (column tile, K block) iterations, tile-major, are split evenly over the
// persistent grid, so every CU streams the same share of B whatever the shape, and one
// load pipeline runs through a workgroup's whole range, across tile boundaries.
// A tile whose K blocks all fall in one workgroup's range is stored as bf16 directly.
// A tile shared by n workgroups (its contributors, consecutive in workgroup order) is
// reduced deterministically with no waiting: each contributor stores its fp32 partial in
// fragment order (one contiguous 1 KB block per 16x16 sub-tile) with device-coherent
// (sc1) stores and, once they are complete, adds one to the tile's arrival counter (a
// device-scope atomic); the contributor that finds n-1 there is the last, resets the
// counter to zero and sums the n partials in workgroup order, then stores bf16.  No
// workgroup ever waits for another, so the result does not depend on which workgroups
// run at the same time.  A workgroup holds at most two shared tiles: the first and the
// last of its range.
// Where the stream-K iterations of the masked form live.  Lane l of every wave holds
// group l's row tiles under its masked_m (clamped to [0, cap]) and, scanned over the
// lanes, the first tile of group l + 1 (the groups' tiles are row-major: all column tiles
// of a group's first row tile, then its second row tile, ...).  At most 64 groups.
struct MaskedPlan {
  int mm;          // this lane's group: rows under masked_m
  int rt;          // its row tiles
  int incl;        // tiles of groups 0 .. lane
  int total;       // tiles of all groups
};

template <class C>
__device__ __forceinline__ MaskedPlan masked_plan(const GemmArgs& p, int lane) {
  MaskedPlan m;
  int v = lane < p.G ? p.masked_m[lane] : 0;
  v = v < 0 ? 0 : (v > p.rows ? p.rows : v);
  m.mm = v;
  m.rt = (v + C::BM - 1) / C::BM;
  int incl = m.rt * p.tiles_n;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int u = __shfl_up(incl, off, 64);
    if (lane >= off) incl += u;
  }
  m.incl = incl;
  m.total = __builtin_amdgcn_readlane(incl, 63);
  return m;
}

// A position in the masked form's tile sequence: group g, row tile r, column tile n.
struct MaskedCursor {
  int g, r, n;
};

// The cursor of tile t (t < total): its group is the number of groups whose tiles all
// come before t.
template <class C>
__device__ __forceinline__ MaskedCursor masked_seek(const MaskedPlan& m, int tiles_n, int t) {
  MaskedCursor c;
  c.g = (int)__builtin_popcountll(__builtin_amdgcn_ballot_w64(m.incl <= t));
  const int first = __builtin_amdgcn_readlane(m.incl, c.g) -
                    __builtin_amdgcn_readlane(m.rt, c.g) * tiles_n;
  const int o = t - first;
  c.r = o / tiles_n;
  c.n = o - c.r * tiles_n;
  return c;
}

// The next tile after c (only called while there is one).
template <class C>
__device__ __forceinline__ void masked_next(const MaskedPlan& m, int tiles_n, MaskedCursor& c) {
  if (++c.n < tiles_n) return;
  c.n = 0;
  if (++c.r < __builtin_amdgcn_readlane(m.rt, c.g)) return;
  c.r = 0;
  // the next group with at least one row tile
  const uint64_t later = __builtin_amdgcn_ballot_w64(m.rt > 0) & ~((2ull << c.g) - 1);
  c.g = later ? (int)__builtin_ctzll(later) : 64;
}

// Tile fields of the copy / math context for cursor c.
template <class C>
__device__ __forceinline__ void masked_tile(const GemmArgs& p, const MaskedPlan& m,
                                            const MaskedCursor& c, TileCtx& x) {
  const int g = c.g < 64 ? c.g : 0;
  const int mm = __builtin_amdgcn_readlane(m.mm, g);
  x.a_row0 = g * p.rows + c.r * C::BM;
  x.rows = min(C::BM, mm - c.r * C::BM);
  x.Bg = p.B + (size_t)g * p.N * p.K;
  x.sBg = p.sB + (size_t)g * p.nnb * p.nkb;
  x.n0 = c.n * C::BN;
  x.nb_first = x.n0 / kBlockK;
}

// Reduction of a shared stream-K tile, spread over its contributors, none of which
// depends on another making progress.  The tile's fragments are split into P parts
// (fragment f of wave w is in part (w*TI*TJ + f) % P, P = min(reducers, fragments, 32),
// the reducers being the contributors whose range ends inside the tile), and
// contributor c < P reduces part c: it polls the contributors' slots for the part
// (their stores are the signal: a written word is never zero), boundedly, sums them in
// workgroup order, stores bf16 and zeroes the slots.  Every contributor then counts its
// arrival at the tile, with the bit of the part it completed, in one 64-bit atomic add on
// the tile's record (arrivals in the high word, completed parts in the low).  The last to
// arrive knows that every partial is stored and that nobody touches the record again:
// it reduces the parts nobody completed (a contributor whose wait ran out leaves its part
// to it) and clears the record.  Each part is summed in the same order whoever reduces
// it.  All of this runs per wave: the fragments of wave w of every contributor form
// their own reduction with their own record, so the waves of a workgroup never wait for
// one another (a wave with no fragment in its part has completed it at once).
//
// This wave's fragments of the parts in `mask`, FCH fragments at a time, their partials
// from CB contributors per batch of loads in flight (polled until every word is written,
// at most `polls` times; slots past the buffer or of no fragment read zeros without
// touching memory and count as written), summed in workgroup order and stored as bf16
// (rows at or past `rows`, columns at or past N are not written).  With ZERO the slots
// are zeroed instead.  Returns false if a poll ran out (nothing is zeroed then).
template <class C, bool ZERO>
__device__ __forceinline__ bool reduce_parts(int mask, int P, int n, int g_first, int first_slot,
                                             __amdgpu_buffer_rsrc_t part_rsrc,
                                             const GemmArgs& p, int row0, int rows, int n0,
                                             int wave, int wm, int wn, int lane, int polls) {
  constexpr int NF = C::TI * C::TJ;
  constexpr int FCH = NF < 2 ? NF : 2;         // 16 loads in flight per poll
  constexpr int CB = 8;
  constexpr int WAVE_SLOT = NF * 64 * 4;                   // floats of one wave's partial
  constexpr int kPastBuffer = 0x7FFFFF00;
  const int l16 = lane & 15, q = lane >> 4;
  int f = 0;
#pragma unroll 1
  for (;;) {
    int fl[FCH];                                          // the chunk's fragments, or -1
#pragma unroll
    for (int k = 0; k < FCH; ++k) {
      while (f < NF && !((mask >> ((wave * NF + f) % P)) & 1)) ++f;
      fl[k] = f < NF ? f : -1;
      f = f < NF ? f + 1 : f;
    }
    if (fl[0] < 0) break;
    v4f sum[FCH];
#pragma unroll
    for (int k = 0; k < FCH; ++k) sum[k] = (v4f){0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
    for (int c0 = 0; c0 < n; c0 += CB) {
      // a contributor's slot for this tile: 0 if its range starts inside the tile (the
      // tile is its first), else 1 (the tile is its last): only the first contributor's
      // range can start before the tile
      int off[CB][FCH];
#pragma unroll
      for (int u = 0; u < CB; ++u) {
        const int gg = g_first + c0 + u;
        const int slot = c0 + u == 0 ? first_slot : 0;
        const int base = ((gg * 2 + slot) * C::W + wave) * WAVE_SLOT * 4;
#pragma unroll
        for (int k = 0; k < FCH; ++k) {
          off[u][k] = c0 + u < n && fl[k] >= 0 ? base + (fl[k] * 64 + lane) * 16 : kPastBuffer;
        }
      }
      if constexpr (ZERO) {
#pragma unroll
        for (int u = 0; u < CB; ++u)
#pragma unroll
          for (int k = 0; k < FCH; ++k)
            if (off[u][k] != kPastBuffer)
              __builtin_amdgcn_raw_buffer_store_b128((v4i){0, 0, 0, 0}, part_rsrc, off[u][k], 0,
                                                     16 /* sc1 */);
        continue;
      }
      // slots of no contributor or fragment read zeros: they count as written
      unsigned dead[CB][FCH];
#pragma unroll
      for (int u = 0; u < CB; ++u)
#pragma unroll
        for (int k = 0; k < FCH; ++k) dead[u][k] = off[u][k] == kPastBuffer ? ~0u : 0u;
      v4i raw[CB][FCH];
      bool ready = false;
#pragma unroll 1
      for (int poll = 0; poll < polls && !ready; ++poll) {
        if (poll > 0) __builtin_amdgcn_s_sleep(2);
#pragma unroll
        for (int u = 0; u < CB; ++u)
#pragma unroll
          for (int k = 0; k < FCH; ++k)
            raw[u][k] = __builtin_amdgcn_raw_buffer_load_b128(part_rsrc, off[u][k], 0, kPollAux);
        // the smallest word over all loads (unsigned; a dead slot counts as all ones) is
        // zero iff some slot is not written yet: min/max arithmetic, one compare per poll
        unsigned least = ~0u;
#pragma unroll
        for (int u = 0; u < CB; ++u)
#pragma unroll
          for (int k = 0; k < FCH; ++k) {
            const v4i r = raw[u][k];
            const unsigned m = min(min((unsigned)r.x, (unsigned)r.y), min((unsigned)r.z, (unsigned)r.w));
            least = min(least, max(m, dead[u][k]));
          }
        ready = __builtin_amdgcn_ballot_w64(least == 0) == 0;
      }
      if (!ready) return false;
#pragma unroll
      for (int u = 0; u < CB; ++u) {
        if (c0 + u >= n) break;
#pragma unroll
        for (int k = 0; k < FCH; ++k) sum[k] += decode_partial(raw[u][k]);
      }
    }
    if constexpr (!ZERO) {
#pragma unroll
      for (int k = 0; k < FCH; ++k) {
        if (fl[k] < 0) continue;
        const int fi = fl[k] / C::TJ, fj = fl[k] - fi * C::TJ;
        const int row = wm * C::WM + 16 * fi + l16;
        const int col = n0 + wn * C::WN + 16 * fj + 4 * q;
        if (row >= rows) continue;
        uint16_t* dst = p.C + (size_t)(row0 + row) * p.N;
        const v4f v = sum[k];
        if (((p.N & 3) == 0) && col + 3 < p.N) {
          *(uint2*)(dst + col) = make_uint2(bf16x2_rne(v[0], v[1]), bf16x2_rne(v[2], v[3]));
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (col + e < p.N) dst[col + e] = bf16_rne(v[e]);
        }
      }
    }
  }
  return true;
}

// n / d for n >= 0, d > 0: a 32-bit unsigned division when both fit (every realistic
// launch: a 64-bit division is a long emulated sequence), else a 64-bit one.
__device__ __forceinline__ long udiv(long n, long d) {
  if ((unsigned long long)n <= 0xFFFFFFFFull && (unsigned long long)d <= 0xFFFFFFFFull)
    return (long)((unsigned)n / (unsigned)d);
  return (long)((unsigned long long)n / (unsigned long long)d);
}

template <class C>
__device__ __forceinline__ long stream_start(long g, long W, long G) { return udiv(g * W, G); }

template <int KIND, class C>
__global__ void __launch_bounds__(C::NT)
gemm_fp8_stream_kernel(GemmArgs p) {
  constexpr int TI = C::TI, TJ = C::TJ, STAGES = C::STAGES;
  constexpr int FRAG_FLOATS = 64 * 4;                        // one 16x16 fp32 sub-tile
  constexpr int WAVE_SLOT = TI * TJ * FRAG_FLOATS;           // one wave's partial
  static_assert(C::W <= 8, "the workspace holds one arrival record per wave, 8 per tile");
  static_assert(C::XW == 0, "every wave of the stream kernel computes");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[STAGES * C::STAGE_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int wm = wave / C::WAVES_N;
  const int wn = wave - wm * C::WAVES_N;
  const int q = lane >> 4;
  const int l16 = lane & 15;
  const int nkb = p.nkb;
  // masked form: the tiles under masked_m, counted on the device (the grid is sized for
  // the capacity, so some workgroups may get no iterations at all)
  MaskedPlan mp;
  int num_tiles = p.num_tiles;
  if (KIND == kMasked) {
    mp = masked_plan<C>(p, lane);
    num_tiles = mp.total;
  }
  const long W = (long)num_tiles * nkb;
  // the iterations are split over the first min(grid, W) workgroups, so that each of them
  // has at least one (the contributor arithmetic of the reduction relies on it); the
  // others have nothing to do
  const long G = W < (long)gridDim.x ? W : (long)gridDim.x;
  const long g = blockIdx.x;
  const long i_begin = g < G ? stream_start<C>(g, W, G) : 0;
  const long i_end = g < G ? stream_start<C>(g + 1, W, G) : 0;
  const int t_first = (int)udiv(i_begin, nkb);

  TileCtx cn, cc;
  cn.A = p.A;
  cn.sA = p.sA;
  cn.Bg = p.B;
  cn.sBg = p.sB;
  cn.K = p.K;
  cn.nkb = nkb;
  cn.nnb = p.nnb;
  cn.N = p.N;
  cn.a_row0 = 0;
  cn.rows = p.rows;
  cn.wave = wave;
  cn.cw = wave;
  cn.lane = lane;
  cn.wm = wm;
  cn.wn = wn;
  cn.q = q;
  cn.l16 = l16;
  cc = cn;

  // partial slots: two per workgroup (the first and the last tile of its range)
  __amdgpu_buffer_rsrc_t part_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      p.partial, (short)0, (int)((size_t)G * 2 * C::W * WAVE_SLOT * 4), 0x00020000);

  v4f acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) acc[i][j] = (v4f){0.f, 0.f, 0.f, 0.f};

  // Iteration bookkeeping with 32-bit counters only (no division in the loop): the copy
  // runs STAGES-1 iterations ahead of the math; relative iteration r lives in stage
  // r % STAGES for both.
  const int n_iter = (int)(i_end - i_begin);
  int tn = t_first, kbn = (int)(i_begin - (long)t_first * nkb), sn = 0;   // next copy
  int tc = tn, kbc = kbn, sc = 0, in_tile = 0;                              // next math
  MaskedCursor mn = {0, 0, 0}, mc = {0, 0, 0};      // masked form: the same two tiles
  if (KIND == kMasked && n_iter > 0) {
    mn = masked_seek<C>(mp, p.tiles_n, t_first);
    mc = mn;
  }
  int shared_tile[2] = {-1, -1};
  int seg_row0[2] = {0, 0}, seg_rows[2] = {0, 0}, seg_n0[2] = {0, 0};  // where they go
  for (int step = 1 - STAGES; step < n_iter; ++step) {
    if (step >= 0) {
      wait_stage_copies<C, STAGES - 2>(wave, min(STAGES - 2, n_iter - 1 - step));
      stage_barrier();
    }
    const bool issue = step + STAGES - 1 < n_iter;
    if (KIND == kMasked) {
      masked_tile<C>(p, mp, mn, cn);
      masked_tile<C>(p, mp, mc, cc);
    } else {
      cn.n0 = tn * C::BN;
      cn.nb_first = cn.n0 / kBlockK;
      cc.n0 = tc * C::BN;
      cc.nb_first = cc.n0 / kBlockK;
    }
    kb_step<C>(smem + sn * C::STAGE_BYTES, smem + sc * C::STAGE_BYTES, cn, issue, kbn, cc,
               step >= 0, acc);
    if (issue) {
      sn = sn + 1 == STAGES ? 0 : sn + 1;
      if (++kbn == nkb) {
        kbn = 0;
        ++tn;
        if (KIND == kMasked && step + STAGES < n_iter) masked_next<C>(mp, p.tiles_n, mn);
      }
    }
    if (step < 0) continue;
    sc = sc + 1 == STAGES ? 0 : sc + 1;
    ++in_tile;
    const bool tile_end = kbc == nkb - 1 || step == n_iter - 1;
    if (++kbc == nkb) kbc = 0;
    if (!tile_end) continue;

    // tile tc ends here for this workgroup
    if (in_tile == nkb) {
      store_tile_bf16<C>(acc, p.C, p.N, cc.a_row0, cc.rows, cc.n0, wm, wn, q, l16);
    } else {
      const int seg = tc == t_first ? 0 : 1;
      shared_tile[seg] = tc;
      seg_row0[seg] = cc.a_row0;
      seg_rows[seg] = cc.rows;
      seg_n0[seg] = cc.n0;
      const int base = (int)(((g * 2 + seg) * C::W + wave) * WAVE_SLOT) * 4;
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j)
          __builtin_amdgcn_raw_buffer_store_b128(encode_partial(acc[i][j]), part_rsrc,
                                                 base + ((i * TJ + j) * 64 + lane) * 16, 0,
                                                 16 /* sc1: device coherent */);
    }
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < TJ; ++j) acc[i][j] = (v4f){0.f, 0.f, 0.f, 0.f};
    ++tc;
    if (KIND == kMasked && step < n_iter - 1) masked_next<C>(mp, p.tiles_n, mc);
    in_tile = 0;
  }

  // ---- hand-off of the shared tiles (see reduce_parts), wave by wave: the waves of a
  // workgroup never wait for one another and touch no LDS here.  Jobs 0 and 1: this
  // wave's own part of the last and the first shared tile; then its arrival at both;
  // jobs 2 and 3: the parts nobody completed, where this wave arrived last.
  if (shared_tile[0] < 0 && shared_tile[1] < 0) return;
  // per shared tile, once: first contributor, contributors, parts, this workgroup's
  // index among the contributors, and the first contributor's slot
  int gfv[2], nv[2], pv[2], cv[2], fsv[2];
#pragma unroll
  for (int sg = 0; sg < 2; ++sg) {
    const long x0 = (long)(shared_tile[sg] < 0 ? 0 : shared_tile[sg]) * nkb, x1 = x0 + nkb - 1;
    const long gf = udiv((x0 + 1) * G + W - 1, W) - 1;
    const long gl = udiv((x1 + 1) * G + W - 1, W) - 1;
    // the parts go to the contributors whose range ends inside the tile: the last
    // contributor's range usually goes on into the next tiles (the tile is its first,
    // stored long before), so it takes a part only when its range ends with the tile
    const int nr = (int)(gl - gf) + (stream_start<C>(gl + 1, W, G) == x1 + 1 ? 1 : 0);
    gfv[sg] = (int)gf;
    nv[sg] = (int)(gl - gf + 1);
    pv[sg] = min(nr, min(C::W * TI * TJ, 32));
    cv[sg] = (int)(g - gf);
    fsv[sg] = stream_start<C>(gf, W, G) < x0 ? 1 : 0;
  }
  bool polled = false;
  int okmask = 0, left0 = 0, left1 = 0;
#pragma unroll 1
  for (int k = 0; k < 4; ++k) {
    if (k == 2) {
      // this wave's partial stores are complete before its arrival is counted: a wave
      // that polled has used loads issued after them (vmcnt retires in issue order); with
      // a zero poll bound nothing was loaded
      if (!polled || p.helper_polls == 0) wait_vmcnt<0>();
      unsigned long long before[2] = {0ull, 0ull};
#pragma unroll
      for (int sg = 0; sg < 2; ++sg) {
        const unsigned long long mine =
            (1ull << 32) | ((okmask >> sg) & 1 ? 1ull << cv[sg] : 0ull);
        if (lane == 0 && shared_tile[sg] >= 0)
          before[sg] = __hip_atomic_fetch_add(
              (unsigned long long*)p.arrivals + gfv[sg] * C::W + wave, mine, __ATOMIC_RELAXED,
              __HIP_MEMORY_SCOPE_AGENT);
      }
#pragma unroll
      for (int sg = 0; sg < 2; ++sg) {
        if (shared_tile[sg] < 0) continue;
        const int hi = __builtin_amdgcn_readlane((int)(before[sg] >> 32), 0);
        const int lo = __builtin_amdgcn_readlane((int)before[sg], 0);
        if (hi == nv[sg] - 1) {                 // the last to arrive
          const int mine_done = (okmask >> sg) & 1 ? 1 << cv[sg] : 0;
          // every part (P can be 32: no 1 << 32 on a 32-bit int)
          const unsigned all = pv[sg] >= 32 ? ~0u : (1u << pv[sg]) - 1u;
          const int left = (int)(all & ~(unsigned)(lo | mine_done));
          if (sg) left1 = left; else left0 = left;
          if (lane == 0)
            __hip_atomic_store((unsigned long long*)p.arrivals + gfv[sg] * C::W + wave, 0ull,
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
    }
    const int sg = (k & 1) ^ 1;              // the last shared tile first
    if ((sg ? shared_tile[1] : shared_tile[0]) < 0) continue;
    const int P = sg ? pv[1] : pv[0], c = sg ? cv[1] : cv[0];
    const int mask = k < 2 ? (c < P ? 1 << c : 0) : (sg ? left1 : left0);
    if (!mask) continue;
    polled = polled || k < 2;
    const int n = sg ? nv[1] : nv[0], gf = sg ? gfv[1] : gfv[0], fs = sg ? fsv[1] : fsv[0];
    const int row0 = sg ? seg_row0[1] : seg_row0[0];
    const int rows = sg ? seg_rows[1] : seg_rows[0];
    const int n0 = sg ? seg_n0[1] : seg_n0[0];
    // an owner polls at most helper_polls times; the last arrival's partials are all
    // stored, so its leftover parts never wait
    if (reduce_parts<C, false>(mask, P, n, gf, fs, part_rsrc, p, row0, rows, n0, wave, wm, wn,
                               lane, k < 2 ? p.helper_polls : kHelperPolls)) {
      reduce_parts<C, true>(mask, P, n, gf, fs, part_rsrc, p, 0, 0, 0, wave, wm, wn, lane, 0);
      if (k < 2) okmask |= 1 << sg;
    }
  }
}

template <int KIND, class C>
void launch_stream(const GemmArgs& a, int grid, hipStream_t stream) {
  hipLaunchKernelGGL((gemm_fp8_stream_kernel<KIND, C>), dim3(grid), dim3(C::NT), 0, stream, a);
}

// persistent stream grid: one workgroup per CU (at most kStreamGrid); dense calls follow
// stream_grid (128x24576x1536 on 192 workgroups shares no tile: 24.5 -> 21.8 us;
// 128x2112x7168 on 231: 14.9 -> 13.1 us); the masked form's tiles are counted on the
// device, so its grid covers the capacity
int grid_stream(const GemmArgs& a, int num_cus) {
  const long g = num_cus < kStreamGrid ? num_cus : kStreamGrid;
  if (a.masked_m) {
    const long work = (long)a.num_tiles * a.nkb;
    return (int)(work < g ? work : g);
  }
  return (int)stream_grid(a.num_tiles, a.nkb, g);
}

template <int KIND, class C>
void launch(const GemmArgs& a, int grid, hipStream_t stream) {
  hipLaunchKernelGGL((gemm_fp8_kernel<KIND, C>), dim3(grid), dim3(C::NT), 0, stream, a);
}

// persistent grid: one workgroup per CU (the LDS budget allows no more), capped by work
int grid_persistent(const GemmArgs& a, int num_cus) {
  return a.num_tiles < num_cus ? a.num_tiles : num_cus;
}

// Tile shapes, each built for the four operand-format pairs (FA, FB).
template <int FA, int FB> using Big = Cfg<256, 256, 4, 2, 2, false, FA, FB, 4>;     // 8 waves, 64x128 each
template <int FA, int FB> using Big224 = Cfg<256, 224, 4, 2, 2, false, FA, FB, 4>;  // non-power-of-two N tile
template <int FA, int FB> using Big160 = Cfg<256, 160, 4, 2, 2, false, FA, FB, 4>;  // for N near 2048
// the contiguous form keeps more per-tile state: its 256x224 tile has no registers to
// spare for the copy waves' doubled copy set, so all of its waves copy.  Its 256x256
// tile prefetches into the L2 two K blocks ahead of the copies (K = 7168: 3-4% faster;
// the dense tiles ran 1-5% slower with it, their L2 hit rate being higher)
template <int FA, int FB> using BigC = Cfg<256, 256, 4, 2, 2, false, FA, FB, 4, 2>;
template <int FA, int FB> using Big224C = Cfg<256, 224, 4, 2, 2, false, FA, FB>;
template <int FA, int FB> using Mid = Cfg<128, 128, 2, 2, 3, false, FA, FB>;     // 4 waves, 64x64 each
// the same with four copy-only waves (register epilogue forms: dense and masked)
template <int FA, int FB> using MidS = Cfg<128, 128, 2, 2, 3, false, FA, FB, 0, 0, 4>;
template <int FA, int FB> using Small = Cfg<64, 128, 1, 4, 4, false, FA, FB>;    // 4 waves, 64x32 each
// stream-K decode instances: 8 waves (a wave's direct-to-LDS copies are issue-bound, so
// a workgroup needs eight of them to draw its share of HBM bandwidth), B non-temporal
template <int FA, int FB> using Str64 = Cfg<64, 128, 2, 4, 5, true, FA, FB>;     // 64 rows x 128 columns
template <int FA, int FB> using Str64n64 = Cfg<64, 64, 2, 4, 8, true, FA, FB>;   // 64 rows x 64 columns
template <int FA, int FB> using Str128 = Cfg<128, 128, 2, 4, 4, true, FA, FB>;   // 128 rows x 128 columns
template <int FA, int FB> using Str128n64 = Cfg<128, 64, 2, 4, 6, true, FA, FB>; // 128 rows x 64 columns
// 4-wave builds of the 128-column tiles (one wave per SIMD; per K block 64 KB of fragment
// reads from LDS instead of 96, 48 instead of 64) for ranges of 16 K blocks or more per
// workgroup: 128x7168x16384 44.0 -> 39.7 us, 64x7168x16384 34.0 -> 33.3 us; on shorter
// ranges they lose 2-7%
template <int FA, int FB> using Str128w4 = Cfg<128, 128, 2, 2, 4, true, FA, FB>;  // 64x64 per wave
template <int FA, int FB> using Str64w4 = Cfg<64, 128, 2, 2, 5, true, FA, FB>;    // 32x64 per wave

}  // namespace

#define DG_INST1(NAME, KIND, C, FA, FB)                                                   \
  Instance { NAME, KIND, C::BM, C::BN, kModeTiled, C::NT, FA, FB, grid_persistent,        \
             launch<KIND, C> }
#define DG_STREAM1(NAME, KIND, C, FA, FB)                                                  \
  Instance { NAME, KIND, C::BM, C::BN, kModeStream, C::NT, FA, FB, grid_stream,           \
             launch_stream<KIND, C> }
#define DG_INST(NAME, KIND, T)                                                             \
  DG_INST1(NAME, KIND, T<0 COMMA 0>, 0, 0), DG_INST1(NAME, KIND, T<1 COMMA 1>, 1, 1),      \
      DG_INST1(NAME, KIND, T<0 COMMA 1>, 0, 1), DG_INST1(NAME, KIND, T<1 COMMA 0>, 1, 0)
#define DG_STREAM(NAME, KIND, T)                                                           \
  DG_STREAM1(NAME, KIND, T<0 COMMA 0>, 0, 0), DG_STREAM1(NAME, KIND, T<1 COMMA 1>, 1, 1),  \
      DG_STREAM1(NAME, KIND, T<0 COMMA 1>, 0, 1), DG_STREAM1(NAME, KIND, T<1 COMMA 0>, 1, 0)
#define COMMA ,

static const Instance kInstances[] = {
    DG_INST("dense_256x256", kDense, Big),
    DG_INST("dense_256x224", kDense, Big224),
    DG_INST("dense_256x160", kDense, Big160),
    DG_INST("dense_128x128", kDense, MidS),
    DG_STREAM("dense_64x128_stream", kDense, Str64),
    DG_STREAM("dense_64x64_stream", kDense, Str64n64),
    DG_STREAM("dense_128x128_stream", kDense, Str128),
    DG_STREAM("dense_128x64_stream", kDense, Str128n64),
    DG_STREAM("dense_128x128_stream_4w", kDense, Str128w4),
    DG_STREAM("dense_64x128_stream_4w", kDense, Str64w4),
    DG_INST("contig_256x256", kContiguous, BigC),
    DG_INST("contig_256x224", kContiguous, Big224C),
    DG_INST("contig_128x128", kContiguous, Mid),
    DG_INST("masked_256x256", kMasked, Big),
    DG_INST("masked_128x128", kMasked, MidS),
    DG_INST("masked_64x128", kMasked, Small),
    DG_STREAM("masked_128x128_stream", kMasked, Str128),
    DG_STREAM("masked_128x64_stream", kMasked, Str128n64),
};

const Instance* instances(int* count) {
  *count = (int)(sizeof(kInstances) / sizeof(kInstances[0]));
  return kInstances;
}

}  // namespace dg
