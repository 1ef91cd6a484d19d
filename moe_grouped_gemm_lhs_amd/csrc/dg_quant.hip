// dg_quant.hip -- fp8 quantisation with block scales for gfx950: the casting step in
// front of the GEMM (turtlesai.it summary, technical paragraph: casting is the user's
// job; the block shapes are the method's fine-grained scaling).
//
// Per block (1x128 along a row, or 128x128): amax = max |x| in fp32; scale = amax /
// FMAX in fp32 (FMAX = 448 for E4M3, 57344 for E5M2; 1 for an all-zero block); each
// code is x / scale (an IEEE fp32 division) rounded to the nearest fp8 value, ties to
// even, saturating at +-FMAX.  Inputs are finite fp32 or bf16.  Memory-bound: every
// load is 16 bytes (4 fp32 or 8 bf16 inputs) and the matching 4 or 8 codes go out in one
// store; each lane keeps several loads in flight; the per-element work is three fp32
// operations for the quotient and the hardware's fp8 conversion.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dg_internal.h"

namespace dg {
namespace {

template <int FMT>
__device__ __forceinline__ float fp8_max() {
  return FMT == kFmtE5M2 ? 57344.0f : 448.0f;
}

// E consecutive inputs as fp32 from one 16-byte load: E = 8 for bf16, 4 for fp32.
template <bool BF16>
struct In {
  static constexpr int E = BF16 ? 8 : 4;
};

// The 16-byte load behind E inputs, and its expansion to fp32.
template <bool BF16>
__device__ __forceinline__ uint4 load_raw(const void* X, int64_t i) {
  return *(const uint4*)((const uint8_t*)X + i * (BF16 ? 2 : 4));
}

template <bool BF16>
__device__ __forceinline__ void expand(const uint4& u, float (&x)[In<BF16>::E]) {
  if (BF16) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      x[2 * k] = __uint_as_float(w[k] << 16);
      x[2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
    }
  } else {
    x[0] = __uint_as_float(u.x);
    x[1] = __uint_as_float(u.y);
    x[2] = __uint_as_float(u.z);
    x[3] = __uint_as_float(u.w);
  }
}

template <int E>
__device__ __forceinline__ float amax_of(const float* x) {
  float m = fabsf(x[0]);
#pragma unroll
  for (int e = 1; e < E; ++e) m = fmaxf(m, fabsf(x[e]));
  return m;
}

// Smallest scale whose quotients take the reciprocal path below.  From 2^-64 up, 1/scale
// is finite and, for every quotient that can round to a non-zero fp8 code (|x/scale| >=
// 2^-18), x >= 2^-82 and y*scale is a multiple of 2^-128, so the residual below is an
// exact fp32 value; smaller quotients give the zero code whatever their last bits.
constexpr float kMinReciprocalScale = 0x1p-64f;

// x / scale rounded to nearest fp32, from a correctly rounded reciprocal r = 1/scale:
// y = x*r is within an ulp of the quotient and the residual x - y*scale is exact (one
// fma), so y + r*residual rounded once is the correctly rounded quotient (Markstein's
// theorem; no overflow: |x| <= amax = scale * FMAX).  The sign comes from x (scale > 0),
// which also keeps the sign of a zero.  Blocks with a scale under kMinReciprocalScale
// (amax below FMAX * 2^-64: tiny and subnormal inputs, where 1/scale overflows or the
// residual underflows) take the IEEE division instead; there a scale that underflowed to
// zero gives +-inf (saturated below) and 0/0 a zero with the sign of x.
// TINY: some lane of the wave holds such a block (decided once per wave by the caller,
// so that the usual case carries no division at all).
template <bool TINY>
__device__ __forceinline__ float div_by_scale(float x, float scale, float r) {
  if (!TINY || scale >= kMinReciprocalScale) {
    const float y = x * r;
    const float e = __builtin_fmaf(-y, scale, x);
    return __builtin_copysignf(__builtin_fmaf(e, r, y), x);
  }
  const float q = x / scale;                      // correctly rounded fp32 division
  return q != q ? __builtin_copysignf(0.0f, x) : q;
}

// Four codes: the quotients saturated to +-FMAX, then converted by the hardware's
// round-to-nearest-even fp8 conversion (OCP E4M3 / E5M2 on gfx950).
template <int FMT, bool TINY>
__device__ __forceinline__ uint32_t pack4(const float* x, float scale, float r) {
  const float m = fp8_max<FMT>();
  float q[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) q[i] = fminf(fmaxf(div_by_scale<TINY>(x[i], scale, r), -m), m);
  int v;
  if (FMT == kFmtE5M2) {
    v = __builtin_amdgcn_cvt_pk_bf8_f32(q[0], q[1], 0, false);
    v = __builtin_amdgcn_cvt_pk_bf8_f32(q[2], q[3], v, true);
  } else {
    v = __builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], 0, false);
    v = __builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], v, true);
  }
  return (uint32_t)v;
}

// E codes of one 16-byte load, stored with one 8- or 4-byte store.
template <int FMT, bool BF16, bool TINY>
__device__ __forceinline__ void store_codes_as(uint8_t* Q, int64_t i, const float* x, float scale,
                                               float r) {
  if (BF16)
    *(uint2*)(Q + i) =
        make_uint2(pack4<FMT, TINY>(x, scale, r), pack4<FMT, TINY>(x + 4, scale, r));
  else
    *(uint32_t*)(Q + i) = pack4<FMT, TINY>(x, scale, r);
}
template <int FMT, bool BF16>
__device__ __forceinline__ void store_codes(uint8_t* Q, int64_t i, const float* x, float scale,
                                            float r) {
  if (__builtin_amdgcn_ballot_w64(scale < kMinReciprocalScale) == 0)
    store_codes_as<FMT, BF16, false>(Q, i, x, scale, r);
  else
    store_codes_as<FMT, BF16, true>(Q, i, x, scale, r);
}

// 1x128 blocks: LPB = 128/E lanes per block (16 for bf16, 32 for fp32), each with one
// 16-byte load; a wave holds 64/LPB blocks side by side and takes U such groups, issuing
// all U loads before it reduces any block, so every lane keeps U loads in flight.  Block
// b is row b / nkb, K block b % nkb, and its scale goes to S[b] (S is rows x nkb).  Loads
// of blocks past the end re-read the last block; their stores are skipped.
template <int FMT, bool BF16>
__global__ void __launch_bounds__(256)
quant_1x128_kernel(const void* X, uint8_t* Q, float* S, int64_t nblk, int nkb, int64_t K) {
  constexpr int E = In<BF16>::E, LPB = kBlockK / E, BPW = 64 / LPB, U = 4;
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int l = lane % LPB;
  int64_t b[U], i[U];
  float x[U][E];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    b[u] = (wave * U + u) * BPW + lane / LPB;
    const int64_t bb = b[u] < nblk ? b[u] : nblk - 1;
    const int64_t r = bb / nkb;
    i[u] = r * K + (bb - r * nkb) * kBlockK + l * E;
    expand<BF16>(load_raw<BF16>(X, i[u]), x[u]);
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    float amax = amax_of<E>(x[u]);
#pragma unroll
    for (int off = LPB / 2; off >= 1; off >>= 1)
      amax = fmaxf(amax, __shfl_xor(amax, off, LPB));
    const float scale = amax == 0.0f ? 1.0f : amax / fp8_max<FMT>();
    const float rcp = 1.0f / scale;      // correctly rounded (unused below 2^-64)
    if (b[u] < nblk) {
      store_codes<FMT, BF16>(Q, i[u], x[u], scale, rcp);
      if (l == 0) S[b[u]] = scale;
    }
  }
}

// 128x128 blocks: a persistent grid of a few workgroups per CU strides over the blocks,
// each workgroup loading its next block while it quantises the current one, so that
// every CU gets the same number of blocks (no partly filled last wave of workgroups) and
// the loads of consecutive blocks overlap.  Thread t takes the E columns starting at
// E(t % (128/E)) of rows t / (128/E) + R j, j = 0 .. 128/R - 1, where R = 256 / (128/E)
// rows are covered per pass (rows past the matrix read as zero and are not stored).  The
// block maximum goes through LDS, double buffered so that one barrier per block suffices.
template <int FMT, bool BF16>
__global__ void __launch_bounds__(256)
quant_128x128_kernel(const void* X, uint8_t* Q, float* S, int64_t rows, int nkb, int64_t K,
                     int64_t nblk) {
  constexpr int E = In<BF16>::E, TPR = kBlockK / E, R = 256 / TPR, J = kBlockK / R;
  __shared__ float wave_max[2][4];
  const int t = threadIdx.x;
  const int64_t G = gridDim.x;
  const int lr = t / TPR;                                  // row inside a pass
  const int lc = (t % TPR) * E;                            // column inside the block
  auto load_block = [&](int64_t b, uint4 (&raw)[J]) {
    const int64_t rb = b / nkb;
    const int64_t col = (b - rb * nkb) * kBlockK + lc, row0 = rb * kBlockK + lr;
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int64_t r = row0 + R * j;
      raw[j] = r < rows ? load_raw<BF16>(X, r * K + col) : make_uint4(0, 0, 0, 0);
    }
  };
  int64_t b = blockIdx.x;
  uint4 cur[J];
  load_block(b, cur);
  for (int k = 0; b < nblk; ++k, b += G) {
    uint4 nxt[J];
    const bool more = b + G < nblk;
    if (more) load_block(b + G, nxt);
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < J; ++j) {
      float x[E];
      expand<BF16>(cur[j], x);
      amax = fmaxf(amax, amax_of<E>(x));
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
    if ((t & 63) == 0) wave_max[k & 1][t >> 6] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(wave_max[k & 1][0], wave_max[k & 1][1]),
                 fmaxf(wave_max[k & 1][2], wave_max[k & 1][3]));
    const float scale = amax == 0.0f ? 1.0f : amax / fp8_max<FMT>();
    const float rcp = 1.0f / scale;      // correctly rounded (unused below 2^-64)
    if (t == 0) S[b] = scale;
    const int64_t rb = b / nkb;
    const int64_t col = (b - rb * nkb) * kBlockK + lc, row0 = rb * kBlockK + lr;
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int64_t r = row0 + R * j;
      if (r < rows) {
        float x[E];
        expand<BF16>(cur[j], x);
        store_codes<FMT, BF16>(Q, r * K + col, x, scale, rcp);
      }
    }
    if (more) {
#pragma unroll
      for (int j = 0; j < J; ++j) cur[j] = nxt[j];
    }
  }
}

// Persistent grid: `per_cu` workgroups per CU at most, each taking the same number of
// blocks (the grid shrinks so that the blocks divide as evenly as they can).
int64_t persistent_grid(int64_t pieces, int num_cus, int per_cu) {
  const int64_t slots = (int64_t)num_cus * per_cu;
  const int64_t each = (pieces + slots - 1) / slots;
  return (pieces + each - 1) / each;
}

template <int FMT, bool BF16>
void launch_1x128(const void* X, uint8_t* Q, float* S, int64_t rows, int64_t K, int,
                  hipStream_t stream) {
  constexpr int E = In<BF16>::E, BPW = 64 / (kBlockK / E), U = 4;
  const int nkb = (int)(K / kBlockK);
  const int64_t nblk = rows * nkb;
  const int64_t per_wg = 4 * U * BPW;                      // blocks per 256-thread workgroup
  hipLaunchKernelGGL((quant_1x128_kernel<FMT, BF16>), dim3((unsigned)((nblk + per_wg - 1) / per_wg)),
                     dim3(256), 0, stream, X, Q, S, nblk, nkb, K);
}

template <int FMT, bool BF16>
void launch_128x128(const void* X, uint8_t* Q, float* S, int64_t rows, int64_t K, int num_cus,
                    hipStream_t stream) {
  const int nkb = (int)(K / kBlockK);
  const int64_t nblk = ((rows + kBlockK - 1) / kBlockK) * nkb;
  // as many workgroups per CU as the registers admit (two blocks' loads per thread)
  const int64_t grid = persistent_grid(nblk, num_cus, BF16 ? 4 : 3);
  hipLaunchKernelGGL((quant_128x128_kernel<FMT, BF16>), dim3((unsigned)grid), dim3(256), 0,
                     stream, X, Q, S, rows, nkb, K, nblk);
}

}  // namespace

// Host-side dispatch over (block shape, format, input type); the caller has validated
// every argument.
void launch_quantize(int block128x128, int fmt, int bf16, const void* X, uint8_t* Q, float* S,
                     int64_t rows, int64_t K, int num_cus, hipStream_t stream) {
  if (block128x128) {
    if (fmt == kFmtE5M2)
      bf16 ? launch_128x128<kFmtE5M2, true>(X, Q, S, rows, K, num_cus, stream)
           : launch_128x128<kFmtE5M2, false>(X, Q, S, rows, K, num_cus, stream);
    else
      bf16 ? launch_128x128<kFmtE4M3, true>(X, Q, S, rows, K, num_cus, stream)
           : launch_128x128<kFmtE4M3, false>(X, Q, S, rows, K, num_cus, stream);
  } else {
    if (fmt == kFmtE5M2)
      bf16 ? launch_1x128<kFmtE5M2, true>(X, Q, S, rows, K, num_cus, stream)
           : launch_1x128<kFmtE5M2, false>(X, Q, S, rows, K, num_cus, stream);
    else
      bf16 ? launch_1x128<kFmtE4M3, true>(X, Q, S, rows, K, num_cus, stream)
           : launch_1x128<kFmtE4M3, false>(X, Q, S, rows, K, num_cus, stream);
  }
}

}  // namespace dg

// ------------------------------------------------------------------------------------
// Byte-matrix transposition (fp8 codes), for operands stored the other way round: the
// pages' calls take B as N x K (NT layout only) and leave transposition to the caller
// (turtlesai.it summary, technical paragraph).  64x64-byte tiles through LDS: each of
// the 256 threads loads one 16-byte row segment and stores one 16-byte segment of the
// transposed tile; rows and columns are multiples of 16, so segments never straddle an
// edge.
namespace dg {
namespace {

__global__ void __launch_bounds__(256)
transpose_u8_kernel(const uint8_t* __restrict__ X, uint8_t* __restrict__ Y, int64_t rows,
                    int64_t cols, int64_t tiles_c) {
  __shared__ uint8_t tile[64][64 + 4];
  const int64_t tr = blockIdx.x / tiles_c, tc = blockIdx.x - tr * tiles_c;
  const int t = threadIdx.x;
  const int seg = t & 3, line = t >> 2;                 // 4 segments of 16 bytes per line
  {
    const int64_t r = tr * 64 + line, c = tc * 64 + seg * 16;
    if (r < rows && c < cols) {
      const uint4 v = *(const uint4*)(X + r * cols + c);
      *(uint4*)&tile[line][seg * 16] = v;
    }
  }
  __syncthreads();
  // output line = input column tc*64 + line, its 16 bytes = input rows tr*64 + 16*seg ..
  const int64_t orow = tc * 64 + line, ocol = tr * 64 + seg * 16;
  if (orow < cols && ocol < rows) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = (uint32_t)tile[seg * 16 + 4 * i][line] | ((uint32_t)tile[seg * 16 + 4 * i + 1][line] << 8) |
             ((uint32_t)tile[seg * 16 + 4 * i + 2][line] << 16) |
             ((uint32_t)tile[seg * 16 + 4 * i + 3][line] << 24);
    *(uint4*)(Y + orow * rows + ocol) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

}  // namespace

void launch_transpose_u8(const uint8_t* X, uint8_t* Y, int64_t rows, int64_t cols,
                         hipStream_t stream) {
  const int64_t tiles_r = (rows + 63) / 64, tiles_c = (cols + 63) / 64;
  hipLaunchKernelGGL(transpose_u8_kernel, dim3((unsigned)(tiles_r * tiles_c)), dim3(256), 0,
                     stream, X, Y, rows, cols, tiles_c);
}

}  // namespace dg
