// Device-side helpers shared by the attention kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef uint16_t bf16_t;  // storage type of bfloat16 tensors

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;
typedef __attribute__((__vector_size__(8 * sizeof(short)))) short i16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kUnbounded = 1 << 30;

__device__ __forceinline__ float bf16_to_f32(bf16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// Round-to-nearest-even float -> bfloat16 bits (the hardware conversion).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  __bf16 b = static_cast<__bf16>(f);
  return __builtin_bit_cast(bf16_t, b);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// 32x32x16 bf16 MFMA, fp32 accumulate.  Operand layouts (wave64):
//   A (32 x 16): lane l holds row l%32, k = 8*(l/32) .. +7
//   B (16 x 32): lane l holds column l%32, k = 8*(l/32) .. +7
//   C (32 x 32): lane l, register r holds row 8*(r/4) + 4*(l/32) + r%4,
//                column l%32
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// LDS transposed read (ds_read_b64_tr_b16).  Within each 16-lane block,
// lane i receives element i%4 of the 8-byte chunks addressed by lanes
// 4*j + i/4, j = 0..3.  If lane s of the block addresses row r0 + s/4,
// columns c0 + 4*(s%4) .. +3 of a row-major 16-bit matrix, lane i receives
// rows r0 .. r0+3 of column c0 + i.
__device__ __forceinline__ i16x4 lds_read_tr16(const bf16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(p));
}

// Concatenate two transposed reads into one MFMA operand.  Done as a whole-
// vector shuffle and bit cast: assembling the bf16 vector element by element
// from 16-bit integer lanes was compiled into code that kept only element 0.
__device__ __forceinline__ bf16x8 cat_frag(i16x4 lo, i16x4 hi) {
  const i16x8 c = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, c);
}

__device__ __forceinline__ float wave_xor32(float x) {
  return __shfl_xor(x, 32, 64);
}

// Per-row allowed key interval for causal / sliding-window masks.
// With delta = Sk - Sq, row i may attend keys j with
//   lo(i) = max(0, i + delta - L) <= j <= hi(i) = min(Sk - 1, i + delta + R)
// where L (left) and R (right; min(R, 0) when causal) may be kUnbounded.
struct RowWindow {
  int Sq, Sk, delta, L, R;
  __host__ __device__ RowWindow(int sq, int sk, int causal, int wl, int wr)
      : Sq(sq), Sk(sk), delta(sk - sq) {
    L = wl < 0 ? kUnbounded : wl;
    R = wr < 0 ? kUnbounded : wr;
    if (causal && R > 0) R = 0;
  }
  __host__ __device__ bool row_nonempty(int i) const {
    if (Sk <= 0) return false;
    if (R != kUnbounded && i + delta + R < 0) return false;
    if (L != kUnbounded && i + delta - L > Sk - 1) return false;
    return true;
  }
  __host__ __device__ int lo(int i) const {
    if (L == kUnbounded) return 0;
    int v = i + delta - L;
    return v < 0 ? 0 : v;
  }
  __host__ __device__ int hi(int i) const {
    if (R == kUnbounded) return Sk - 1;
    int v = i + delta + R;
    return v > Sk - 1 ? Sk - 1 : v;
  }
};

// Tiles of one row block [r0, r0 + bm) against key tiles of width bn.
// Non-empty rows form one interval [i_first, i_last] and the union of their
// key intervals is the contiguous range [lo(i_first), hi(i_last)], so the
// non-empty key tiles are [kt_begin, kt_end).  A tile is FULL when the row
// block and the key tile are wholly in bounds, every row is non-empty and
// every row's interval covers the tile; otherwise it is PARTIAL.
struct TileRange {
  int kt_begin, kt_end;
  int r0, r1, i_first, i_last;
  __host__ __device__ TileRange(const RowWindow& w, int qt, int bm, int bn) {
    r0 = qt * bm;
    r1 = min(r0 + bm, w.Sq) - 1;
    i_first = r0;
    i_last = r1;
    if (w.R != kUnbounded) i_first = max(i_first, -w.delta - w.R);
    if (w.L != kUnbounded) i_last = min(i_last, w.Sk - 1 - w.delta + w.L);
    kt_begin = 0;
    kt_end = 0;
    if (w.Sk <= 0 || i_first > i_last) return;
    int kmin = w.lo(i_first), kmax = w.hi(i_last);
    if (kmax < kmin) return;
    kt_begin = kmin / bn;
    kt_end = kmax / bn + 1;
  }
  __host__ __device__ bool full(const RowWindow& w, int kt, int bm, int bn) const {
    if (r0 + bm > w.Sq || (kt + 1) * bn > w.Sk) return false;
    if (i_first != r0 || i_last != r1) return false;
    if (w.lo(r1) > kt * bn) return false;
    if (w.hi(r0) < (kt + 1) * bn - 1) return false;
    return true;
  }
};

}  // namespace attn
