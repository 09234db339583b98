// Device-side helpers shared by the attention kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef uint16_t bf16_t;  // storage type of bfloat16 tensors

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8;
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
// The same shape with fp16 operands (identical operand and result layouts).
__device__ __forceinline__ f32x16 mfma32(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// 16-bit input element types of the matrix-core kernels.  Both are stored as
// 16-bit patterns (bf16_t); kernels take one of these as a template
// parameter and use vec8 for MFMA operands and elem for conversions (both
// conversions from fp32 round to nearest even).
struct Bf16T {
  using vec8 = bf16x8;
  using elem = __bf16;
  static constexpr uint32_t kNan2 = 0x7FC07FC0u;  // two quiet NaNs
  __device__ static float to_f32(uint16_t h) { return __uint_as_float(static_cast<uint32_t>(h) << 16); }
};
struct F16T {
  using vec8 = f16x8;
  using elem = _Float16;
  static constexpr uint32_t kNan2 = 0x7E007E00u;  // two quiet NaNs
  __device__ static float to_f32(uint16_t h) { return static_cast<float>(__builtin_bit_cast(_Float16, h)); }
};
template <typename T>
__device__ __forceinline__ uint16_t f32_to_elem(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<typename T::elem>(f));
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
template <typename V = bf16x8>
__device__ __forceinline__ V cat_frag(i16x4 lo, i16x4 hi) {
  const i16x8 c = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(V, c);
}

__device__ __forceinline__ float wave_xor32(float x) {
  return __shfl_xor(x, 32, 64);
}

// Max without NaN canonicalisation.  Inline assembly gets no hazard wait
// states from the compiler: never feed it a matrix-core result directly.
__device__ __forceinline__ float max_nc(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ float max3_nc(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// Both halves' values of x in every lane, without an LDS round trip:
// v_permlane32_swap exchanges lanes 32..63 of its first register with lanes
// 0..31 of its second, so on two copies of x lane l ends with x[l % 32] in the
// first and x[l % 32 + 32] in the second.  (Written as assembly on two
// read-write operands, because the compiler builtin's second result was found
// folded onto the first; the s_nops cover the VALU-write -> permlane-read and
// permlane-write -> VALU-read hazards that the compiler does not see here.)
__device__ __forceinline__ void halves32(float x, float* lo, float* hi) {
  float a = x, b = x;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
  *lo = a;
  *hi = b;
}
// Max / sum of x with the value in lane l ^ 32.
__device__ __forceinline__ float pair_max32(float x) {
  float lo, hi;
  halves32(x, &lo, &hi);
  return max_nc(lo, hi);
}
__device__ __forceinline__ float pair_sum32(float x) {
  float lo, hi;
  halves32(x, &lo, &hi);
  return lo + hi;
}

// LDS image of a 64-row x D bf16 tile written by direct global->LDS loads.
// A global_load_lds_dwordx4 instruction stores 16 bytes per lane at
// consecutive 16-byte slots of a wave-uniform LDS base, so one instruction
// fills a 1 KB "group" of RG = 512 / D rows.  Inside a group the slots are
// chunk-major (slot = chunk * RG + row % RG) and groups are GS bytes apart.
// With that layout 16 consecutive rows at one 16-byte chunk (a K fragment
// read) fall in 16 different 4-bank groups, and the transposed reads of 4
// consecutive rows x 32 columns touch 256 contiguous bytes.
template <int D>
struct TileLayout {
  static constexpr int RG = 512 / D;                      // rows per group
  static constexpr int CH = D / 8;                        // 16-byte chunks per row
  static constexpr int GS = 1024 + (D == 128 ? 64 : 128); // group stride (bytes)
  static constexpr int BYTES = (64 / RG) * GS;            // one 64-row tile
  __device__ static constexpr int off(int row, int chunk) {
    return (row / RG) * GS + (chunk * RG + row % RG) * 16;
  }
};

// LDS byte address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

// One global_load_lds_dwordx4 issued from inline assembly: lane i's 16 bytes
// at gptr land at LDS byte lds_base + 16 * i (lds_base wave-uniform, via M0).
// The compiler does not count these copies, so it adds no waits for them
// before LDS reads; the caller orders them with its own vmcnt waits.  All
// later VMEM waits the compiler emits stay correct (they can only over-wait,
// since the counter retires in order).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const void* gptr, uint32_t lds_base) {
  lds_base = __builtin_amdgcn_readfirstlane(lds_base);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
               :: "s"(lds_base), "v"(gptr) : "memory", "m0");
}
// The same with 4 bytes per lane (global_load_lds_dword): lane i's word lands
// at lds_base + 4 * i.
__device__ __forceinline__ void dma4(const void* gptr, uint32_t lds_base) {
  lds_base = __builtin_amdgcn_readfirstlane(lds_base);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off"
               :: "s"(lds_base), "v"(gptr) : "memory", "m0");
}
#pragma clang diagnostic pop

// Wave-cooperative copy of rows [row0, row0 + 64) of a [rows, D] bf16 matrix
// (row stride `ld` elements) into a TileLayout image at `tile`.  Rows at or
// past `nrows` are read from row nrows - 1 instead (callers mask them), so no
// address leaves the matrix.  NW waves; wave w copies groups w, w + NW, ...
// ASM: issue the copies from inline assembly (dma16), so the compiler's wait
// counting never sees them (the caller waits with wait_dma()).
template <int D, int NW = 4, bool ASM = false>
__device__ __forceinline__ void tile_dma(bf16_t* tile, const bf16_t* src, int64_t ld, int row0,
                                         int nrows, int wave, int lane) {
  using L = TileLayout<D>;
  static_assert((64 / L::RG) % NW == 0, "groups must divide among the waves");
#pragma unroll
  for (int u = 0; u < 64 / L::RG / NW; ++u) {
    const int grp = wave + NW * u;
    const int row = grp * L::RG + lane % L::RG;
    const int chunk = lane / L::RG;
    int key = row0 + row;
    key = key < nrows ? key : nrows - 1;
    const bf16_t* gp = src + (int64_t)key * ld + chunk * 8;
    bf16_t* lp = reinterpret_cast<bf16_t*>(reinterpret_cast<char*>(tile) + grp * L::GS);
    if constexpr (ASM)
      dma16(gp, lds_addr(lp));
    else
      __builtin_amdgcn_global_load_lds(gp, (__attribute__((address_space(3))) void*)lp, 16, 0, 0);
  }
}

// The same copy with the per-lane part of the address computed once: a tile
// at row0 then costs one scalar base and one 64-bit add per copy (the
// clamping form above is kept for a tile that runs past nrows).  ASM as in
// tile_dma.
template <int D, int NW = 4, bool ASM = false>
struct TileCopy {
  using L = TileLayout<D>;
  static constexpr int NU = 64 / L::RG / NW;  // copies per lane per tile
  static_assert((64 / L::RG) % NW == 0, "groups must divide among the waves");
  const bf16_t* src;
  int64_t ld;
  int64_t lane_off;  // bytes from a tile's first row to this lane's 16 bytes (copy 0)
  int nrows, wave, lane;
  __device__ TileCopy(const bf16_t* src_, int64_t ld_, int nrows_, int wave_, int lane_)
      : src(src_), ld(ld_), nrows(nrows_), wave(wave_), lane(lane_) {
    lane_off = ((int64_t)(wave_ * L::RG + lane_ % L::RG) * ld_ + (lane_ / L::RG) * 8) * 2;
  }
  // elem_off: elements added to the source (another head of the same layout)
  __device__ __forceinline__ void operator()(bf16_t* tile, int row0, int64_t elem_off = 0) const {
    if (row0 + 64 > nrows) {
      tile_dma<D, NW, ASM>(tile, src + elem_off, ld, row0, nrows, wave, lane);
      return;
    }
    const char* base = reinterpret_cast<const char*>(src + elem_off) + (int64_t)row0 * ld * 2;
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const char* gp = base + (int64_t)u * NW * L::RG * ld * 2 + lane_off;
      char* lp = reinterpret_cast<char*>(tile) + (wave + NW * u) * L::GS;
      if constexpr (ASM)
        dma16(gp, lds_addr(lp));
      else
        __builtin_amdgcn_global_load_lds(gp, (__attribute__((address_space(3))) void*)lp, 16, 0, 0);
    }
  }
};

__device__ __forceinline__ void wait_dma() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }



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
  // Allowed keys of row i as [*first, *first + *count) (count 0: none).
  __host__ __device__ void row_keys(int i, int* first, int* count) const {
    *first = 0;
    *count = 0;
    if (i < 0 || i >= Sq || !row_nonempty(i)) return;
    *first = lo(i);
    *count = hi(i) - *first + 1;
  }
  // Rows that may attend key j as [*first, *first + *count): the rows i with
  // i + delta - L <= j <= i + delta + R, clipped to [0, Sq).
  __host__ __device__ void key_rows(int j, int* first, int* count) const {
    *first = 0;
    *count = 0;
    if (j < 0 || j >= Sk) return;
    const int a = R == kUnbounded ? 0 : max(0, j - delta - R);
    const int b = L == kUnbounded ? Sq - 1 : min(Sq - 1, j - delta + L);
    if (b < a) return;
    *first = a;
    *count = b - a + 1;
  }
};

// Tiles of one row block [r0, r0 + bm) against key tiles of width bn.
// Non-empty rows form one interval [i_first, i_last] and the union of their
// key intervals is the contiguous range [lo(i_first), hi(i_last)], so the
// non-empty key tiles are [kt_begin, kt_end).  A tile is FULL when the row
// block and the key tile are wholly in bounds, every row is non-empty and
// every row's interval covers the tile; otherwise it is PARTIAL.
struct TileRange {
  int kt_begin, kt_end;   // non-empty key tiles
  int f_begin, f_end;     // FULL key tiles (a sub-range; empty when f_begin >= f_end)
  int r0, r1, i_first, i_last;
  __host__ __device__ TileRange(const RowWindow& w, int qt, int bm, int bn) {
    r0 = qt * bm;
    r1 = min(r0 + bm, w.Sq) - 1;
    i_first = r0;
    i_last = r1;
    if (w.R != kUnbounded) i_first = max(i_first, -w.delta - w.R);
    if (w.L != kUnbounded) i_last = min(i_last, w.Sk - 1 - w.delta + w.L);
    kt_begin = kt_end = f_begin = f_end = 0;
    if (w.Sk <= 0 || i_first > i_last) return;
    const int kmin = w.lo(i_first), kmax = w.hi(i_last);
    if (kmax < kmin) return;
    kt_begin = kmin / bn;
    kt_end = kmax / bn + 1;
    // FULL: the row block and key tile lie inside the matrix, no row is
    // empty, and every row's interval covers the tile.  lo() grows with the
    // row, so the binding rows are r1 for the lower and r0 for the upper end.
    if (r0 + bm > w.Sq || i_first != r0 || i_last != r1) return;
    const int lo_max = w.lo(r1), hi_min = w.hi(r0);
    const int fb = (lo_max + bn - 1) / bn;
    int fe = (hi_min + 1) / bn;                 // tiles with (kt + 1) * bn - 1 <= hi_min
    if (fe > w.Sk / bn) fe = w.Sk / bn;         // and (kt + 1) * bn <= Sk
    f_begin = max(fb, kt_begin);
    f_end = min(fe, kt_end);
    if (f_end < f_begin) f_end = f_begin;
  }
  __host__ __device__ bool full(int kt) const { return kt >= f_begin && kt < f_end; }
  __host__ __device__ int n_full() const { return f_end - f_begin; }
  // The t-th tile when FULL tiles come first, then the partial ones in
  // ascending order.
  __host__ __device__ int kt_at(int t) const {
    const int nf = f_end - f_begin;
    if (t < nf) return f_begin + t;
    const int p = t - nf;
    const int before = f_begin - kt_begin;
    return p < before ? kt_begin + p : f_end + (p - before);
  }
};

}  // namespace attn
