// Block-mask construction on the device.
//
// The FlexAttention block mask ("FlexAttention uses much more GPU memory than
// FlashAttention-2": create_block_mask(mask_mod, B, H, Q_LEN, KV_LEN,
// BLOCK_SIZE); "Lightning Talk: FlexAttention + FlashAttention-4": block
// sparsity lets the kernel skip tiles with nothing to compute) classifies
// every (block_m x block_n) tile as EMPTY (0), PARTIAL (1) or FULL (2).
//
// classify: one wave per tile.  The causal / sliding-window part of the
//   predicate is an interval of keys per query row, so whether it leaves the
//   tile non-empty and whether it covers it completely follow in closed form
//   from the row block's first and last rows (TileRange, the same arithmetic
//   the attention kernels use to skip tiles).  Without a document mask that
//   is the class.  With one, the tile's row and column document ids are read
//   once each (into LDS): when both sides hold a single document the class
//   follows from comparing the two ids; otherwise (a tile at a document
//   boundary) the in-bounds pairs the window allows are tested against the
//   LDS copies until one shares a document.  FULL requires the tile to lie
//   wholly inside [0, Sq) x [0, Sk) and every pair allowed.
// compact:  one wave per tile row (kv lists) or tile column (q lists) builds
//   the ascending CSR lists with ballots and bit counts, 64 tiles per round,
//   and zero-fills the unused tail.

#include "common.h"
#include "internal.h"

namespace attn {
namespace {

constexpr int kMaxBlock = 1024;  // largest block_m / block_n with document ids staged in LDS

// One wave per tile.
__global__ __launch_bounds__(64) void classify_kernel(BlockMaskArgs a) {
  __shared__ int rdoc[kMaxBlock];
  __shared__ int cdoc[kMaxBlock];
  const int kb = blockIdx.x, qb = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x;
  const RowWindow win(a.Sq, a.Sk, a.mask.causal, a.mask.wl, a.mask.wr);
  const TileRange range(win, qb, a.bm, a.bn);
  uint8_t* out = a.cls + ((int64_t)b * a.nQ + qb) * a.nK + kb;
  const bool nonempty = kb >= range.kt_begin && kb < range.kt_end;
  if (!nonempty || a.mask.doc_q == nullptr) {
    // causal / window only: the closed-form class
    if (lane == 0) *out = nonempty ? (range.full(kb) ? 2 : 1) : 0;
    return;
  }
  const int i0 = qb * a.bm, j0 = kb * a.bn;
  const int nrow = min(a.bm, a.Sq - i0), ncol = min(a.bn, a.Sk - j0);
  const int* dq = a.mask.doc_q + (int64_t)b * a.Sq + i0;
  const int* dk = a.mask.doc_k + (int64_t)b * a.Sk + j0;
  const int row_doc = dq[0], col_doc = dk[0];
  int same = 1;
  for (int t = lane; t < nrow; t += 64) {
    const int d = dq[t];
    rdoc[t] = d;
    same &= d == row_doc;
  }
  for (int t = lane; t < ncol; t += 64) {
    const int d = dk[t];
    cdoc[t] = d;
    same &= d == col_doc;
  }
  const bool uniform = __all(same);
  uint8_t c;
  if (uniform) {
    // one document on each side: every pair, or no pair, shares a document
    c = row_doc != col_doc ? 0 : (range.full(kb) ? 2 : 1);
  } else {
    // a document boundary crosses the tile: test the pairs the window
    // allows; such a tile is never FULL (not all pairs share a document)
    __syncthreads();  // the LDS copies are complete
    int any = 0;
    const int npair = nrow * ncol;
    for (int e = lane; e < npair; e += 64) {
      const int r = e / ncol, cc = e - r * ncol;
      const int i = i0 + r, j = j0 + cc;
      if (win.row_nonempty(i) && j >= win.lo(i) && j <= win.hi(i) && rdoc[r] == cdoc[cc]) any = 1;
      if (__any(any)) break;
    }
    c = __any(any) ? 1 : 0;
  }
  if (lane == 0) *out = c;
}

// Ascending CSR list of the positions holding class `want` among n classes
// cls[0], cls[stride], ...: one wave, 64 positions per round (ballot and bit
// count give each hit its slot); the unused tail is zero-filled.
__device__ __forceinline__ int wave_compact(const uint8_t* cls, int64_t stride, int n, uint8_t want,
                                            int32_t* idx, int lane) {
  int count = 0;
  for (int base = 0; base < n; base += 64) {
    const int p = base + lane;
    const bool hit = p < n && cls[(int64_t)p * stride] == want;
    const uint64_t m = __ballot(hit);
    if (hit) idx[count + __popcll(m & ((1ull << lane) - 1))] = p;
    count += __popcll(m);
  }
  for (int p = count + lane; p < n; p += 64) idx[p] = 0;
  return count;
}

__global__ __launch_bounds__(256) void compact_kernel(BlockMaskArgs a) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);  // one wave per row or column of tiles
  const int nrows = a.B * a.nQ, ncols = a.B * a.nK;
  if (t < nrows) {
    const uint8_t* c = a.cls + (int64_t)t * a.nK;
    const int np = wave_compact(c, 1, a.nK, 1, a.kv_idx_partial + (int64_t)t * a.nK, lane);
    const int nf = wave_compact(c, 1, a.nK, 2, a.kv_idx_full + (int64_t)t * a.nK, lane);
    if (lane == 0) {
      a.kv_num_partial[t] = np;
      a.kv_num_full[t] = nf;
    }
  } else if (t < nrows + ncols) {
    const int u = t - nrows;
    const int b = u / a.nK, kb = u % a.nK;
    const uint8_t* c = a.cls + (int64_t)b * a.nQ * a.nK + kb;
    const int np = wave_compact(c, a.nK, a.nQ, 1, a.q_idx_partial + (int64_t)u * a.nQ, lane);
    const int nf = wave_compact(c, a.nK, a.nQ, 2, a.q_idx_full + (int64_t)u * a.nQ, lane);
    if (lane == 0) {
      a.q_num_partial[u] = np;
      a.q_num_full[u] = nf;
    }
  }
}

}  // namespace

int block_mask_max_block() { return kMaxBlock; }

hipError_t launch_block_mask(const BlockMaskArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(classify_kernel, dim3(a.nK, a.nQ, a.B), dim3(64), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int waves = a.B * (a.nQ + a.nK);
  hipLaunchKernelGGL(compact_kernel, dim3((waves + 3) / 4), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace attn
