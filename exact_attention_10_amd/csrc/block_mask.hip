// Block-mask construction on the device.
//
// The FlexAttention block mask ("FlexAttention uses much more GPU memory than
// FlashAttention-2": create_block_mask(mask_mod, B, H, Q_LEN, KV_LEN,
// BLOCK_SIZE); "Lightning Talk: FlexAttention + FlashAttention-4": block
// sparsity lets the kernel skip tiles with nothing to compute) classifies
// every (block_m x block_n) tile as EMPTY (0), PARTIAL (1) or FULL (2).
//
// classify: one workgroup per row of tiles, a wave per tile at a time.  The
//   causal / sliding-window part of the predicate is an interval of keys per
//   query row, so whether it leaves the tile non-empty and whether it covers
//   it completely follow in closed form from the row block's first and last
//   rows (TileRange, the same arithmetic the attention kernels use to skip
//   tiles).  Without a document mask that is the class.  With one, the row
//   block's document ids are read once per workgroup and each tile's column
//   ids once (a wave loads the ids of several tiles together, so their
//   latencies overlap).  When the ranges [least, greatest] of the two sides'
//   ids do not meet, no pair shares a document and the tile is EMPTY; when
//   both sides hold one document (the same one) the window class stands;
//   when one side holds one document, one test per row (or column) of the
//   other side against the window decides; only when both sides mix
//   documents are the pairs the window allows tested, 64 rows at a time,
//   until one shares a document.  FULL requires the tile to lie wholly
//   inside [0, Sq) x [0, Sk) and every pair allowed.
// compact:  one wave per tile row (kv lists) or tile column (q lists) builds
//   the ascending CSR lists with ballots and bit counts, 64 tiles per round,
//   and zero-fills the unused tail.

#include "common.h"
#include "internal.h"

namespace attn {
namespace {

constexpr int kMaxBlock = 1024;  // largest block_m / block_n with document ids staged in LDS
constexpr int kWaves = 4;         // waves per workgroup (one row of tiles)
constexpr int kBatch = 16;        // key tiles a wave classifies per round

__device__ __forceinline__ int wave_min(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ int wave_max(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o, 64));
  return v;
}

// One workgroup per row of tiles (b, qb); wave w takes key tiles w, w + 4,
// ..., kBatch at a time, with all their column ids loaded at once.
__global__ __launch_bounds__(64 * kWaves) void classify_kernel(BlockMaskArgs a) {
  __shared__ int rdoc[kMaxBlock];
  __shared__ __align__(16) int cdoc_w[kWaves][kMaxBlock];
  __shared__ int rlo_w[kWaves], rhi_w[kWaves];
  const int qb = blockIdx.x, b = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const RowWindow win(a.Sq, a.Sk, a.mask.causal, a.mask.wl, a.mask.wr);
  const TileRange range(win, qb, a.bm, a.bn);
  uint8_t* out = a.cls + ((int64_t)b * a.nQ + qb) * a.nK;
  const bool has_doc = a.mask.doc_q != nullptr;
  const int i0 = qb * a.bm, nrow = min(a.bm, a.Sq - i0), i1 = i0 + nrow - 1;
  int* cdoc = cdoc_w[wave];

  // column ids of a round's tiles: lane l holds columns l and l + 64 of
  // each tile (loaded together, so their latencies overlap); columns past
  // 128 are read where they are needed
  int cid[kBatch][2];
  auto load_round = [&](int kb0) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      cid[u][0] = cid[u][1] = 0;
      const int kb = kb0 + kWaves * u;
      if (has_doc && kb < a.nK && kb >= range.kt_begin && kb < range.kt_end) {
        const int j0 = kb * a.bn, ncol = min(a.bn, a.Sk - j0);
        const int* dk = a.mask.doc_k + (int64_t)b * a.Sk + j0;
        if (lane < ncol) cid[u][0] = dk[lane];
        if (lane + 64 < ncol) cid[u][1] = dk[lane + 64];
      }
    }
  };
  // the first round's loads are in flight while the row ids arrive
  load_round(wave);

  // the row block's document ids (into LDS) and their least and greatest
  // value, once per workgroup
  int row_lo = 0, row_hi = 0;
  if (has_doc) {
    const int* dq = a.mask.doc_q + (int64_t)b * a.Sq + i0;
    int lo = INT_MAX, hi = INT_MIN;
    for (int t = threadIdx.x; t < nrow; t += 64 * kWaves) {
      const int v = dq[t];
      rdoc[t] = v;
      lo = min(lo, v);
      hi = max(hi, v);
    }
    lo = wave_min(lo);
    hi = wave_max(hi);
    if (lane == 0) {
      rlo_w[wave] = lo;
      rhi_w[wave] = hi;
    }
    __syncthreads();
    row_lo = rlo_w[0];
    row_hi = rhi_w[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) {
      row_lo = min(row_lo, rlo_w[w]);
      row_hi = max(row_hi, rhi_w[w]);
    }
  }
  const bool row_uniform = row_lo == row_hi;

  for (int kb0 = wave; kb0 < a.nK; kb0 += kWaves * kBatch) {
    if (kb0 != wave) load_round(kb0);
    // the round's classes, two bits per tile, stored together at the end
    // (a store per tile would make each later wait on the load counter also
    // wait for the previous store to complete)
    uint32_t pack = 0;
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int kb = kb0 + kWaves * u;
      if (kb >= a.nK) break;
      const bool nonempty = kb >= range.kt_begin && kb < range.kt_end;
      uint32_t c = nonempty ? (range.full(kb) ? 2 : 1) : 0;
      if (has_doc && nonempty) {
        const int j0 = kb * a.bn, ncol = min(a.bn, a.Sk - j0), j1 = j0 + ncol - 1;
        const int* dk = a.mask.doc_k + (int64_t)b * a.Sk + j0;
        const bool in0 = lane < ncol, in1 = lane + 64 < ncol;
        const int col_first = __shfl(cid[u][0], 0, 64);
        // least and greatest column id (columns past 128 also go to LDS)
        int lo = in0 ? cid[u][0] : INT_MAX, hi = in0 ? cid[u][0] : INT_MIN;
        if (in1) {
          lo = min(lo, cid[u][1]);
          hi = max(hi, cid[u][1]);
        }
        for (int t = lane + 128; t < ncol; t += 64) {
          const int v = dk[t];
          cdoc[t] = v;
          lo = min(lo, v);
          hi = max(hi, v);
        }
        const bool col_uniform = __all(!in0 || (lo == col_first && hi == col_first));
        int col_lo = col_first, col_hi = col_first;
        if (!col_uniform) {
          col_lo = wave_min(lo);
          col_hi = wave_max(hi);
        }
        if (col_hi < row_lo || row_hi < col_lo) {
          // no document id occurs on both sides
          c = 0;
        } else if (row_uniform && col_uniform) {
          // one document on each side, the same one: every pair shares it
        } else {
          // A document boundary crosses the tile, so not every pair shares
          // a document and the tile is not FULL; it is PARTIAL if some pair
          // the window allows does.
          int any = 0;
          if (col_uniform) {
            // one column document: a row of it whose key interval meets the tile
            for (int r = lane; r < nrow; r += 64) {
              const int i = i0 + r;
              if (rdoc[r] == col_first && win.row_nonempty(i) && win.lo(i) <= j1 && win.hi(i) >= j0) any = 1;
            }
          } else {
            if (in0) cdoc[lane] = cid[u][0];
            if (in1) cdoc[lane + 64] = cid[u][1];
            if (row_uniform) {
              // one row document: a column of it whose row interval meets the tile
              for (int cc = lane; cc < ncol; cc += 64) {
                int first, count;
                win.key_rows(j0 + cc, &first, &count);
                if (cdoc[cc] == row_lo && count > 0 && first <= i1 && first + count - 1 >= i0) any = 1;
              }
            } else {
              // both sides mixed: lanes over rows, each holding its row's
              // document and the part of its key interval inside the tile;
              // the column ids are read four at a time as LDS broadcasts
              // (columns past ncol lie outside every interval, so the stale
              // ids read there never count)
              for (int r0 = 0; r0 < nrow && !__any(any); r0 += 64) {
                const int r = r0 + lane, i = i0 + r;
                int dr = 0, a0 = 1, a1 = 0;  // empty interval by default
                if (r < nrow && win.row_nonempty(i)) {
                  dr = rdoc[r];
                  a0 = max(win.lo(i), j0) - j0;
                  a1 = min(win.hi(i), j1) - j0;
                }
                for (int cb = 0; cb < ncol && !__any(any); cb += 16) {
#pragma unroll
                  for (int q = 0; q < 16; q += 4) {
                    const int4 v = *reinterpret_cast<const int4*>(cdoc + cb + q);
                    const int cc = cb + q;
                    any |= (v.x == dr) & (cc >= a0) & (cc <= a1);
                    any |= (v.y == dr) & (cc + 1 >= a0) & (cc + 1 <= a1);
                    any |= (v.z == dr) & (cc + 2 >= a0) & (cc + 2 <= a1);
                    any |= (v.w == dr) & (cc + 3 >= a0) & (cc + 3 <= a1);
                  }
                }
              }
            }
          }
          c = __any(any) ? 1 : 0;
        }
      }
      pack |= c << (2 * u);
    }
    const int kb = kb0 + kWaves * lane;
    if (lane < kBatch && kb < a.nK) out[kb] = (pack >> (2 * lane)) & 3;
  }
}

// Ascending CSR lists of the PARTIAL (1) and FULL (2) positions among n
// classes cls[0], cls[stride], ...: one wave, 64 positions per round, each
// class byte read once (ballots and bit counts give each hit its slot); the
// unused tails are zero-filled.
__device__ __forceinline__ void wave_compact(const uint8_t* cls, int64_t stride, int n, int32_t* idx_p,
                                             int32_t* idx_f, int* num_p, int* num_f, int lane) {
  int np = 0, nf = 0;
  const uint64_t below = (1ull << lane) - 1;
  for (int base = 0; base < n; base += 64) {
    const int p = base + lane;
    const int c = p < n ? cls[(int64_t)p * stride] : 0;
    const uint64_t mp = __ballot(c == 1), mf = __ballot(c == 2);
    if (c == 1) idx_p[np + __popcll(mp & below)] = p;
    if (c == 2) idx_f[nf + __popcll(mf & below)] = p;
    np += __popcll(mp);
    nf += __popcll(mf);
  }
  for (int p = np + lane; p < n; p += 64) idx_p[p] = 0;
  for (int p = nf + lane; p < n; p += 64) idx_f[p] = 0;
  if (lane == 0) {
    *num_p = np;
    *num_f = nf;
  }
}

__global__ __launch_bounds__(256) void compact_kernel(BlockMaskArgs a) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);  // one wave per row or column of tiles
  const int nrows = a.B * a.nQ, ncols = a.B * a.nK;
  if (t < nrows) {
    const int64_t o = (int64_t)t * a.nK;
    wave_compact(a.cls + o, 1, a.nK, a.kv_idx_partial + o, a.kv_idx_full + o, a.kv_num_partial + t,
                 a.kv_num_full + t, lane);
  } else if (t < nrows + ncols) {
    const int u = t - nrows;
    const int b = u / a.nK, kb = u % a.nK;
    const int64_t o = (int64_t)u * a.nQ;
    wave_compact(a.cls + (int64_t)b * a.nQ * a.nK + kb, a.nK, a.nQ, a.q_idx_partial + o, a.q_idx_full + o,
                 a.q_num_partial + u, a.q_num_full + u, lane);
  }
}

}  // namespace

int block_mask_max_block() { return kMaxBlock; }

hipError_t launch_block_mask(const BlockMaskArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(classify_kernel, dim3(a.nQ, a.B), dim3(64 * kWaves), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int waves = a.B * (a.nQ + a.nK);
  hipLaunchKernelGGL(compact_kernel, dim3((waves + 3) / 4), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace attn
