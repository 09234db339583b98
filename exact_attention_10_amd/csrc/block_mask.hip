// Block-mask construction on the device.
//
// The FlexAttention block mask ("FlexAttention uses much more GPU memory than
// FlashAttention-2": create_block_mask(mask_mod, B, H, Q_LEN, KV_LEN,
// BLOCK_SIZE); "Lightning Talk: FlexAttention + FlashAttention-4": block
// sparsity lets the kernel skip tiles with nothing to compute) classifies
// every (block_m x block_n) tile as EMPTY (0), PARTIAL (1) or FULL (2).
//
// classify: one workgroup per tile evaluates the mask predicate on every
//   in-bounds pair of the tile and reduces "any allowed" and "all allowed"
//   across the workgroup.  FULL additionally requires the tile to lie wholly
//   inside [0, Sq) x [0, Sk).
// compact:  one lane per tile row (kv lists) or tile column (q lists) scans
//   the classes in ascending order and writes the CSR lists, zero-filling
//   the unused tail.

#include "common.h"
#include "internal.h"

namespace attn {
namespace {

__device__ __forceinline__ bool allowed(const MaskArgs& m, int b, int Sq, int Sk, int i, int j) {
  const int ii = i + (Sk - Sq);
  if (m.causal && j > ii) return false;
  if (m.wl >= 0 && j < ii - m.wl) return false;
  if (m.wr >= 0 && j > ii + m.wr) return false;
  if (m.doc_q != nullptr && m.doc_q[(int64_t)b * Sq + i] != m.doc_k[(int64_t)b * Sk + j]) return false;
  return true;
}

__global__ __launch_bounds__(256) void classify_kernel(BlockMaskArgs a) {
  const int kb = blockIdx.x, qb = blockIdx.y, b = blockIdx.z;
  const int i0 = qb * a.bm, j0 = kb * a.bn;
  const bool inside = i0 + a.bm <= a.Sq && j0 + a.bn <= a.Sk;
  int any_ok = 0, all_ok = 1;
  const int n = a.bm * a.bn;
  for (int e = threadIdx.x; e < n; e += blockDim.x) {
    const int i = i0 + e / a.bn, j = j0 + e % a.bn;
    const bool inb = i < a.Sq && j < a.Sk;
    const bool ok = inb && allowed(a.mask, b, a.Sq, a.Sk, i, j);
    any_ok |= ok;
    all_ok &= ok;
  }
  any_ok = __syncthreads_or(any_ok);
  all_ok = __syncthreads_and(all_ok);
  if (threadIdx.x == 0) {
    const uint8_t c = !any_ok ? 0 : (inside && all_ok ? 2 : 1);
    a.cls[((int64_t)b * a.nQ + qb) * a.nK + kb] = c;
  }
}

__global__ __launch_bounds__(256) void compact_kernel(BlockMaskArgs a) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  const int nrows = a.B * a.nQ, ncols = a.B * a.nK;
  if (t < nrows) {
    const int b = t / a.nQ, qb = t % a.nQ;
    const uint8_t* c = a.cls + ((int64_t)b * a.nQ + qb) * a.nK;
    int32_t* ip = a.kv_idx_partial + (int64_t)t * a.nK;
    int32_t* iff = a.kv_idx_full + (int64_t)t * a.nK;
    int np = 0, nf = 0;
    for (int kb = 0; kb < a.nK; ++kb) {
      if (c[kb] == 1) ip[np++] = kb;
      else if (c[kb] == 2) iff[nf++] = kb;
    }
    for (int x = np; x < a.nK; ++x) ip[x] = 0;
    for (int x = nf; x < a.nK; ++x) iff[x] = 0;
    a.kv_num_partial[t] = np;
    a.kv_num_full[t] = nf;
  } else if (t < nrows + ncols) {
    const int u = t - nrows;
    const int b = u / a.nK, kb = u % a.nK;
    const uint8_t* c = a.cls + (int64_t)b * a.nQ * a.nK + kb;
    int32_t* ip = a.q_idx_partial + (int64_t)u * a.nQ;
    int32_t* iff = a.q_idx_full + (int64_t)u * a.nQ;
    int np = 0, nf = 0;
    for (int qb = 0; qb < a.nQ; ++qb) {
      const uint8_t v = c[(int64_t)qb * a.nK];
      if (v == 1) ip[np++] = qb;
      else if (v == 2) iff[nf++] = qb;
    }
    for (int x = np; x < a.nQ; ++x) ip[x] = 0;
    for (int x = nf; x < a.nQ; ++x) iff[x] = 0;
    a.q_num_partial[u] = np;
    a.q_num_full[u] = nf;
  }
}

}  // namespace

hipError_t launch_block_mask(const BlockMaskArgs& a, hipStream_t s) {
  const dim3 grid1(a.nK, a.nQ, a.B);
  hipLaunchKernelGGL(classify_kernel, grid1, dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int total = a.B * (a.nQ + a.nK);
  hipLaunchKernelGGL(compact_kernel, dim3((total + 255) / 256), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace attn
