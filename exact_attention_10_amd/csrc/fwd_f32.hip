// Forward attention, fp32 inputs, vector ALU (gfx950).
//
// Same definition and tile schedule as the bf16 MFMA kernel (tiling and
// online softmax per "Accelerating AI: A Deep Dive into Flash Attention",
// "Tiling the Computation" and "2. Online Softmax"), computed entirely in
// fp32: one lane per query row, 64-row query tiles, 64-key tiles of the
// key/value head staged in LDS and read by every lane as broadcasts.  Used
// for fp32 problems, where no fp32 matrix-core rate would change the picture
// at the sizes such problems come in.

#include "common.h"
#include "internal.h"

namespace attn {
namespace {

constexpr float kNegInf = -__builtin_huge_valf();

template <int D>
__global__ __launch_bounds__(64) void fwd_f32_kernel(FwdArgs a) {
  constexpr int BM = kFwdF32BM, BN = kFwdF32BN;
  __shared__ float lk[BN * D];
  __shared__ float lv[BN * D];
  __shared__ int ldoc[BN];

  const int lane = threadIdx.x;
  const int nqt = (a.Sq + BM - 1) / BM;
  const int per_qt = a.Hq * a.B;
  const int qt = nqt - 1 - blockIdx.x / per_qt;
  const int rem = blockIdx.x % per_qt;
  const int b = rem / a.Hq, h = rem % a.Hq;
  const int kvh = h / (a.Hq / a.Hkv);
  const float* qp = static_cast<const float*>(a.q) + b * a.q_sb + h * a.q_sh;
  const float* kp = static_cast<const float*>(a.k) + b * a.k_sb + kvh * a.k_sh;
  const float* vp = static_cast<const float*>(a.v) + b * a.v_sb + kvh * a.v_sh;

  const int my_q = qt * BM + lane;
  const bool q_ok = my_q < a.Sq;
  float qr[D], acc[D];
  for (int d = 0; d < D; ++d) {
    qr[d] = q_ok ? qp[(int64_t)my_q * a.q_ss + d] : 0.0f;
    acc[d] = 0.0f;
  }
  const float slope = a.alibi != nullptr ? a.alibi[b * a.alibi_sb + h] : 0.0f;
  const bool has_doc = a.mask.doc_q != nullptr;
  const int doc_mine = (has_doc && q_ok) ? a.mask.doc_q[(int64_t)b * a.Sq + my_q] : 0;
  const int delta = a.Sk - a.Sq;

  const RowWindow win(a.Sq, a.Sk, a.mask.causal, a.mask.wl, a.mask.wr);
  const TileRange range(win, qt, BM, BN);
  const bool sparse = a.tiles.kv_num_full != nullptr;
  int n_full = 0, ntiles, qb = qt, mrow = 0;
  if (sparse) {
    qb = (qt * BM) / a.tiles.block_m;
    mrow = b * a.tiles.nQ + qb;
    n_full = a.tiles.kv_num_full[mrow];
    ntiles = (n_full + a.tiles.kv_num_partial[mrow]) * a.tiles.sub;
  } else {
    ntiles = range.kt_end - range.kt_begin;
  }

  float m_run = kNegInf, l_run = 0.0f;
  for (int t = 0; t < ntiles; ++t) {
    int kt;
    bool full;
    if (!sparse) {
      kt = range.kt_begin + t;
      full = range.full(kt);
    } else {
      const int mt = t / a.tiles.sub, sb = t % a.tiles.sub;
      const int64_t base = (int64_t)mrow * a.tiles.nK;
      if (mt < n_full) {
        kt = a.tiles.kv_idx_full[base + mt] * a.tiles.sub + sb;
        full = true;
      } else {
        kt = a.tiles.kv_idx_partial[base + mt - n_full] * a.tiles.sub + sb;
        full = false;
      }
    }
    if (a.trace != nullptr && lane == 0) {
      uint8_t* tr = a.trace + ((int64_t)(b * a.Hq + h) * a.nQt + qb) * a.nKt;
      if (!sparse) tr[kt] = full ? 2 : 1;
      else if (kt % a.tiles.sub == 0) tr[kt / a.tiles.sub] = full ? 2 : 1;
    }
    __syncthreads();
    for (int e = lane; e < BN * D; e += 64) {
      const int row = e / D, d = e % D;
      const int key = kt * BN + row;
      const bool ok = key < a.Sk;
      lk[e] = ok ? kp[(int64_t)key * a.k_ss + d] : 0.0f;
      lv[e] = ok ? vp[(int64_t)key * a.v_ss + d] : 0.0f;
    }
    if (has_doc) {
      const int key = kt * BN + lane;
      ldoc[lane] = key < a.Sk ? a.mask.doc_k[(int64_t)b * a.Sk + key] : -1;
    }
    __syncthreads();

    float sc[BN];
    float mx = kNegInf;
    for (int j = 0; j < BN; ++j) {
      float s = 0.0f;
      for (int d = 0; d < D; ++d) s = __builtin_fmaf(qr[d], lk[j * D + d], s);
      float u = s * a.scale;
      if (a.softcap > 0.0f) u = a.softcap * tanhf(u / a.softcap);
      const int key = kt * BN + j;
      if (a.alibi != nullptr) u -= slope * fabsf(static_cast<float>(my_q + delta - key));
      if (!full) {
        const int i = my_q + delta;
        bool ok = q_ok && key < a.Sk;
        if (a.mask.causal) ok = ok && key <= i;
        if (a.mask.wl >= 0) ok = ok && key >= i - a.mask.wl;
        if (a.mask.wr >= 0) ok = ok && key <= i + a.mask.wr;
        if (has_doc) ok = ok && ldoc[j] == doc_mine;
        if (!ok) u = kNegInf;
      }
      sc[j] = u * kLog2e;
      mx = fmaxf(mx, sc[j]);
    }
    const float m_new = fmaxf(m_run, mx);
    const float msub = m_new == kNegInf ? 0.0f : m_new;
    const float alpha = m_run == kNegInf ? 0.0f : exp2f(m_run - msub);
    l_run *= alpha;
    for (int d = 0; d < D; ++d) acc[d] *= alpha;
    for (int j = 0; j < BN; ++j) {
      const float p = exp2f(sc[j] - msub);
      l_run += p;
      for (int d = 0; d < D; ++d) acc[d] = __builtin_fmaf(p, lv[j * D + d], acc[d]);
    }
    m_run = m_new;
  }
  if (q_ok) {
    const float inv = l_run > 0.0f ? 1.0f / l_run : 0.0f;
    float* op = static_cast<float*>(a.o) + b * a.o_sb + (int64_t)my_q * a.o_ss + h * a.o_sh;
    for (int d = 0; d < D; ++d) op[d] = acc[d] * inv;
    a.lse[((int64_t)b * a.Hq + h) * a.Sq + my_q] =
        l_run > 0.0f ? (m_run + log2f(l_run)) * kLn2 : kNegInf;
  }
}

}  // namespace

hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t s) {
  if (a.Sq == 0 || a.B == 0 || a.Hq == 0) return hipSuccess;
  const int nqt = (a.Sq + kFwdF32BM - 1) / kFwdF32BM;
  const dim3 grid(nqt * a.Hq * a.B), block(64);
  if (a.D == 64) hipLaunchKernelGGL(fwd_f32_kernel<64>, grid, block, 0, s, a);
  else hipLaunchKernelGGL(fwd_f32_kernel<128>, grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace attn
