// Backward attention from the saved log-sum-exp, bf16 (gfx950).
//
// "Lightning Talk: FlexAttention + FlashAttention-4" notes that the backward
// reuses the forward's machinery; "FlashAttention: Fast and Memory-Efficient
// Exact Attention" ("Examples") offers a deterministic backward.  Here the
// probabilities are recomputed tile by tile from the saved LSE, never stored:
//
//   P    = exp(u - lse)                   (u: scaled, capped, biased score)
//   dV  += P^T dO
//   dP   = dO V^T
//   dS   = P * (dP - Delta) * (softcap ? 1 - tanh^2 : 1),  Delta = rowsum(dO * O)
//   dK  += scale * dS^T Q
//   dQ  += scale * dS K
//
// Three kernels, no atomics (every output element is summed in a fixed
// order, so results are bitwise repeatable):
//  1. preprocess: Delta_i = <dO_i, O_i> in fp32.
//  2. dK/dV: a workgroup owns 128 keys of one (batch, query head); each wave
//     keeps its 32 keys of K and V in registers as MFMA operands and streams
//     32-query tiles of Q and dO through LDS.  S = Q K^T puts one key per
//     lane, so P and dS (rounded to bf16) are directly the A operands of
//     dV += P^T dO and dK += dS^T Q, whose B operands are transposed LDS
//     reads of the dO and Q tiles.  With grouped-query heads each query head
//     writes an fp32 partial and a reduction kernel sums the group in head
//     order; with one query head per kv head the result is written directly.
//  3. dQ: the forward's layout -- a workgroup owns 128 query rows, Q and dO
//     stay in registers, K and V tiles stream through LDS; S^T = K Q^T and
//     dP^T = V dO^T give one query per lane, and dQ^T += K^T dS^T uses
//     transposed reads of the K tile.

#include "common.h"
#include "internal.h"

namespace attn {
namespace {

constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kPosInf = __builtin_huge_valf();

// ---------------------------------------------------------------------------
// 1. Delta = rowsum(dO * O), one 16-lane group per (b, i, h) row.

template <int D>
__global__ __launch_bounds__(256) void bwd_delta_kernel(BwdArgs a) {
  constexpr int LPR = D / 8;  // lanes per row (8 elements each)
  const int64_t rows = (int64_t)a.B * a.Sq * a.Hq;
  const int64_t row = ((int64_t)blockIdx.x * 256 + threadIdx.x) / LPR;
  const int part = threadIdx.x % LPR;
  float acc = 0.0f;
  int b = 0, i = 0, h = 0;
  if (row < rows) {
    h = static_cast<int>(row % a.Hq);
    i = static_cast<int>((row / a.Hq) % a.Sq);
    b = static_cast<int>(row / ((int64_t)a.Hq * a.Sq));
    const uint4 o4 = *reinterpret_cast<const uint4*>(static_cast<const bf16_t*>(a.o) + b * a.o_sb +
                                                     (int64_t)i * a.o_ss + h * a.o_sh + part * 8);
    const uint4 d4 = *reinterpret_cast<const uint4*>(static_cast<const bf16_t*>(a.dout) + b * a.do_sb +
                                                     (int64_t)i * a.do_ss + h * a.do_sh + part * 8);
    const uint32_t ow[4] = {o4.x, o4.y, o4.z, o4.w};
    const uint32_t dw[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc = __builtin_fmaf(__uint_as_float(ow[e] << 16), __uint_as_float(dw[e] << 16), acc);
      acc = __builtin_fmaf(__uint_as_float(ow[e] & 0xffff0000u), __uint_as_float(dw[e] & 0xffff0000u), acc);
    }
  }
#pragma unroll
  for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
  if (row < rows && part == 0) a.delta[((int64_t)b * a.Hq + h) * a.Sq + i] = acc;
}

// Scores in the exp2 domain for a raw dot product r of (query i, key j).
template <bool kAlibi, bool kSoftcap>
__device__ __forceinline__ float score_x(float r, float scale_log2, float cap_k2, float cap_log2,
                                         float slope_log2, int dist, float* tanh_out) {
  float x;
  if (kSoftcap) {
    const float e = fast_exp2(r * cap_k2);
    const float th = 1.0f - 2.0f * fast_rcp(e + 1.0f);
    *tanh_out = th;
    x = cap_log2 * th;
  } else {
    x = r * scale_log2;
  }
  if (kAlibi) x = __builtin_fmaf(-slope_log2, fabsf(static_cast<float>(dist)), x);
  return x;
}

__device__ __forceinline__ bool mask_ok(const MaskArgs& m, int Sq, int Sk, int i, int j) {
  if (i >= Sq || j >= Sk) return false;
  const int ii = i + (Sk - Sq);
  if (m.causal && j > ii) return false;
  if (m.wl >= 0 && j < ii - m.wl) return false;
  if (m.wr >= 0 && j > ii + m.wr) return false;
  return true;
}

// ---------------------------------------------------------------------------
// 2. dK / dV

template <int D>
struct KVCfg {
  static constexpr int BN = 128;           // keys per workgroup (4 waves x 32)
  static constexpr int BM = 32;            // queries per streamed tile
  static constexpr int NT = 256;
  static constexpr int QS = D + 16;        // LDS row stride of the Q / dO tiles
  static constexpr int QT = BM * QS;
  static constexpr int CPT = BM * D / 8 / NT;  // 16-byte chunks per thread (Q or dO)
  static constexpr int DSTEPS = D / 16;
  static constexpr int DBLK = D / 32;
};

template <int D, int MOD>
__global__ __launch_bounds__(256, 1) void bwd_dkdv_kernel(BwdArgs a, int partial) {
  using C = KVCfg<D>;
  constexpr bool kAlibi = MOD & 1;
  constexpr bool kSoftcap = MOD & 2;
  __shared__ __attribute__((aligned(16))) bf16_t lds_q[2 * C::QT];
  __shared__ __attribute__((aligned(16))) bf16_t lds_do[2 * C::QT];
  __shared__ __attribute__((aligned(16))) float lds_lse[2 * C::BM];
  __shared__ __attribute__((aligned(16))) float lds_dl[2 * C::BM];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, c = lane & 31;
  const int nkt = (a.Sk + C::BN - 1) / C::BN;
  const int per = a.Hq * a.B;
  const int kt = blockIdx.x / per;  // key tiles near the start see the most causal rows
  const int rem = blockIdx.x % per;
  const int b = rem / a.Hq;
  int h = rem % a.Hq;
  if ((a.Hq & 7) == 0) h = (h & 7) * (a.Hq >> 3) + (h >> 3);
  const int G = a.Hq / a.Hkv;
  const int kvh = h / G;
  (void)nkt;

  const bf16_t* qp = static_cast<const bf16_t*>(a.q) + b * a.q_sb + h * a.q_sh;
  const bf16_t* dop = static_cast<const bf16_t*>(a.dout) + b * a.do_sb + h * a.do_sh;
  const bf16_t* kp = static_cast<const bf16_t*>(a.k) + b * a.k_sb + kvh * a.k_sh;
  const bf16_t* vp = static_cast<const bf16_t*>(a.v) + b * a.v_sb + kvh * a.v_sh;
  const float* lsep = a.lse + ((int64_t)b * a.Hq + h) * a.Sq;
  const float* dlp = a.delta + ((int64_t)b * a.Hq + h) * a.Sq;

  const int kv0 = kt * C::BN + wave * 32;  // this wave's first key
  const int my_key = kv0 + c;
  const bool k_ok = my_key < a.Sk;

  // K and V rows of this lane's key as B operands (d = 16*ds + 8*g .. +7).
  bf16x8 kf[C::DSTEPS], vf[C::DSTEPS];
#pragma unroll
  for (int ds = 0; ds < C::DSTEPS; ++ds) {
    uint4 kr = make_uint4(0, 0, 0, 0), vr = make_uint4(0, 0, 0, 0);
    if (k_ok) {
      kr = *reinterpret_cast<const uint4*>(kp + (int64_t)my_key * a.k_ss + 16 * ds + 8 * g);
      vr = *reinterpret_cast<const uint4*>(vp + (int64_t)my_key * a.v_ss + 16 * ds + 8 * g);
    }
    kf[ds] = __builtin_bit_cast(bf16x8, kr);
    vf[ds] = __builtin_bit_cast(bf16x8, vr);
  }

  const float scale = a.scale;
  const float scale_abs = fabsf(scale);
  // A negative scale is applied by negating the raw dot product in the
  // exponent (and the gradient's scale keeps its sign).
  const float sgn = scale < 0.0f ? -1.0f : 1.0f;
  const float scale_log2 = scale_abs * kLog2e;
  const float cap_k2 = kSoftcap ? 2.0f * kLog2e * scale_abs / a.softcap : 0.0f;
  const float cap_log2 = a.softcap * kLog2e;
  const float slope_log2 = kAlibi ? a.alibi[b * a.alibi_sb + h] * kLog2e : 0.0f;
  const int delta_pos = a.Sk - a.Sq;

  // Query tiles that meet this key tile: rows i with lo(i) <= last key and
  // hi(i) >= first key of the workgroup's 128 keys.
  const RowWindow win(a.Sq, a.Sk, a.mask.causal, a.mask.wl, a.mask.wr);
  const int c0 = kt * C::BN, c1 = min(a.Sk, c0 + C::BN) - 1;
  int i_lo = 0, i_hi = a.Sq - 1;
  if (win.R != kUnbounded) i_lo = max(i_lo, c0 - delta_pos - win.R);
  if (win.L != kUnbounded) i_hi = min(i_hi, c1 - delta_pos + win.L);
  const int qt_begin = i_lo <= i_hi ? i_lo / C::BM : 0;
  const int qt_end = i_lo <= i_hi ? i_hi / C::BM + 1 : 0;
  const int ntiles = qt_end - qt_begin;

  uint4 qr[C::CPT], dr[C::CPT];
  float lse_r = 0.0f;
  auto load_regs = [&](int qt) {
#pragma unroll
    for (int u = 0; u < C::CPT; ++u) {
      const int chunk = tid + u * C::NT;
      const int row = chunk / (D / 8);
      const int col = (chunk % (D / 8)) * 8;
      const int i = qt * C::BM + row;
      if (i < a.Sq) {
        qr[u] = *reinterpret_cast<const uint4*>(qp + (int64_t)i * a.q_ss + col);
        dr[u] = *reinterpret_cast<const uint4*>(dop + (int64_t)i * a.do_ss + col);
      } else {
        qr[u] = make_uint4(0, 0, 0, 0);
        dr[u] = make_uint4(0, 0, 0, 0);
      }
    }
    if (tid < 2 * C::BM) {
      const int i = qt * C::BM + (tid & (C::BM - 1));
      if (tid < C::BM) {
        const float l = i < a.Sq ? lsep[i] : kNegInf;
        lse_r = l == kNegInf ? kPosInf : l * kLog2e;  // empty rows: P = 0
      } else {
        lse_r = i < a.Sq ? dlp[i] : 0.0f;
      }
    }
  };
  auto store_regs = [&](int buf) {
#pragma unroll
    for (int u = 0; u < C::CPT; ++u) {
      const int chunk = tid + u * C::NT;
      const int row = chunk / (D / 8);
      const int col = (chunk % (D / 8)) * 8;
      *reinterpret_cast<uint4*>(lds_q + buf * C::QT + row * C::QS + col) = qr[u];
      *reinterpret_cast<uint4*>(lds_do + buf * C::QT + row * C::QS + col) = dr[u];
    }
    if (tid < C::BM) lds_lse[buf * C::BM + tid] = lse_r;
    else if (tid < 2 * C::BM) lds_dl[buf * C::BM + tid - C::BM] = lse_r;
  };

  f32x16 dv[C::DBLK], dk[C::DBLK];
#pragma unroll
  for (int db = 0; db < C::DBLK; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      dv[db][r] = 0.0f;
      dk[db][r] = 0.0f;
    }

  if (ntiles > 0) {
    load_regs(qt_begin);
    store_regs(0);
  }
  __syncthreads();

  const int beta = lane >> 4, s16 = lane & 15;
  const int tr_row = 4 * (beta >> 1) + (s16 >> 2);
  const int tr_col = 16 * (beta & 1) + 4 * (s16 & 3);

  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    const int qt = qt_begin + t;
    const bool has_next = t + 1 < ntiles;
    if (has_next) load_regs(qt + 1);

    // Is this (32-query x 32-key) block wholly allowed?  Same interval test
    // as the forward's tile classification, for this wave's 32 keys.
    const TileRange tr_q(win, qt, C::BM, 32);
    const int kt32 = kv0 / 32;
    const bool full = tr_q.full(kt32);
    const bool any = kt32 >= tr_q.kt_begin && kt32 < tr_q.kt_end;

    if (any) {
      const bf16_t* qb = lds_q + buf * C::QT;
      const bf16_t* dob = lds_do + buf * C::QT;
      f32x16 s, dp;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s[r] = 0.0f;
        dp[r] = 0.0f;
      }
#pragma unroll
      for (int ds = 0; ds < C::DSTEPS; ++ds) {
        const bf16x8 qa = *reinterpret_cast<const bf16x8*>(qb + c * C::QS + 16 * ds + 8 * g);
        s = mfma32(qa, kf[ds], s);
        const bf16x8 da = *reinterpret_cast<const bf16x8*>(dob + c * C::QS + 16 * ds + 8 * g);
        dp = mfma32(da, vf[ds], dp);
      }
      // s[r]: query q0 + 8*(r/4) + 4*g + r%4, key my_key.
      const float* lse_t = lds_lse + buf * C::BM;
      const float* dl_t = lds_dl + buf * C::BM;
      const int q0 = qt * C::BM;
      bf16x8 pf[2], sf[2];
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const float4 l4 = *reinterpret_cast<const float4*>(lse_t + 8 * rr + 4 * g);
        const float4 d4 = *reinterpret_cast<const float4*>(dl_t + 8 * rr + 4 * g);
        const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
        const float dvv[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * rr + e;
          const int i = q0 + 8 * rr + 4 * g + e;
          float th = 0.0f;
          const float x = score_x<kAlibi, kSoftcap>(sgn * s[r], scale_log2, cap_k2, cap_log2,
                                                    slope_log2, i + delta_pos - my_key, &th);
          float p = fast_exp2(x - lv[e]);
          if (!full && !mask_ok(a.mask, a.Sq, a.Sk, i, my_key)) p = 0.0f;
          float dsv = p * (dp[r] - dvv[e]);
          if (kSoftcap) dsv *= 1.0f - th * th;
          pf[r >> 3][r & 7] = static_cast<__bf16>(p);
          sf[r >> 3][r & 7] = static_cast<__bf16>(dsv);
        }
      }
      // dV += P^T dO ; dK += dS^T Q   (B operands: transposed tile reads)
#pragma unroll
      for (int db = 0; db < C::DBLK; ++db) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const int off = (16 * ks + tr_row) * C::QS + 32 * db + tr_col;
          const bf16x8 dob_f = cat_frag(lds_read_tr16(dob + off), lds_read_tr16(dob + off + 8 * C::QS));
          dv[db] = mfma32(pf[ks], dob_f, dv[db]);
          const bf16x8 qb_f = cat_frag(lds_read_tr16(qb + off), lds_read_tr16(qb + off + 8 * C::QS));
          dk[db] = mfma32(sf[ks], qb_f, dk[db]);
        }
      }
    }

    if (has_next) store_regs(buf ^ 1);
    __syncthreads();
  }

  // dv[db][r], dk[db][r]: key kv0 + 8*(r/4) + 4*g + r%4, d = 32*db + c.
#pragma unroll
  for (int db = 0; db < C::DBLK; ++db) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = kv0 + 8 * (r >> 2) + 4 * g + (r & 3);
      if (key >= a.Sk) continue;
      const int d = 32 * db + c;
      const float vval = dv[db][r];
      const float kval = dk[db][r] * scale;
      if (partial) {
        // fp32 partials [B, Sk, Hq, D] in the workspace, summed per group later.
        const int64_t idx = (((int64_t)b * a.Sk + key) * a.Hq + h) * D + d;
        a.part_dk[idx] = kval;
        a.part_dv[idx] = vval;
      } else {
        bf16_t* dkp = static_cast<bf16_t*>(a.dk) + b * a.dk_sb + (int64_t)key * a.dk_ss + kvh * a.dk_sh;
        bf16_t* dvp = static_cast<bf16_t*>(a.dv) + b * a.dv_sb + (int64_t)key * a.dv_ss + kvh * a.dv_sh;
        dkp[d] = f32_to_bf16(kval);
        dvp[d] = f32_to_bf16(vval);
      }
    }
  }
}

// Sum the G per-head partials of each kv head in head order -> bf16.
template <int D>
__global__ __launch_bounds__(256) void bwd_group_sum_kernel(BwdArgs a) {
  const int64_t n = (int64_t)a.B * a.Sk * a.Hkv * D;
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= n) return;
  const int d = static_cast<int>(t % D);
  const int g = static_cast<int>((t / D) % a.Hkv);
  const int64_t bj = t / ((int64_t)D * a.Hkv);
  const int j = static_cast<int>(bj % a.Sk);
  const int b = static_cast<int>(bj / a.Sk);
  const int G = a.Hq / a.Hkv;
  const int64_t base = (((int64_t)b * a.Sk + j) * a.Hq + (int64_t)g * G) * D + d;
  float sk = 0.0f, sv = 0.0f;
  for (int x = 0; x < G; ++x) {
    sk += a.part_dk[base + (int64_t)x * D];
    sv += a.part_dv[base + (int64_t)x * D];
  }
  bf16_t* dkp = static_cast<bf16_t*>(a.dk) + b * a.dk_sb + (int64_t)j * a.dk_ss + g * a.dk_sh;
  bf16_t* dvp = static_cast<bf16_t*>(a.dv) + b * a.dv_sb + (int64_t)j * a.dv_ss + g * a.dv_sh;
  dkp[d] = f32_to_bf16(sk);
  dvp[d] = f32_to_bf16(sv);
}

// ---------------------------------------------------------------------------
// 3. dQ

template <int D>
struct QCfg {
  static constexpr int BM = 128;           // query rows per workgroup (4 waves x 32)
  static constexpr int BN = 64;            // keys per streamed tile
  static constexpr int NT = 256;
  static constexpr int KS = D + 8;         // K tile stride (row reads and transposed reads)
  static constexpr int VS = D + 8;         // V tile stride (row reads)
  static constexpr int KT = BN * KS;
  static constexpr int VT = BN * VS;
  static constexpr int CPT = BN * D / 8 / NT;
  static constexpr int DSTEPS = D / 16;
  static constexpr int DBLK = D / 32;
};

template <int D, int MOD>
__global__ __launch_bounds__(256, 1) void bwd_dq_kernel(BwdArgs a) {
  using C = QCfg<D>;
  constexpr bool kAlibi = MOD & 1;
  constexpr bool kSoftcap = MOD & 2;
  __shared__ __attribute__((aligned(16))) bf16_t lds_k[2 * C::KT];
  __shared__ __attribute__((aligned(16))) bf16_t lds_v[2 * C::VT];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, c = lane & 31;
  const int nqt = (a.Sq + C::BM - 1) / C::BM;
  const int per = a.Hq * a.B;
  const int qt = nqt - 1 - blockIdx.x / per;
  const int rem = blockIdx.x % per;
  const int b = rem / a.Hq;
  int h = rem % a.Hq;
  if ((a.Hq & 7) == 0) h = (h & 7) * (a.Hq >> 3) + (h >> 3);
  const int G = a.Hq / a.Hkv;
  const int kvh = h / G;

  const bf16_t* qp = static_cast<const bf16_t*>(a.q) + b * a.q_sb + h * a.q_sh;
  const bf16_t* dop = static_cast<const bf16_t*>(a.dout) + b * a.do_sb + h * a.do_sh;
  const bf16_t* kp = static_cast<const bf16_t*>(a.k) + b * a.k_sb + kvh * a.k_sh;
  const bf16_t* vp = static_cast<const bf16_t*>(a.v) + b * a.v_sb + kvh * a.v_sh;

  const int my_q = qt * C::BM + wave * 32 + c;
  const bool q_ok = my_q < a.Sq;
  bf16x8 qf[C::DSTEPS], df[C::DSTEPS];
#pragma unroll
  for (int ds = 0; ds < C::DSTEPS; ++ds) {
    uint4 r1 = make_uint4(0, 0, 0, 0), r2 = make_uint4(0, 0, 0, 0);
    if (q_ok) {
      r1 = *reinterpret_cast<const uint4*>(qp + (int64_t)my_q * a.q_ss + 16 * ds + 8 * g);
      r2 = *reinterpret_cast<const uint4*>(dop + (int64_t)my_q * a.do_ss + 16 * ds + 8 * g);
    }
    qf[ds] = __builtin_bit_cast(bf16x8, r1);
    df[ds] = __builtin_bit_cast(bf16x8, r2);
  }
  const float scale = a.scale;
  const float scale_abs = fabsf(scale);
  const float sgn = scale < 0.0f ? -1.0f : 1.0f;
  const float scale_log2 = scale_abs * kLog2e;
  const float cap_k2 = kSoftcap ? 2.0f * kLog2e * scale_abs / a.softcap : 0.0f;
  const float cap_log2 = a.softcap * kLog2e;
  const float slope_log2 = kAlibi ? a.alibi[b * a.alibi_sb + h] * kLog2e : 0.0f;
  const int delta_pos = a.Sk - a.Sq;
  float lse2 = kPosInf, dl = 0.0f;
  if (q_ok) {
    const float l = a.lse[((int64_t)b * a.Hq + h) * a.Sq + my_q];
    lse2 = l == kNegInf ? kPosInf : l * kLog2e;
    dl = a.delta[((int64_t)b * a.Hq + h) * a.Sq + my_q];
  }

  const RowWindow win(a.Sq, a.Sk, a.mask.causal, a.mask.wl, a.mask.wr);
  const TileRange range(win, qt, C::BM, C::BN);
  const int ntiles = range.kt_end - range.kt_begin;

  uint4 kr[C::CPT], vr[C::CPT];
  auto load_regs = [&](int kt) {
#pragma unroll
    for (int u = 0; u < C::CPT; ++u) {
      const int chunk = tid + u * C::NT;
      const int row = chunk / (D / 8);
      const int col = (chunk % (D / 8)) * 8;
      const int key = kt * C::BN + row;
      if (key < a.Sk) {
        kr[u] = *reinterpret_cast<const uint4*>(kp + (int64_t)key * a.k_ss + col);
        vr[u] = *reinterpret_cast<const uint4*>(vp + (int64_t)key * a.v_ss + col);
      } else {
        kr[u] = make_uint4(0, 0, 0, 0);
        vr[u] = make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto store_regs = [&](int buf) {
#pragma unroll
    for (int u = 0; u < C::CPT; ++u) {
      const int chunk = tid + u * C::NT;
      const int row = chunk / (D / 8);
      const int col = (chunk % (D / 8)) * 8;
      *reinterpret_cast<uint4*>(lds_k + buf * C::KT + row * C::KS + col) = kr[u];
      *reinterpret_cast<uint4*>(lds_v + buf * C::VT + row * C::VS + col) = vr[u];
    }
  };

  f32x16 dq[C::DBLK];
#pragma unroll
  for (int db = 0; db < C::DBLK; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) dq[db][r] = 0.0f;

  if (ntiles > 0) {
    load_regs(range.kt_begin);
    store_regs(0);
  }
  __syncthreads();

  const int beta = lane >> 4, s16 = lane & 15;
  const int tr_row = 4 * (beta >> 1) + (s16 >> 2);
  const int tr_col = 16 * (beta & 1) + 4 * (s16 & 3);

  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    const int kt = range.kt_begin + t;
    const bool full = range.full(kt);
    const bool has_next = t + 1 < ntiles;
    if (has_next) load_regs(kt + 1);

    const bf16_t* kb = lds_k + buf * C::KT;
    const bf16_t* vb = lds_v + buf * C::VT;
    f32x16 s[2], dp[2];
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s[h2][r] = 0.0f;
        dp[h2][r] = 0.0f;
      }
#pragma unroll
    for (int ds = 0; ds < C::DSTEPS; ++ds) {
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const bf16x8 ka = *reinterpret_cast<const bf16x8*>(kb + (32 * h2 + c) * C::KS + 16 * ds + 8 * g);
        s[h2] = mfma32(ka, qf[ds], s[h2]);
        const bf16x8 va = *reinterpret_cast<const bf16x8*>(vb + (32 * h2 + c) * C::VS + 16 * ds + 8 * g);
        dp[h2] = mfma32(va, df[ds], dp[h2]);
      }
    }
    // s[h2][r]: key kt*BN + 32*h2 + 8*(r/4) + 4*g + r%4, query my_q.
    bf16x8 sf[2][2];
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int j = kt * C::BN + 32 * h2 + 8 * (r >> 2) + 4 * g + (r & 3);
        float th = 0.0f;
        const float x = score_x<kAlibi, kSoftcap>(sgn * s[h2][r], scale_log2, cap_k2, cap_log2,
                                                  slope_log2, my_q + delta_pos - j, &th);
        float p = fast_exp2(x - lse2);
        if (!full && !mask_ok(a.mask, a.Sq, a.Sk, my_q, j)) p = 0.0f;
        float dsv = p * (dp[h2][r] - dl);
        if (kSoftcap) dsv *= 1.0f - th * th;
        sf[h2][r >> 3][r & 7] = static_cast<__bf16>(dsv);
      }
    }
    // dQ^T += K^T dS^T
#pragma unroll
    for (int db = 0; db < C::DBLK; ++db) {
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const bf16_t* p0 = kb + (32 * h2 + 16 * ks + tr_row) * C::KS + 32 * db + tr_col;
          const bf16x8 ka = cat_frag(lds_read_tr16(p0), lds_read_tr16(p0 + 8 * C::KS));
          dq[db] = mfma32(ka, sf[h2][ks], dq[db]);
        }
      }
    }

    if (has_next) store_regs(buf ^ 1);
    __syncthreads();
  }

  if (q_ok) {
    bf16_t* out = static_cast<bf16_t*>(a.dq) + b * a.dq_sb + (int64_t)my_q * a.dq_ss + h * a.dq_sh;
#pragma unroll
    for (int db = 0; db < C::DBLK; ++db) {
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int d0 = 32 * db + 8 * rr + 4 * g;
        uint2 packed;
        packed.x = f32_to_bf16(dq[db][4 * rr] * scale) | (uint32_t)f32_to_bf16(dq[db][4 * rr + 1] * scale) << 16;
        packed.y = f32_to_bf16(dq[db][4 * rr + 2] * scale) | (uint32_t)f32_to_bf16(dq[db][4 * rr + 3] * scale) << 16;
        *reinterpret_cast<uint2*>(out + d0) = packed;
      }
    }
  }
}

template <int D, int MOD>
hipError_t launch_mod(const BwdArgs& a, int stages, hipStream_t s) {
  const int G = a.Hq / a.Hkv;
  const int partial = G > 1 ? 1 : 0;
  const int nkt = (a.Sk + KVCfg<D>::BN - 1) / KVCfg<D>::BN;
  if ((stages & 2) && nkt > 0) {
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, MOD>), dim3(nkt * a.Hq * a.B), dim3(256), 0, s, a, partial);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if ((stages & 4) && partial && a.Sk > 0) {
    const int64_t n = (int64_t)a.B * a.Sk * a.Hkv * D;
    hipLaunchKernelGGL(bwd_group_sum_kernel<D>, dim3((n + 255) / 256), dim3(256), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int nqt = (a.Sq + QCfg<D>::BM - 1) / QCfg<D>::BM;
  if (!(stages & 8) || nqt == 0) return hipSuccess;
  hipLaunchKernelGGL((bwd_dq_kernel<D, MOD>), dim3(nqt * a.Hq * a.B), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const BwdArgs& a, int stages, hipStream_t s) {
  const int64_t rows = (int64_t)a.B * a.Sq * a.Hq;
  constexpr int LPR = D / 8;
  if ((stages & 1) && rows > 0) {
    hipLaunchKernelGGL(bwd_delta_kernel<D>, dim3((rows * LPR + 255) / 256), dim3(256), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int mod = (a.alibi != nullptr ? 1 : 0) | (a.softcap > 0.0f ? 2 : 0);
  switch (mod) {
    case 0: return launch_mod<D, 0>(a, stages, s);
    case 1: return launch_mod<D, 1>(a, stages, s);
    case 2: return launch_mod<D, 2>(a, stages, s);
    default: return launch_mod<D, 3>(a, stages, s);
  }
}

}  // namespace

size_t bwd_workspace_bytes(int B, int Hq, int Hkv, int Sq, int Sk, int D) {
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  size_t n = up((size_t)B * Hq * Sq * sizeof(float));
  if (Hkv > 0 && Hq / Hkv > 1) n += 2 * up((size_t)B * Sk * Hq * D * sizeof(float));
  return n;
}

hipError_t launch_bwd_bf16(const BwdArgs& a, int stage_mask, hipStream_t s) {
  if (a.B == 0 || a.Hq == 0) return hipSuccess;
  if (a.D == 64) return launch_d<64>(a, stage_mask, s);
  return launch_d<128>(a, stage_mask, s);
}

}  // namespace attn
