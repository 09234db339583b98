// Backward attention from the saved log-sum-exp, bf16 or fp16 (gfx950).
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
// Kernels of the deterministic schedule, no atomics (every output element is
// summed in a fixed order, so results are bitwise repeatable), in launch
// order: dQ (which also forms Delta_i = <dO_i, O_i> in fp32 and the LSE in
// exp2 units for its rows), dK/dV, and for GQA the group sum.  The atomic-dQ
// schedule runs a separate Delta pass (1) first.
//  1. preprocess (atomic-dQ schedule): Delta and lse2, zeroed dQ accumulator.
//  2. dK/dV: a workgroup owns 128 keys of one (batch, query head); each wave
//     keeps its 32 keys of K and V in registers as MFMA operands and streams
//     32-query tiles of Q and dO through LDS.  S = Q K^T puts one key per
//     lane, so P and dS (rounded to bf16) are directly the A operands of
//     dV += P^T dO and dK += dS^T Q, whose B operands are transposed LDS
//     reads of the dO and Q tiles.  At D = 128 the deterministic schedule
//     splits each 32-key block over two waves instead (2b): one holds K and
//     produces P and dV, the other holds V and produces dS and dK, which
//     halves the registers per wave so that two waves share each SIMD.
//     With grouped-query heads each query head writes an fp32 partial and a
//     reduction kernel sums the group in head order; with one query head per
//     kv head the result is written directly.
//  3. dQ: the forward's layout -- a workgroup owns 128 query rows, Q and dO
//     stay in registers, K and V tiles stream through LDS; S^T = K Q^T and
//     dP^T = V dO^T give one query per lane, and dQ^T += K^T dS^T uses
//     transposed reads of the K tile.  Each lane holds half of its row's dO,
//     so Delta is its half of <dO, O> plus the partner lane's.

#include <type_traits>

#include "common.h"
#include "internal.h"

namespace attn {
namespace {

constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kPosInf = __builtin_huge_valf();

// ---------------------------------------------------------------------------
// 1. Delta = rowsum(dO * O), one 16-lane group per (b, i, h) row; the same
//    pass stores the LSE in exp2 units for the dK/dV kernel.

template <typename T, int D>
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
      acc = __builtin_fmaf(T::to_f32(ow[e] & 0xffffu), T::to_f32(dw[e] & 0xffffu), acc);
      acc = __builtin_fmaf(T::to_f32(ow[e] >> 16), T::to_f32(dw[e] >> 16), acc);
    }
  }
#pragma unroll
  for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
  if (a.dq_acc != nullptr && row < rows) {
    // the non-deterministic dQ accumulator of this row starts at zero
    float4* z = reinterpret_cast<float4*>(a.dq_acc + row * D + part * 8);
    z[0] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    z[1] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  }
  if (row < rows && part == 0) {
    const int64_t idx = ((int64_t)b * a.Hq + h) * a.Sq + i;
    a.delta[idx] = acc;
    const float l = a.lse[idx];
    a.lse2[idx] = l == kNegInf ? kPosInf : l * kLog2e;  // empty rows: P = 0
  }
}

struct BwdCtx {
  float scale_log2;   // scale * log2(e) (signed)
  float slope_log2;   // ALiBi slope * log2(e)
  float cap_k2;       // 2 log2(e) scale / softcap (signed)
  float cap_log2;     // softcap * log2(e)
  int delta_pos;      // Sk - Sq
};

__device__ __forceinline__ BwdCtx make_ctx(const BwdArgs& a, int b, int h, bool alibi, bool softcap) {
  BwdCtx cx;
  cx.scale_log2 = a.scale * kLog2e;
  cx.slope_log2 = alibi ? a.alibi[b * a.alibi_sb + h] * kLog2e : 0.0f;
  cx.cap_k2 = softcap ? 2.0f * kLog2e * a.scale / a.softcap : 0.0f;
  cx.cap_log2 = a.softcap * kLog2e;
  cx.delta_pos = a.Sk - a.Sq;
  return cx;
}

// exp2-domain score minus the row's lse2 for raw dot product s; *th gets
// tanh of the capped score (softcap only).  dist = query position - key.
template <bool kAlibi, bool kSoftcap>
__device__ __forceinline__ float score_minus(float s, float lse2, const BwdCtx& cx, int dist, float* th) {
  if (!kAlibi && !kSoftcap) return __builtin_fmaf(s, cx.scale_log2, -lse2);
  float x;
  if (kSoftcap) {
    const float ex = fast_exp2(s * cx.cap_k2);
    *th = 1.0f - 2.0f * fast_rcp(ex + 1.0f);
    x = cx.cap_log2 * *th;
  } else {
    x = s * cx.scale_log2;
  }
  if (kAlibi) x = __builtin_fmaf(-cx.slope_log2, fabsf(static_cast<float>(dist)), x);
  return x - lse2;
}

// Key offset (within a 64-row tile, relative to 4*g) of accumulator
// register r of 32-row block kb: rows 8*(r/4) + r%4 of a 32x32 MFMA result.
__device__ __forceinline__ constexpr int roff(int kb, int r) { return 32 * kb + 8 * (r >> 2) + (r & 3); }

// Transposed-read address (bytes) inside a TileLayout<D> image for the
// 16-row step kk and 32-column block db: rows 16*kk + tr_row (and +8),
// columns 32*db + tr_col .. +3 (see lds_read_tr16).
template <typename T, int D>
__device__ __forceinline__ typename T::vec8 tr_frag(const char* tile, int kk, int db, int lane) {
  using L = TileLayout<D>;
  const int beta = lane >> 4, s16 = lane & 15;
  const int row = 16 * kk + 4 * (beta >> 1) + (s16 >> 2);
  const int chunk = 4 * db + 2 * (beta & 1) + ((s16 & 3) >> 1);
  const int half = 8 * (s16 & 1);
  const char* p0 = tile + L::off(row, chunk) + half;
  const char* p1 = tile + L::off(row + 8, chunk) + half;
  return cat_frag<typename T::vec8>(lds_read_tr16(reinterpret_cast<const bf16_t*>(p0)),
                  lds_read_tr16(reinterpret_cast<const bf16_t*>(p1)));
}

// A-operand row read (16 bytes) of row `row`, d = 16*ds + 8*g .. +7.
template <typename T, int D>
__device__ __forceinline__ typename T::vec8 row_frag(const char* tile, int row, int ds, int g) {
  return *reinterpret_cast<const typename T::vec8*>(tile + TileLayout<D>::off(row, 2 * ds + g));
}

// ---------------------------------------------------------------------------
// 2. dK / dV

template <int D>
struct KVCfg {
  static constexpr int BN = 128;           // keys per workgroup (4 waves x 32)
  static constexpr int BM = 64;            // queries per streamed tile
  using L = TileLayout<D>;
  static constexpr int TB = L::BYTES;
  static constexpr int DSTEPS = D / 16;
  static constexpr int DBLK = D / 32;
};

// Stores this lane's dS (key row key_row, 64 query columns) into a
// TileLayout<64> image of dS^T for the dQ product.
template <typename T>
__device__ __forceinline__ void store_ds(char* ds_lds, const typename T::vec8 (&sf)[2][2], int key_row, int g) {
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const uint4 w = __builtin_bit_cast(uint4, sf[qb][m >> 1]);
      const uint2 h = (m & 1) ? make_uint2(w.z, w.w) : make_uint2(w.x, w.y);
      *reinterpret_cast<uint2*>(ds_lds + TileLayout<64>::off(key_row, 4 * qb + m) + 8 * g) = h;
    }
}

// One 64-query tile against this wave's 32 keys, first half: S = Q K^T and
// dP = dO V^T give one key per lane (queries along the accumulator
// registers); P and dS rounded to bf16 come out as pf / sf, which are the A
// operands of dV += P^T dO and dK += dS^T Q (dkdv_accum).
template <typename T, int D, int MOD>
__device__ __forceinline__ void dkdv_scores(const char* qt_lds, const char* dot_lds, const float* lse_t,
                                            const float* dl_t, const typename T::vec8 (&kf)[D / 16],
                                            const typename T::vec8 (&vf)[D / 16], const BwdCtx& cx, int q0,
                                            int my_key, bool masked, int rows_first, int rows_count,
                                            const int* docq_t, bool has_doc, int my_doc,
                                            typename T::vec8 (&pf)[2][2], typename T::vec8 (&sf)[2][2], int lane) {
  using C = KVCfg<D>;
  constexpr bool kAlibi = MOD & 1;
  constexpr bool kSoftcap = MOD & 2;
  const int g = lane >> 5, c = lane & 31;

  f32x16 s[2], dp[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s[qb][r] = 0.0f;
      dp[qb][r] = 0.0f;
    }
#pragma unroll
  for (int ds = 0; ds < C::DSTEPS; ++ds) {
    typename T::vec8 qa[2], da[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      qa[qb] = row_frag<T, D>(qt_lds, 32 * qb + c, ds, g);
      da[qb] = row_frag<T, D>(dot_lds, 32 * qb + c, ds, g);
    }
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      s[qb] = mfma32(qa[qb], kf[ds], s[qb]);
      dp[qb] = mfma32(da[qb], vf[ds], dp[qb]);
    }
  }

  // P = exp2(x - lse2) and dS = P (dP - Delta) [* (1 - tanh^2)], in place.
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const float4 l4 = *reinterpret_cast<const float4*>(lse_t + 32 * qb + 8 * rr + 4 * g);
      const float4 d4 = *reinterpret_cast<const float4*>(dl_t + 32 * qb + 8 * rr + 4 * g);
      const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
      const float dlv[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * rr + e;
        float th = 0.0f;
        const int i = q0 + roff(qb, r) + 4 * g;
        const float p = fast_exp2(score_minus<kAlibi, kSoftcap>(s[qb][r], lv[e], cx, i + cx.delta_pos - my_key, &th));
        float dsv = p * (dp[qb][r] - dlv[e]);
        if (kSoftcap) dsv *= 1.0f - th * th;
        s[qb][r] = p;
        dp[qb][r] = dsv;
      }
    }
  if (masked) {
    // rows [rows_first, rows_first + rows_count) may see this key (window and
    // bounds); with a document mask the row's document must be the key's.
    const uint32_t span = static_cast<uint32_t>(rows_count);
    const int ib = q0 + 4 * g - rows_first;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        // (document ids read whatever has_doc says, and ignored without a
        // document mask: a test guarded by has_doc became a branch per element)
        const int4 d4 = *reinterpret_cast<const int4*>(docq_t + 32 * qb + 8 * rr + 4 * g);
        const int dv4[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * rr + e;
          const bool ok = (static_cast<uint32_t>(ib + roff(qb, r)) < span) & (!has_doc | (dv4[e] == my_doc));
          s[qb][r] = ok ? s[qb][r] : 0.0f;
          dp[qb][r] = ok ? dp[qb][r] : 0.0f;
        }
      }
  }
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      pf[qb][r >> 3][r & 7] = static_cast<typename T::elem>(s[qb][r]);
      sf[qb][r >> 3][r & 7] = static_cast<typename T::elem>(dp[qb][r]);
    }
}

// Second half: dV += P^T dO ; dK += dS^T Q (the D/32 output blocks are
// independent), with transposed reads of the dO and Q tiles.
template <typename T, int D>
__device__ __forceinline__ void dkdv_accum(const char* qt_lds, const char* dot_lds, const typename T::vec8 (&pf)[2][2],
                                           const typename T::vec8 (&sf)[2][2], f32x16 (&dk)[D / 32],
                                           f32x16 (&dv)[D / 32], int lane) {
  using C = KVCfg<D>;
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    typename T::vec8 fo[C::DBLK], fq[C::DBLK];
#pragma unroll
    for (int db = 0; db < C::DBLK; ++db) {
      fo[db] = tr_frag<T, D>(dot_lds, kk, db, lane);
      fq[db] = tr_frag<T, D>(qt_lds, kk, db, lane);
    }
#pragma unroll
    for (int db = 0; db < C::DBLK; ++db) {
      dv[db] = mfma32(pf[kk >> 1][kk & 1], fo[db], dv[db]);
      dk[db] = mfma32(sf[kk >> 1][kk & 1], fq[db], dk[db]);
    }
  }
}

template <typename T, int D, int MOD, bool kDq>
__global__ __launch_bounds__(256, 1) void bwd_dkdv_kernel(BwdArgs a, int partial) {
  using C = KVCfg<D>;
  // Three buffers (one workgroup per CU leaves the LDS room): the copies of
  // tiles t+1 and t+2 are in flight while tile t is processed.  Distinct LDS
  // objects per buffer let alias analysis see that a copy never targets the
  // buffer being read, so no wait for it is placed before the reads.
  __shared__ __attribute__((aligned(16))) char lq0[C::TB];
  __shared__ __attribute__((aligned(16))) char lq1[C::TB];
  __shared__ __attribute__((aligned(16))) char lq2[C::TB];
  __shared__ __attribute__((aligned(16))) char ld0[C::TB];
  __shared__ __attribute__((aligned(16))) char ld1[C::TB];
  __shared__ __attribute__((aligned(16))) char ld2[C::TB];
  __shared__ __attribute__((aligned(16))) float ll0[C::BM];
  __shared__ __attribute__((aligned(16))) float ll1[C::BM];
  __shared__ __attribute__((aligned(16))) float ll2[C::BM];
  __shared__ __attribute__((aligned(16))) float lg0[C::BM];
  __shared__ __attribute__((aligned(16))) float lg1[C::BM];
  __shared__ __attribute__((aligned(16))) float lg2[C::BM];
  __shared__ __attribute__((aligned(16))) int lz0[C::BM];
  __shared__ __attribute__((aligned(16))) int lz1[C::BM];
  __shared__ __attribute__((aligned(16))) int lz2[C::BM];
  // dQ in this kernel (non-deterministic variant): the workgroup's 128 K rows
  // and each tile's dS^T (128 keys x 64 queries) in LDS.
  __shared__ __attribute__((aligned(16))) char lkk[kDq ? 2 * C::TB : 16];
  __shared__ __attribute__((aligned(16))) char lds_s[kDq ? 2 * TileLayout<64>::BYTES : 16];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, c = lane & 31;
  const int per = a.Hq * a.B;
  const int kt = blockIdx.x / per;  // key tiles near the start see the most causal rows
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
  const float* lsep = a.lse2 + ((int64_t)b * a.Hq + h) * a.Sq;
  const float* dlp = a.delta + ((int64_t)b * a.Hq + h) * a.Sq;

  const int kv0 = kt * C::BN + wave * 32;  // this wave's first key
  const int my_key = kv0 + c;
  const bool k_ok = my_key < a.Sk;

  // K and V rows of this lane's key as B operands (d = 16*ds + 8*g .. +7).
  typename T::vec8 kf[C::DSTEPS], vf[C::DSTEPS];
  // (Guarded loads here: issuing all of them unconditionally, as the dQ
  // kernel does, measured slower in this register-bound kernel.)
#pragma unroll
  for (int ds = 0; ds < C::DSTEPS; ++ds) {
    uint4 kr = make_uint4(0, 0, 0, 0), vr = make_uint4(0, 0, 0, 0);
    if (k_ok) {
      kr = *reinterpret_cast<const uint4*>(kp + (int64_t)my_key * a.k_ss + 16 * ds + 8 * g);
      vr = *reinterpret_cast<const uint4*>(vp + (int64_t)my_key * a.v_ss + 16 * ds + 8 * g);
    }
    kf[ds] = __builtin_bit_cast(typename T::vec8, kr);
    vf[ds] = __builtin_bit_cast(typename T::vec8, vr);
  }
  const BwdCtx cx = make_ctx(a, b, h, MOD & 1, MOD & 2);

  // Query tiles that meet the workgroup's keys.  Dense: rows i with
  // lo(i) <= last key and hi(i) >= first key, one interval.  Block-sparse:
  // the FULL then the PARTIAL query blocks (128 rows = two tiles) listed for
  // the mask's key block holding these keys.
  const RowWindow win(a.Sq, a.Sk, a.mask.causal, a.mask.wl, a.mask.wr);
  constexpr bool sparse = (MOD & 4) != 0;  // block-mask lists (else the dense band)
  int qt_begin = 0, ntiles = 0, n_full_blk = 0;
  const int32_t* qi_full = nullptr;
  const int32_t* qi_part = nullptr;
  if (sparse) {
    const int u = b * a.tiles.nK + (kt * C::BN) / a.tiles.block_n;
    n_full_blk = a.tiles.q_num_full[u];
    ntiles = 2 * (n_full_blk + a.tiles.q_num_partial[u]);
    qi_full = a.tiles.q_idx_full + (int64_t)u * a.tiles.nQ;
    qi_part = a.tiles.q_idx_partial + (int64_t)u * a.tiles.nQ;
  } else {
    const int c0 = kt * C::BN, c1 = min(a.Sk, c0 + C::BN) - 1;
    int i_lo = 0, i_hi = a.Sq - 1;
    if (win.R != kUnbounded) i_lo = max(i_lo, c0 - cx.delta_pos - win.R);
    if (win.L != kUnbounded) i_hi = min(i_hi, c1 - cx.delta_pos + win.L);
    qt_begin = i_lo <= i_hi ? i_lo / C::BM : 0;
    ntiles = i_lo <= i_hi ? i_hi / C::BM + 1 - qt_begin : 0;
  }
  auto qt_of = [&](int t) __attribute__((always_inline)) -> int {
    if (!sparse) return qt_begin + t;
    const int blk = t >> 1;
    return 2 * (blk < n_full_blk ? qi_full[blk] : qi_part[blk - n_full_blk]) + (t & 1);
  };
  int rows_first, rows_count;
  win.key_rows(my_key, &rows_first, &rows_count);
  const bool has_doc = sparse && a.mask.doc_q != nullptr;  // document masks come with block masks
  const int my_doc = has_doc && k_ok ? a.mask.doc_k[(int64_t)b * a.Sk + my_key] : 0;
  const int32_t* docq = has_doc ? a.mask.doc_q + (int64_t)b * a.Sq : nullptr;

  // Every wave issues the same number of memory operations per tile (its
  // share of the Q and dO rows, plus one 64-entry row: lse2 for wave 0, Delta
  // for waves 1 and 3, the rows' document ids for wave 2 when a document mask
  // is given, else lse2 again), so one counter value means "all but the
  // newest tile have landed".
  constexpr int kOpsPerTile = 2 * (64 / C::L::RG / 4) + 1;
  auto load_tile = [&](int qt, auto buf_tag) __attribute__((always_inline)) {
    constexpr int BUF = decltype(buf_tag)::value;
    char* qd = BUF == 0 ? lq0 : (BUF == 1 ? lq1 : lq2);
    char* dd = BUF == 0 ? ld0 : (BUF == 1 ? ld1 : ld2);
    tile_dma<D>(reinterpret_cast<bf16_t*>(qd), qp, a.q_ss, qt * C::BM, a.Sq, wave, lane);
    tile_dma<D>(reinterpret_cast<bf16_t*>(dd), dop, a.do_ss, qt * C::BM, a.Sq, wave, lane);
    // rows past Sq repeat the last row; they are masked on partial tiles
    const int i = min(qt * C::BM + lane, a.Sq - 1);
    const void* src;
    void* dst;
    if (wave & 1) {
      src = dlp + i;
      dst = BUF == 0 ? lg0 : (BUF == 1 ? lg1 : lg2);
    } else if (wave == 2 && has_doc) {
      src = docq + i;
      dst = BUF == 0 ? lz0 : (BUF == 1 ? lz1 : lz2);
    } else {
      src = lsep + i;
      dst = BUF == 0 ? ll0 : (BUF == 1 ? ll1 : ll2);
    }
    __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)dst, 4, 0, 0);
  };
  auto wait_older = [&](bool newest_in_flight) __attribute__((always_inline)) {
    if (newest_in_flight) {
      if constexpr (kOpsPerTile == 9) asm volatile("s_waitcnt vmcnt(9)" ::: "memory");
      else asm volatile("s_waitcnt vmcnt(5)" ::: "memory");
    } else {
      wait_dma();
    }
  };
  static_assert(kOpsPerTile == 9 || kOpsPerTile == 5, "ops per tile");
  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  using B2 = std::integral_constant<int, 2>;

  f32x16 dv[C::DBLK], dk[C::DBLK];
#pragma unroll
  for (int db = 0; db < C::DBLK; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      dv[db][r] = 0.0f;
      dk[db][r] = 0.0f;
    }

  if constexpr (kDq) {
    tile_dma<D>(reinterpret_cast<bf16_t*>(lkk), kp, a.k_ss, kt * C::BN, a.Sk, wave, lane);
    tile_dma<D>(reinterpret_cast<bf16_t*>(lkk + C::TB), kp, a.k_ss, kt * C::BN + 64, a.Sk, wave, lane);
  }
  if (ntiles > 0) load_tile(qt_of(0), B0{});
  if (ntiles > 1) load_tile(qt_of(1), B1{});
  wait_older(ntiles > 1);  // also covers the K copies, issued first
  __syncthreads();

  // dQ rows of tile qt += dS K over the workgroup's 128 keys: wave w owns
  // query block w % 2 and D/64 of the 32-column blocks; fp32 atomic adds
  // into the accumulator (rows past Sq skipped; their dS is zero anyway).
  float* dq_row0 = kDq ? a.dq_acc + ((int64_t)b * a.Sq * a.Hq + h) * D : nullptr;
  auto dq_update = [&](int qt) __attribute__((always_inline)) {
    constexpr int NDB = C::DBLK / 2 > 0 ? C::DBLK / 2 : 1;
    const int qblk = wave & 1;
    f32x16 acc[NDB];
#pragma unroll
    for (int j = 0; j < NDB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[j][r] = 0.0f;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const typename T::vec8 af = tr_frag<T, 64>(lds_s, kk, qblk, lane);
#pragma unroll
      for (int j = 0; j < NDB; ++j)
        acc[j] = mfma32(af, tr_frag<T, D>(lkk, kk, NDB * (wave >> 1) + j, lane), acc[j]);
    }
#pragma unroll
    for (int j = 0; j < NDB; ++j) {
      const int d = 32 * (NDB * (wave >> 1) + j) + c;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int i = qt * C::BM + 32 * qblk + 8 * (r >> 2) + 4 * g + (r & 3);
        if (i < a.Sq) unsafeAtomicAdd(dq_row0 + (int64_t)i * a.Hq * D + d, acc[j][r]);
      }
    }
  };

  const int kw = kv0 / 32;  // this wave's 32-key block index
  auto step = [&](int t, auto buf_tag) __attribute__((always_inline)) {
    constexpr int BUF = decltype(buf_tag)::value;
    using AHEAD = std::integral_constant<int, (BUF + 2) % 3>;
    const int qt = qt_of(t);
    const bool ahead = t + 2 < ntiles;
    if (ahead) load_tile(qt_of(t + 2), AHEAD{});
    bool run, masked;
    if (sparse) {
      run = true;
      masked = (t >> 1) >= n_full_blk;
    } else {
      const TileRange trq(win, qt, C::BM, 32);
      run = kw >= trq.kt_begin && kw < trq.kt_end;
      masked = !trq.full(kw);
    }
    const char* qbuf = BUF == 0 ? lq0 : (BUF == 1 ? lq1 : lq2);
    const char* dbuf = BUF == 0 ? ld0 : (BUF == 1 ? ld1 : ld2);
    typename T::vec8 pf[2][2], sf[2][2];
    auto scores = [&]() __attribute__((always_inline)) {
      dkdv_scores<T, D, MOD>(qbuf, dbuf, BUF == 0 ? ll0 : (BUF == 1 ? ll1 : ll2),
                          BUF == 0 ? lg0 : (BUF == 1 ? lg1 : lg2), kf, vf, cx, qt * C::BM, my_key, masked,
                          rows_first, rows_count, BUF == 0 ? lz0 : (BUF == 1 ? lz1 : lz2), has_doc, my_doc,
                          pf, sf, lane);
    };
    if constexpr (!kDq) {
      if (run) {
        scores();
        dkdv_accum<T, D>(qbuf, dbuf, pf, sf, dk, dv, lane);
      }
    } else {
      if (run) scores();
      if (!run) {
#pragma unroll
        for (int x = 0; x < 2; ++x)
#pragma unroll
          for (int y = 0; y < 2; ++y)
#pragma unroll
            for (int e = 0; e < 8; ++e) sf[x][y][e] = static_cast<typename T::elem>(0.0f);
      }
      __syncthreads();  // every wave has finished reading the previous dS^T
      store_ds<T>(lds_s, sf, 32 * wave + c, g);
      if (run) dkdv_accum<T, D>(qbuf, dbuf, pf, sf, dk, dv, lane);
    }
    wait_older(ahead);  // tile t + 1 has landed
    __syncthreads();    // ... for every wave; with kDq also: dS^T is complete
    if constexpr (kDq) dq_update(qt);
  };
  int t = 0;
  for (; t + 2 < ntiles; t += 3) {
    step(t, B0{});
    step(t + 1, B1{});
    step(t + 2, B2{});
  }
  if (t < ntiles) step(t++, B0{});
  if (t < ntiles) step(t++, B1{});

  // dv[db][r], dk[db][r]: key kv0 + 8*(r/4) + 4*g + r%4, d = 32*db + c.  One
  // base address per lane and output, per-element offsets in multiples of the
  // key stride, the key bound tested only when the wave's keys run past Sk.
  const float scale = a.scale;
  const int key0 = kv0 + 4 * g;
  const bool whole = kv0 + 32 <= a.Sk;
  auto stores = [&](auto kout, auto vout, int64_t kst, int64_t vst, auto conv) __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int ko = 8 * (r >> 2) + (r & 3);
      if (!whole && key0 + ko >= a.Sk) continue;
#pragma unroll
      for (int db = 0; db < C::DBLK; ++db) {
        kout[ko * kst + 32 * db] = conv(dk[db][r] * scale);
        vout[ko * vst + 32 * db] = conv(dv[db][r]);
      }
    }
  };
  if (partial) {
    // fp32 partials [B, Sk, Hq, D] in the workspace, summed per group later.
    const int64_t i0 = (((int64_t)b * a.Sk + key0) * a.Hq + h) * D + c;
    stores(a.part_dk + i0, a.part_dv + i0, (int64_t)a.Hq * D, (int64_t)a.Hq * D, [](float v) { return v; });
  } else {
    bf16_t* dkp = static_cast<bf16_t*>(a.dk) + b * a.dk_sb + (int64_t)key0 * a.dk_ss + kvh * a.dk_sh + c;
    bf16_t* dvp = static_cast<bf16_t*>(a.dv) + b * a.dv_sb + (int64_t)key0 * a.dv_ss + kvh * a.dv_sh + c;
    stores(dkp, dvp, a.dk_ss, a.dv_ss, [](float v) { return f32_to_elem<T>(v); });
  }
}

// ---------------------------------------------------------------------------
// 2b. dK / dV with paired waves (the deterministic schedule).
//
// The kernel above keeps K, V, dK and dV of 32 keys in one wave (over 400
// registers), so one wave runs per SIMD and its matrix-core, vector and LDS
// work serialise.  Here the four products of a 32-key block are split over
// two waves of one workgroup (eight waves, 128 keys):
//   wave A (waves 0-3) holds K:  S = Q K^T, P (masks, score mods), dV += P^T dO;
//   wave B (waves 4-7) holds V:  dP = dO V^T, dS = P' (dP - Delta), dK += dS^T Q,
// with P' = P (times 1 - tanh^2 under softcap) handed from A to B through LDS
// in fp16 (P' lies in [0, 1], where fp16 keeps three more bits than bf16), one
// tile later: at step t wave A works on query tile t
// and wave B on tile t - 1, so the hand-over needs only the barrier that ends
// each step.  Each wave holds about half the registers, so two run per SIMD,
// and the LDS reads per tile are those of the single-wave kernel plus the
// hand-over.

template <int D>
struct KVPairCfg {
  static constexpr int NW = 8;
  static constexpr int BN = 128;           // keys per workgroup (4 pairs x 32)
  static constexpr int BM = 64;            // queries per streamed tile
  using L = TileLayout<D>;
  static constexpr int TB = L::BYTES;
  static constexpr int DSTEPS = D / 16;
  static constexpr int DBLK = D / 32;
  static constexpr int XB = 4096;          // one wave's P' tile: 32 keys x 64 queries x 2 bytes
};

// LDS offsets of the pair kernel's fragment reads, split into a per-lane part
// (computed once) and a compile-time part (an instruction offset), so the
// register allocator never holds one address per buffer and fragment.
//   row read (A operand, row 32*qb + c, d = 16*ds + 8*g .. +7)
//   transposed read (as tr_frag: 16-row step kk, 32-column block db; the
//   second half of the fragment lies 8 rows further)
template <int D>
struct PairOff {
  static constexpr int RG = TileLayout<D>::RG;
  static constexpr int GS = TileLayout<D>::GS;
  __device__ static int row_lane(int lane) {
    const int g = lane >> 5, c = lane & 31;
    return (c / RG) * GS + (g * RG + c % RG) * 16;
  }
  static constexpr int row(int qb, int ds) { return (32 * qb / RG) * GS + ds * 2 * RG * 16; }
  __device__ static int tr_lane(int lane) {
    const int beta = lane >> 4, s16 = lane & 15;
    const int lr = 4 * (beta >> 1) + (s16 >> 2);
    const int lc = 2 * (beta & 1) + ((s16 & 3) >> 1);
    return (lr / RG) * GS + (lc * RG + lr % RG) * 16 + 8 * (s16 & 1);
  }
  static constexpr int tr(int kk, int db) { return (16 * kk / RG) * GS + db * 4 * RG * 16; }
  static constexpr int TR_HI = (8 / RG) * GS;
};

template <typename T, int D>
__device__ __forceinline__ typename T::vec8 pair_row(const char* tile_lane, int qb, int ds) {
  return *reinterpret_cast<const typename T::vec8*>(tile_lane + PairOff<D>::row(qb, ds));
}
template <typename T, int D>
__device__ __forceinline__ typename T::vec8 pair_tr(const char* tile_lane, int kk, int db) {
  const char* p = tile_lane + PairOff<D>::tr(kk, db);
  return cat_frag<typename T::vec8>(lds_read_tr16(reinterpret_cast<const bf16_t*>(p)),
                                    lds_read_tr16(reinterpret_cast<const bf16_t*>(p + PairOff<D>::TR_HI)));
}

// Wave A on one tile: S, P, the hand-over of P' and dV += P^T dO.
template <typename T, int D, int MOD>
__device__ __forceinline__ void pair_side_a(const char* qt_lds, const char* dot_lds, int lo_row, int lo_tr,
                                            const float* lse_t,
                                            const typename T::vec8 (&kf)[D / 16], f32x16 (&dv)[D / 32],
                                            const BwdCtx& cx, int q0, int my_key, bool masked, int rows_first,
                                            int rows_count, const int* docq_t, bool has_doc, int my_doc,
                                            char* xb, int lane) {
  using C = KVPairCfg<D>;
  constexpr bool kAlibi = MOD & 1;
  constexpr bool kSoftcap = MOD & 2;
  const int g = lane >> 5, c = lane & 31;

  f32x16 s[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int r = 0; r < 16; ++r) s[qb][r] = 0.0f;
#pragma unroll
  for (int ds = 0; ds < C::DSTEPS; ++ds) {
    typename T::vec8 qa[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) qa[qb] = pair_row<T, D>(qt_lds + lo_row, qb, ds);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) s[qb] = mfma32(qa[qb], kf[ds], s[qb]);
  }

  typename T::vec8 pf[2][2];
  f16x8 xh[2][2];  // P' for wave B, in fp16 whatever the input type (P' lies in [0, 1])
  const uint32_t span = static_cast<uint32_t>(rows_count);
  const int ib = q0 + 4 * g - rows_first;
  // P for every element, with the predicate compiled only into the partial
  // tiles' copy (kept inside the loop as a runtime test, the compiler turned
  // it into selects that every tile paid for).  Only P is written in the two
  // branches; the accumulators are not touched before they join.
  auto probs = [&](auto mtag) __attribute__((always_inline)) {
    constexpr bool kMasked = decltype(mtag)::value;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const float4 l4 = *reinterpret_cast<const float4*>(lse_t + 32 * qb + 8 * rr + 4 * g);
        const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
        // (the document ids are read whatever has_doc says and ignored without
        // a document mask: a test guarded by has_doc became a branch per element)
        int dv4[4] = {0, 0, 0, 0};
        if constexpr (kMasked) {
          const int4 d4 = *reinterpret_cast<const int4*>(docq_t + 32 * qb + 8 * rr + 4 * g);
          dv4[0] = d4.x; dv4[1] = d4.y; dv4[2] = d4.z; dv4[3] = d4.w;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * rr + e;
          float th = 0.0f;
          const int i = q0 + roff(qb, r) + 4 * g;
          float p = fast_exp2(score_minus<kAlibi, kSoftcap>(s[qb][r], lv[e], cx, i + cx.delta_pos - my_key, &th));
          if constexpr (kMasked) {
            // rows [rows_first, rows_first + rows_count) may see this key; with
            // a document mask the row's document must also be the key's
            const bool ok = (static_cast<uint32_t>(ib + roff(qb, r)) < span) & (!has_doc | (dv4[e] == my_doc));
            p = ok ? p : 0.0f;
          }
          pf[qb][r >> 3][r & 7] = static_cast<typename T::elem>(p);
          xh[qb][r >> 3][r & 7] = static_cast<_Float16>(kSoftcap ? p * (1.0f - th * th) : p);
        }
      }
  };
  if (masked)
    probs(std::true_type{});
  else
    probs(std::false_type{});
  // hand-over: chunk j = 2 qb + h of every lane at j * 1 KB + 16 * lane
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
      *reinterpret_cast<f16x8*>(xb + (2 * qb + hh) * 1024 + 16 * lane) = xh[qb][hh];

#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    typename T::vec8 fo[C::DBLK];
#pragma unroll
    for (int db = 0; db < C::DBLK; ++db) fo[db] = pair_tr<T, D>(dot_lds + lo_tr, kk, db);
#pragma unroll
    for (int db = 0; db < C::DBLK; ++db) dv[db] = mfma32(pf[kk >> 1][kk & 1], fo[db], dv[db]);
  }
}

// Wave B on the previous tile: dP, dS from the handed-over P', dK += dS^T Q.
template <typename T, int D>
__device__ __forceinline__ void pair_side_b(const char* qt_lds, const char* dot_lds, int lo_row, int lo_tr,
                                            const float* dl_t,
                                            const typename T::vec8 (&vf)[D / 16], f32x16 (&dk)[D / 32],
                                            const char* xb, int lane) {
  using C = KVPairCfg<D>;
  const int g = lane >> 5, c = lane & 31;

  f32x16 dp[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int r = 0; r < 16; ++r) dp[qb][r] = 0.0f;
#pragma unroll
  for (int ds = 0; ds < C::DSTEPS; ++ds) {
    typename T::vec8 da[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) da[qb] = pair_row<T, D>(dot_lds + lo_row, qb, ds);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) dp[qb] = mfma32(da[qb], vf[ds], dp[qb]);
  }

  f16x8 xh[2][2];
  typename T::vec8 sf[2][2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
      xh[qb][hh] = *reinterpret_cast<const f16x8*>(xb + (2 * qb + hh) * 1024 + 16 * lane);
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const float4 d4 = *reinterpret_cast<const float4*>(dl_t + 32 * qb + 8 * rr + 4 * g);
      const float dlv[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * rr + e;
        // written as an fma with a zero addend so the fp16 operand is read
        // by one mixed-precision fma (no separate conversion); it differs
        // from the product only in the sign of a zero result
        const float pv = static_cast<float>(xh[qb][r >> 3][r & 7]);
        sf[qb][r >> 3][r & 7] = static_cast<typename T::elem>(__builtin_fmaf(pv, dp[qb][r] - dlv[e], 0.0f));
      }
    }

#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    typename T::vec8 fq[C::DBLK];
#pragma unroll
    for (int db = 0; db < C::DBLK; ++db) fq[db] = pair_tr<T, D>(qt_lds + lo_tr, kk, db);
#pragma unroll
    for (int db = 0; db < C::DBLK; ++db) dk[db] = mfma32(sf[kk >> 1][kk & 1], fq[db], dk[db]);
  }
}

// GL (grouped-query heads looped in the workgroup): a workgroup owns 128 keys
// of one (batch, kv head) and streams the query tiles of the G query heads of
// its group one head after another into the same dK/dV accumulators, which it
// writes rounded once; without GL it owns 128 keys of one query head.
template <typename T, int D, int MOD, bool GL>
__global__ __launch_bounds__(512, 1) void bwd_dkdv_pair_kernel(BwdArgs a, int partial) {
  using C = KVPairCfg<D>;
  // Three tile buffers (distinct LDS objects: a copy is never taken to alias
  // the buffers being read): step t reads tiles t and t - 1 while t + 1 copies.
  __shared__ __attribute__((aligned(16))) char lq0[C::TB];
  __shared__ __attribute__((aligned(16))) char lq1[C::TB];
  __shared__ __attribute__((aligned(16))) char lq2[C::TB];
  __shared__ __attribute__((aligned(16))) char ld0[C::TB];
  __shared__ __attribute__((aligned(16))) char ld1[C::TB];
  __shared__ __attribute__((aligned(16))) char ld2[C::TB];
  __shared__ __attribute__((aligned(16))) float ll0[C::BM];
  __shared__ __attribute__((aligned(16))) float ll1[C::BM];
  __shared__ __attribute__((aligned(16))) float ll2[C::BM];
  __shared__ __attribute__((aligned(16))) float lg0[C::BM];
  __shared__ __attribute__((aligned(16))) float lg1[C::BM];
  __shared__ __attribute__((aligned(16))) float lg2[C::BM];
  __shared__ __attribute__((aligned(16))) int lz0[C::BM];
  __shared__ __attribute__((aligned(16))) int lz1[C::BM];
  __shared__ __attribute__((aligned(16))) int lz2[C::BM];
  __shared__ __attribute__((aligned(16))) char lx[2 * 4 * C::XB];  // P' hand-over, by step parity and pair

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool side_a = wave < 4;
  const int pair = wave & 3;
  const int lo_row = PairOff<D>::row_lane(lane), lo_tr = PairOff<D>::tr_lane(lane);
  const int g = lane >> 5, c = lane & 31;
  const int Gq = a.Hq / a.Hkv;
  const int nh = GL ? a.Hkv : a.Hq;  // heads the grid enumerates
  const int per = nh * a.B;
  const int kt = blockIdx.x / per;  // key tiles near the start see the most causal rows
  const int rem = blockIdx.x % per;
  const int b = rem / nh;
  int hw = rem % nh;
  if ((nh & 7) == 0) hw = (hw & 7) * (nh >> 3) + (hw >> 3);
  const int kvh = GL ? hw : hw / Gq;
  const int h = GL ? kvh * Gq : hw;  // the (first) query head
  const int nhead = GL ? Gq : 1;

  const bf16_t* qp = static_cast<const bf16_t*>(a.q) + b * a.q_sb + h * a.q_sh;
  const bf16_t* dop = static_cast<const bf16_t*>(a.dout) + b * a.do_sb + h * a.do_sh;
  const float* lsep = a.lse2 + ((int64_t)b * a.Hq + h) * a.Sq;
  const float* dlp = a.delta + ((int64_t)b * a.Hq + h) * a.Sq;

  const int kv0 = kt * C::BN + 32 * pair;  // the pair's first key
  const int my_key = kv0 + c;
  const bool k_ok = my_key < a.Sk;

  // K (wave A) or V (wave B) of this lane's key as B operands, d = 16*ds + 8*g .. +7.
  typename T::vec8 xf[C::DSTEPS];
  {
    const bf16_t* src = side_a ? static_cast<const bf16_t*>(a.k) + b * a.k_sb + kvh * a.k_sh
                               : static_cast<const bf16_t*>(a.v) + b * a.v_sb + kvh * a.v_sh;
    const int64_t ld = side_a ? a.k_ss : a.v_ss;
#pragma unroll
    for (int ds = 0; ds < C::DSTEPS; ++ds) {
      uint4 x = make_uint4(0, 0, 0, 0);
      if (k_ok) x = *reinterpret_cast<const uint4*>(src + (int64_t)my_key * ld + 16 * ds + 8 * g);
      xf[ds] = __builtin_bit_cast(typename T::vec8, x);
    }
  }
  const BwdCtx cx0 = make_ctx(a, b, h, MOD & 1, MOD & 2);

  // Query tiles that meet the workgroup's keys (as in the kernel above), per
  // head; with GL the step stream runs through them once per head.
  const RowWindow win(a.Sq, a.Sk, a.mask.causal, a.mask.wl, a.mask.wr);
  constexpr bool sparse = (MOD & 4) != 0;
  int qt_begin = 0, ntiles = 0, n_full_blk = 0;
  const int32_t* qi_full = nullptr;
  const int32_t* qi_part = nullptr;
  if (sparse) {
    const int u = b * a.tiles.nK + (kt * C::BN) / a.tiles.block_n;
    n_full_blk = a.tiles.q_num_full[u];
    ntiles = 2 * (n_full_blk + a.tiles.q_num_partial[u]);
    qi_full = a.tiles.q_idx_full + (int64_t)u * a.tiles.nQ;
    qi_part = a.tiles.q_idx_partial + (int64_t)u * a.tiles.nQ;
  } else {
    const int c0 = kt * C::BN, c1 = min(a.Sk, c0 + C::BN) - 1;
    int i_lo = 0, i_hi = a.Sq - 1;
    if (win.R != kUnbounded) i_lo = max(i_lo, c0 - cx0.delta_pos - win.R);
    if (win.L != kUnbounded) i_hi = min(i_hi, c1 - cx0.delta_pos + win.L);
    qt_begin = i_lo <= i_hi ? i_lo / C::BM : 0;
    ntiles = i_lo <= i_hi ? i_hi / C::BM + 1 - qt_begin : 0;
  }
  const int ntq = ntiles;  // query tiles per head
  ntiles *= nhead;
  // Step t is query tile t % ntq of head h + t / ntq.
  auto head_of = [&](int t) __attribute__((always_inline)) -> int { return GL ? t / ntq : 0; };
  auto qt_of = [&](int t) __attribute__((always_inline)) -> int {
    if (GL) t -= ntq * (t / ntq);
    if (!sparse) return qt_begin + t;
    const int blk = t >> 1;
    return 2 * (blk < n_full_blk ? qi_full[blk] : qi_part[blk - n_full_blk]) + (t & 1);
  };
  // Whether this pair's 32 keys meet query tile t, and whether a predicate is needed.
  auto tile_state = [&](int t, int qt, bool* masked) __attribute__((always_inline)) -> bool {
    if (sparse) {
      if (GL) t -= ntq * (t / ntq);
      *masked = (t >> 1) >= n_full_blk;
      return true;
    }
    const TileRange trq(win, qt, C::BM, 32);
    const int kw = kv0 / 32;
    *masked = !trq.full(kw);
    return kw >= trq.kt_begin && kw < trq.kt_end;
  };
  int rows_first, rows_count;
  win.key_rows(my_key, &rows_first, &rows_count);
  const bool has_doc = sparse && a.mask.doc_q != nullptr;
  const int my_doc = has_doc && k_ok ? a.mask.doc_k[(int64_t)b * a.Sk + my_key] : 0;
  const int32_t* docq = has_doc ? a.mask.doc_q + (int64_t)b * a.Sq : nullptr;

  // Copies of one tile: every wave its share of the Q and dO rows; waves 0,
  // 1 and 2 (with a document mask) one 64-entry row of lse2, Delta and the
  // rows' document ids.  Rows past Sq repeat the last row (masked by wave A,
  // and their P' is zero for wave B).
  // (Copies stay compiler-visible here: issued from inline assembly, which
  // lets the compiler count LDS reads precisely, this kernel was 19% slower.)
  const TileCopy<D, C::NW> qcopy(qp, a.q_ss, a.Sq, wave, lane);
  const TileCopy<D, C::NW> dcopy(dop, a.do_ss, a.Sq, wave, lane);
  auto load_tile = [&](int t, auto buf_tag) __attribute__((always_inline)) {
    constexpr int BUF = decltype(buf_tag)::value;
    const int qt = qt_of(t), x = head_of(t);
    char* qd = BUF == 0 ? lq0 : (BUF == 1 ? lq1 : lq2);
    char* dd = BUF == 0 ? ld0 : (BUF == 1 ? ld1 : ld2);
    qcopy(reinterpret_cast<bf16_t*>(qd), qt * C::BM, (int64_t)x * a.q_sh);
    dcopy(reinterpret_cast<bf16_t*>(dd), qt * C::BM, (int64_t)x * a.do_sh);
    const int i = min(qt * C::BM + lane, a.Sq - 1) + x * a.Sq;
    if (wave == 0)
      __builtin_amdgcn_global_load_lds(lsep + i, (__attribute__((address_space(3))) void*)(BUF == 0 ? ll0 : (BUF == 1 ? ll1 : ll2)), 4, 0, 0);
    else if (wave == 1)
      __builtin_amdgcn_global_load_lds(dlp + i, (__attribute__((address_space(3))) void*)(BUF == 0 ? lg0 : (BUF == 1 ? lg1 : lg2)), 4, 0, 0);
    else if (wave == 2 && has_doc)
      __builtin_amdgcn_global_load_lds(docq + i - x * a.Sq, (__attribute__((address_space(3))) void*)(BUF == 0 ? lz0 : (BUF == 1 ? lz1 : lz2)), 4, 0, 0);
  };
  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  using B2 = std::integral_constant<int, 2>;

  f32x16 acc[C::DBLK];  // dV (wave A) or dK (wave B)
#pragma unroll
  for (int db = 0; db < C::DBLK; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.0f;

  if (ntiles > 0) load_tile(0, B0{});
  wait_dma();
  __syncthreads();

  // Step t (BUF = t mod 3): wave A on tile t, wave B on tile t - 1, the copy
  // of tile t + 1 in flight.  The role is a compile-time tag and each role
  // runs its own copy of the loop (the same steps and barriers), so the
  // accumulators never meet a branch join inside the loop (a join made the
  // compiler copy them every step).
  auto step = [&](int t, auto buf_tag, auto role_tag) __attribute__((always_inline)) {
    constexpr int BUF = decltype(buf_tag)::value;
    constexpr bool kA = decltype(role_tag)::value;
    using NEXT = std::integral_constant<int, (BUF + 1) % 3>;
    constexpr int PREV = (BUF + 2) % 3;
    if (t + 1 < ntiles) load_tile(t + 1, NEXT{});
    if constexpr (kA) {
      if (t < ntiles) {
        const int qt = qt_of(t);
        bool masked;
        // the ALiBi slope is the only per-head term of the score
        const BwdCtx cx = (GL && (MOD & 1)) ? make_ctx(a, b, h + head_of(t), true, MOD & 2) : cx0;
        if (tile_state(t, qt, &masked))
          pair_side_a<T, D, MOD>(BUF == 0 ? lq0 : (BUF == 1 ? lq1 : lq2), BUF == 0 ? ld0 : (BUF == 1 ? ld1 : ld2),
                                 lo_row, lo_tr, BUF == 0 ? ll0 : (BUF == 1 ? ll1 : ll2), xf, acc, cx, qt * C::BM, my_key, masked,
                                 rows_first, rows_count, BUF == 0 ? lz0 : (BUF == 1 ? lz1 : lz2), has_doc, my_doc,
                                 lx + ((t & 1) * 4 + pair) * C::XB, lane);
      }
    } else if (t >= 1) {
      const int qt = qt_of(t - 1);
      bool masked;
      if (tile_state(t - 1, qt, &masked))
        pair_side_b<T, D>(PREV == 0 ? lq0 : (PREV == 1 ? lq1 : lq2), PREV == 0 ? ld0 : (PREV == 1 ? ld1 : ld2),
                          lo_row, lo_tr, PREV == 0 ? lg0 : (PREV == 1 ? lg1 : lg2), xf, acc,
                          lx + (((t - 1) & 1) * 4 + pair) * C::XB, lane);
    }
    wait_dma();       // tile t + 1 has landed ...
    __syncthreads();  // ... for every wave, and P'(t) is visible to wave B
  };
  const int nsteps = ntiles > 0 ? ntiles + 1 : 0;
  auto run = [&](auto role_tag) __attribute__((always_inline)) {
    int t = 0;
    for (; t + 2 < nsteps; t += 3) {
      step(t, B0{}, role_tag);
      step(t + 1, B1{}, role_tag);
      step(t + 2, B2{}, role_tag);
    }
    if (t < nsteps) step(t++, B0{}, role_tag);
    if (t < nsteps) step(t++, B1{}, role_tag);
  };
  if (side_a)
    run(std::true_type{});
  else
    run(std::false_type{});

  // acc[db][r]: key kv0 + 8*(r/4) + 4*g + r%4, d = 32*db + c; wave A holds
  // dV, wave B dK (scaled here).
  // One base address per lane (its first key and d = c) and per-element
  // offsets that are multiples of the key stride; the key bound is tested only
  // when the wave's 32 keys run past Sk.
  const float mul = side_a ? 1.0f : a.scale;
  const int key0 = kv0 + 4 * g;
  const bool whole = kv0 + 32 <= a.Sk;
  auto stores = [&](auto out, int64_t kstride, auto conv) __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int ko = 8 * (r >> 2) + (r & 3);
      if (!whole && key0 + ko >= a.Sk) continue;
#pragma unroll
      for (int db = 0; db < C::DBLK; ++db) out[ko * kstride + 32 * db] = conv(acc[db][r] * mul);
    }
  };
  if (partial) {
    float* base = (side_a ? a.part_dv : a.part_dk) + (((int64_t)b * a.Sk + key0) * a.Hq + h) * D + c;
    stores(base, (int64_t)a.Hq * D, [](float v) { return v; });
  } else {
    bf16_t* base = side_a ? static_cast<bf16_t*>(a.dv) + b * a.dv_sb + (int64_t)key0 * a.dv_ss + kvh * a.dv_sh + c
                          : static_cast<bf16_t*>(a.dk) + b * a.dk_sb + (int64_t)key0 * a.dk_ss + kvh * a.dk_sh + c;
    stores(base, side_a ? a.dv_ss : a.dk_ss, [](float v) { return f32_to_elem<T>(v); });
  }
}

// Sum the G per-head partials of each kv head in head order -> bf16.  One
// thread per 8 consecutive d of one (b, key, kv head): 16-byte loads of each
// head's partials and one 16-byte store per output.  Row indices fit 32 bits
// (the fp32 partials of B*Sk*Hq rows of D floats must fit device memory).
template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_group_sum_kernel(BwdArgs a) {
  constexpr int CH = D / 8;  // 8-element chunks per row
  const uint32_t rows = static_cast<uint32_t>(a.B) * a.Sk * a.Hkv;
  const uint32_t t = blockIdx.x * 256u + threadIdx.x;
  if ((uint64_t)t >= (uint64_t)rows * CH) return;
  const int ch = static_cast<int>(t % CH);
  const uint32_t row = t / CH;  // (b * Sk + j) * Hkv + g
  const int g = static_cast<int>(row % a.Hkv);
  const uint32_t bj = row / a.Hkv;
  const int j = static_cast<int>(bj % a.Sk);
  const int b = static_cast<int>(bj / a.Sk);
  const int G = a.Hq / a.Hkv;
  const int64_t base = ((int64_t)bj * a.Hq + (int64_t)g * G) * D + 8 * ch;
  float sk[8], sv[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) sk[e] = sv[e] = 0.0f;
  for (int x = 0; x < G; ++x) {
    const float4* pk = reinterpret_cast<const float4*>(a.part_dk + base + (int64_t)x * D);
    const float4* pv = reinterpret_cast<const float4*>(a.part_dv + base + (int64_t)x * D);
    const float4 k0 = pk[0], k1 = pk[1], v0 = pv[0], v1 = pv[1];
    const float kx[8] = {k0.x, k0.y, k0.z, k0.w, k1.x, k1.y, k1.z, k1.w};
    const float vx[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      sk[e] += kx[e];
      sv[e] += vx[e];
    }
  }
  uint32_t wk[4], wv[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    wk[e] = f32_to_elem<T>(sk[2 * e]) | (uint32_t)f32_to_elem<T>(sk[2 * e + 1]) << 16;
    wv[e] = f32_to_elem<T>(sv[2 * e]) | (uint32_t)f32_to_elem<T>(sv[2 * e + 1]) << 16;
  }
  bf16_t* dkp = static_cast<bf16_t*>(a.dk) + b * a.dk_sb + (int64_t)j * a.dk_ss + g * a.dk_sh + 8 * ch;
  bf16_t* dvp = static_cast<bf16_t*>(a.dv) + b * a.dv_sb + (int64_t)j * a.dv_ss + g * a.dv_sh + 8 * ch;
  *reinterpret_cast<uint4*>(dkp) = make_uint4(wk[0], wk[1], wk[2], wk[3]);
  *reinterpret_cast<uint4*>(dvp) = make_uint4(wv[0], wv[1], wv[2], wv[3]);
}

// Non-deterministic dQ: scale the fp32 accumulator and round to bf16.
template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_dq_convert_kernel(BwdArgs a) {
  const int64_t n = (int64_t)a.B * a.Sq * a.Hq * (D / 8);
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= n) return;
  const int part = static_cast<int>(t % (D / 8));
  const int64_t row = t / (D / 8);  // (b * Sq + i) * Hq + h
  const int h = static_cast<int>(row % a.Hq);
  const int i = static_cast<int>((row / a.Hq) % a.Sq);
  const int b = static_cast<int>(row / ((int64_t)a.Hq * a.Sq));
  const float4* src = reinterpret_cast<const float4*>(a.dq_acc + row * D + part * 8);
  const float4 x = src[0], y = src[1];
  const float sc = a.scale;
  uint4 o;
  o.x = f32_to_elem<T>(x.x * sc) | (uint32_t)f32_to_elem<T>(x.y * sc) << 16;
  o.y = f32_to_elem<T>(x.z * sc) | (uint32_t)f32_to_elem<T>(x.w * sc) << 16;
  o.z = f32_to_elem<T>(y.x * sc) | (uint32_t)f32_to_elem<T>(y.y * sc) << 16;
  o.w = f32_to_elem<T>(y.z * sc) | (uint32_t)f32_to_elem<T>(y.w * sc) << 16;
  *reinterpret_cast<uint4*>(static_cast<bf16_t*>(a.dq) + b * a.dq_sb + (int64_t)i * a.dq_ss + h * a.dq_sh +
                            part * 8) = o;
}

// ---------------------------------------------------------------------------
// 3. dQ

template <int D>
struct QCfg {
  static constexpr int BM = 128;           // query rows per workgroup (4 waves x 32)
  static constexpr int BN = 64;            // keys per streamed tile
  using L = TileLayout<D>;
  static constexpr int TB = L::BYTES;
  static constexpr int DSTEPS = D / 16;
  static constexpr int DBLK = D / 32;
};

// One 64-key tile: S^T = K Q^T and dP^T = V dO^T (one query per lane),
// dS^T from the saved LSE and Delta, dQ^T += K^T dS^T.
template <typename T, int D, int MOD, bool MASKED>
__device__ __forceinline__ void dq_tile(const char* kt_lds, const char* vt_lds, const typename T::vec8 (&qf)[D / 16],
                                        const typename T::vec8 (&df)[D / 16], f32x16 (&dq)[D / 32],
                                        const BwdCtx& cx, float lse2, float dl, int my_q, int key_base,
                                        int row_first, int row_count, const int* dock_t, bool has_doc,
                                        int my_doc, int lane) {
  using C = QCfg<D>;
  constexpr bool kAlibi = MOD & 1;
  constexpr bool kSoftcap = MOD & 2;
  const int g = lane >> 5, c = lane & 31;
  f32x16 s[2], dp[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s[kb][r] = 0.0f;
      dp[kb][r] = 0.0f;
    }
#pragma unroll
  for (int ds = 0; ds < C::DSTEPS; ++ds) {
    typename T::vec8 ka[2], va[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      ka[kb] = row_frag<T, D>(kt_lds, 32 * kb + c, ds, g);
      va[kb] = row_frag<T, D>(vt_lds, 32 * kb + c, ds, g);
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = mfma32(ka[kb], qf[ds], s[kb]);
      dp[kb] = mfma32(va[kb], df[ds], dp[kb]);
    }
  }
  const uint32_t span = static_cast<uint32_t>(row_count);
  const int jb = key_base + 4 * g - row_first;
  typename T::vec8 sf[2][2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      // (on partial tiles the document ids are read whatever has_doc says and
      // ignored without a document mask: a test guarded by has_doc became a
      // branch per element)
      int4 d4 = make_int4(0, 0, 0, 0);
      if (MASKED) d4 = *reinterpret_cast<const int4*>(dock_t + 32 * kb + 8 * rr + 4 * g);
      const int dv4[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * rr + e;
        float th = 0.0f;
        const int j = key_base + 4 * g + roff(kb, r);
        float p = fast_exp2(score_minus<kAlibi, kSoftcap>(s[kb][r], lse2, cx, my_q + cx.delta_pos - j, &th));
        if (MASKED) {
          const bool ok = (static_cast<uint32_t>(jb + roff(kb, r)) < span) & (!has_doc | (dv4[e] == my_doc));
          p = ok ? p : 0.0f;
        }
        float dsv = p * (dp[kb][r] - dl);
        if (kSoftcap) dsv *= 1.0f - th * th;
        sf[kb][r >> 3][r & 7] = static_cast<typename T::elem>(dsv);
      }
    }
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    typename T::vec8 ka[C::DBLK];
#pragma unroll
    for (int db = 0; db < C::DBLK; ++db) ka[db] = tr_frag<T, D>(kt_lds, kk, db, lane);
#pragma unroll
    for (int db = 0; db < C::DBLK; ++db) dq[db] = mfma32(ka[db], sf[kk >> 1][kk & 1], dq[db]);
  }
}

template <typename T, int D, int MOD>
__global__ __launch_bounds__(256, 2) void bwd_dq_kernel(BwdArgs a, int fold) {
  using C = QCfg<D>;
  __shared__ __attribute__((aligned(16))) char lk0[C::TB];
  __shared__ __attribute__((aligned(16))) char lk1[C::TB];
  __shared__ __attribute__((aligned(16))) char lv0[C::TB];
  __shared__ __attribute__((aligned(16))) char lv1[C::TB];
  __shared__ __attribute__((aligned(16))) int lz0[C::BN];
  __shared__ __attribute__((aligned(16))) int lz1[C::BN];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, c = lane & 31;
  const int nqt = (a.Sq + C::BM - 1) / C::BM;
  const int per = a.Hq * a.B;
  // Query tiles heaviest first; with fold > 0 the grid rows from fold on run
  // lightest first instead.  Two workgroups share a CU, and when the whole
  // grid is resident at once the dispatcher pairs workgroup x with x + (the
  // number of CUs), so folding pairs heavy causal tiles with light ones.
  const int u_row = blockIdx.x / per;
  const int qt = (fold == 0 || u_row < fold) ? nqt - 1 - u_row : u_row - fold;
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
  typename T::vec8 qf[C::DSTEPS], df[C::DSTEPS];
  // (All loads issued before any use; rows past Sq read row Sq - 1 and are
  // zeroed after.)
  const int q_row = q_ok ? my_q : a.Sq - 1;
  const int64_t row_idx = ((int64_t)b * a.Hq + h) * a.Sq + q_row;
  float d_part = 0.0f;  // this lane's half of Delta = <dO, O> (d = 16*ds + 8*g .. +7)
  {
    const bf16_t* op = static_cast<const bf16_t*>(a.o) + b * a.o_sb + h * a.o_sh;
    uint4 r1[C::DSTEPS], r2[C::DSTEPS], r3[C::DSTEPS];
#pragma unroll
    for (int ds = 0; ds < C::DSTEPS; ++ds) {
      r1[ds] = *reinterpret_cast<const uint4*>(qp + (int64_t)q_row * a.q_ss + 16 * ds + 8 * g);
      r2[ds] = *reinterpret_cast<const uint4*>(dop + (int64_t)q_row * a.do_ss + 16 * ds + 8 * g);
      r3[ds] = *reinterpret_cast<const uint4*>(op + (int64_t)q_row * a.o_ss + 16 * ds + 8 * g);
    }
#pragma unroll
    for (int ds = 0; ds < C::DSTEPS; ++ds) {
      const uint32_t dw[4] = {r2[ds].x, r2[ds].y, r2[ds].z, r2[ds].w};
      const uint32_t ow[4] = {r3[ds].x, r3[ds].y, r3[ds].z, r3[ds].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        d_part = __builtin_fmaf(T::to_f32(dw[e] & 0xffffu), T::to_f32(ow[e] & 0xffffu), d_part);
        d_part = __builtin_fmaf(T::to_f32(dw[e] >> 16), T::to_f32(ow[e] >> 16), d_part);
      }
    }
#pragma unroll
    for (int ds = 0; ds < C::DSTEPS; ++ds) {
      const uint4 z = make_uint4(0, 0, 0, 0);
      qf[ds] = __builtin_bit_cast(typename T::vec8, q_ok ? r1[ds] : z);
      df[ds] = __builtin_bit_cast(typename T::vec8, q_ok ? r2[ds] : z);
    }
  }
  const BwdCtx cx = make_ctx(a, b, h, MOD & 1, MOD & 2);
  const float l_row = a.lse[row_idx];
  const float lse2 = !q_ok || l_row == kNegInf ? kPosInf : l_row * kLog2e;  // empty rows: P = 0
  const float d_row = d_part + wave_xor32(d_part);
  const float dl = q_ok ? d_row : 0.0f;
  // Delta and lse2 of every row for the dK/dV kernel, which runs after this
  // one (written before any early exit: it reads them for every row it meets).
  if (q_ok && g == 0) {
    a.delta[row_idx] = d_row;
    a.lse2[row_idx] = lse2;
  }

  // Key tiles in processing order, FULL ones first.  Dense: the interval of
  // the causal / window band.  Block-sparse: the mask's FULL then PARTIAL
  // key blocks of this query block (block_n / 64 tiles each).
  const RowWindow win(a.Sq, a.Sk, a.mask.causal, a.mask.wl, a.mask.wr);
  const TileRange range(win, qt, C::BM, C::BN);
  constexpr bool sparse = (MOD & 4) != 0;  // block-mask lists (else the dense band)
  int ntiles, nfull, n_full_blk = 0, sub = 1;
  const int32_t* ki_full = nullptr;
  const int32_t* ki_part = nullptr;
  if (sparse) {
    const int row = b * a.tiles.nQ + qt;
    sub = a.tiles.block_n / C::BN;
    n_full_blk = a.tiles.kv_num_full[row];
    ntiles = (n_full_blk + a.tiles.kv_num_partial[row]) * sub;
    nfull = n_full_blk * sub;
    ki_full = a.tiles.kv_idx_full + (int64_t)row * a.tiles.nK;
    ki_part = a.tiles.kv_idx_partial + (int64_t)row * a.tiles.nK;
  } else {
    ntiles = range.kt_end - range.kt_begin;
    nfull = range.n_full();
  }
  auto kt_of = [&](int t) -> int {
    if (!sparse) return range.kt_at(t);
    const int blk = t / sub;
    return (blk < n_full_blk ? ki_full[blk] : ki_part[blk - n_full_blk]) * sub + t % sub;
  };
  int row_first, row_count;
  win.row_keys(my_q, &row_first, &row_count);
  const bool has_doc = sparse && a.mask.doc_q != nullptr;  // document masks come with block masks
  const int my_doc = has_doc && q_ok ? a.mask.doc_q[(int64_t)b * a.Sq + my_q] : 0;
  const int32_t* dock = has_doc ? a.mask.doc_k + (int64_t)b * a.Sk : nullptr;

  // K and V of tile kt into buffer BUF, and (document masks) the tile's 64
  // key document ids, copied by wave 0; every wait below is a full one.
  // Copies issued from inline assembly (dma16 / dma4): copies the compiler
  // can see make it treat every LDS read as unordered and wait for each one
  // in full (lgkmcnt(0)); hidden from it, the fragment reads overlap.
  const TileCopy<D, 4, true> kcopy(kp, a.k_ss, a.Sk, wave, lane);
  const TileCopy<D, 4, true> vcopy(vp, a.v_ss, a.Sk, wave, lane);
  auto load_tile = [&](int kt, auto buf_tag) {
    constexpr int BUF = decltype(buf_tag)::value;
    kcopy(reinterpret_cast<bf16_t*>(BUF ? lk1 : lk0), kt * C::BN);
    vcopy(reinterpret_cast<bf16_t*>(BUF ? lv1 : lv0), kt * C::BN);
    if (has_doc && wave == 0) {
      const int j = min(kt * C::BN + lane, a.Sk - 1);  // keys past Sk are masked
      dma4(dock + j, lds_addr(BUF ? lz1 : lz0));
    }
  };
  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;

  f32x16 dq[C::DBLK];
#pragma unroll
  for (int db = 0; db < C::DBLK; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) dq[db][r] = 0.0f;

  if (ntiles > 0) load_tile(kt_of(0), B0{});
  wait_dma();
  __syncthreads();

  auto step = [&](int t, auto buf_tag, auto masked) {
    constexpr int BUF = decltype(buf_tag)::value;
    using NEXT = std::integral_constant<int, 1 - BUF>;
    const int kt = kt_of(t);
    const bool has_next = t + 1 < ntiles;
    if (has_next) load_tile(kt_of(t + 1), NEXT{});
    dq_tile<T, D, MOD, decltype(masked)::value>(BUF ? lk1 : lk0, BUF ? lv1 : lv0, qf, df, dq, cx, lse2, dl,
                                             my_q, kt * C::BN, row_first, row_count, BUF ? lz1 : lz0,
                                             has_doc, my_doc, lane);
    wait_dma();
    __syncthreads();
  };
  using FULL = std::false_type;
  using PART = std::true_type;
  int t = 0;
  for (; t + 1 < nfull; t += 2) {
    step(t, B0{}, FULL{});
    step(t + 1, B1{}, FULL{});
  }
  if (t < nfull) step(t++, B0{}, FULL{});
  if (t < ntiles && (t & 1)) step(t++, B1{}, PART{});
  for (; t + 1 < ntiles; t += 2) {
    step(t, B0{}, PART{});
    step(t + 1, B1{}, PART{});
  }
  if (t < ntiles) step(t++, B0{}, PART{});

  if (q_ok) {
    const float scale = a.scale;
    bf16_t* out = static_cast<bf16_t*>(a.dq) + b * a.dq_sb + (int64_t)my_q * a.dq_ss + h * a.dq_sh;
#pragma unroll
    for (int db = 0; db < C::DBLK; ++db) {
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int d0 = 32 * db + 8 * rr + 4 * g;
        uint2 packed;
        packed.x = f32_to_elem<T>(dq[db][4 * rr] * scale) | (uint32_t)f32_to_elem<T>(dq[db][4 * rr + 1] * scale) << 16;
        packed.y = f32_to_elem<T>(dq[db][4 * rr + 2] * scale) | (uint32_t)f32_to_elem<T>(dq[db][4 * rr + 3] * scale) << 16;
        *reinterpret_cast<uint2*>(out + d0) = packed;
      }
    }
  }
}

template <typename T, int D, int MOD>
hipError_t launch_mod(const BwdArgs& a, int stages, hipStream_t s) {
  const int G = a.Hq / a.Hkv;
  static_assert(KVPairCfg<D>::BN == KVCfg<D>::BN, "both dK/dV kernels take 128 keys per workgroup");
  const int nkt = (a.Sk + KVCfg<D>::BN - 1) / KVCfg<D>::BN;
  const bool atomic_dq = a.dq_acc != nullptr;
  constexpr bool kPairOk = D == 128 || !(MOD & 4);
  // Grouped-query heads: loop the G heads inside each dK/dV workgroup (no
  // per-head partials and no group sum) when the kv-head grid alone has at
  // least two workgroups per CU to balance; else one workgroup per query
  // head writes an fp32 partial and the group-sum kernel adds them up.
  const bool group_loop = kPairOk && !atomic_dq && G > 1 &&
                          bwd_group_loop_choice((long)nkt * a.Hkv * a.B, device_cu_count());
  const int partial = (G > 1 && !group_loop) ? 1 : 0;
  // Deterministic schedule: stage 0 is the dQ kernel, which also writes
  // Delta and lse2 for the dK/dV kernel (no separate Delta pass).
  const int nqt0 = (a.Sq + QCfg<D>::BM - 1) / QCfg<D>::BM;
  if ((stages & 1) && !atomic_dq && nqt0 > 0) {
    // Fold the tile order (see the kernel) when causal work is uneven and the
    // grid fits the GPU at two workgroups per CU; a larger grid is balanced
    // by dispatching heaviest first as CUs free up.
    const long grid = (long)nqt0 * a.Hq * a.B;
    const int fold = (a.mask.causal && !(MOD & 4) && grid <= 2L * device_cu_count()) ? (nqt0 + 1) / 2 : 0;
    hipLaunchKernelGGL((bwd_dq_kernel<T, D, MOD>), dim3(nqt0 * a.Hq * a.B), dim3(256), 0, s, a, fold);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if ((stages & 2) && nkt > 0) {
    // Paired waves at D = 128, and at D = 64 without block masks.  With a
    // block mask at D = 64 the single-wave kernel measured faster: a tile has
    // half the matrix work against the same softmax work, and the paired
    // kernel reads the block lists with vector loads it must wait for.
    if (atomic_dq)
      hipLaunchKernelGGL((bwd_dkdv_kernel<T, D, MOD, true>), dim3(nkt * a.Hq * a.B), dim3(256), 0, s, a, partial);
    else if constexpr (kPairOk) {
      if (group_loop)
        hipLaunchKernelGGL((bwd_dkdv_pair_kernel<T, D, MOD, true>), dim3(nkt * a.Hkv * a.B), dim3(512), 0, s, a, 0);
      else
        hipLaunchKernelGGL((bwd_dkdv_pair_kernel<T, D, MOD, false>), dim3(nkt * a.Hq * a.B), dim3(512), 0, s, a,
                           partial);
    } else
      hipLaunchKernelGGL((bwd_dkdv_kernel<T, D, MOD, false>), dim3(nkt * a.Hq * a.B), dim3(256), 0, s, a, partial);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if ((stages & 4) && partial && a.Sk > 0) {
    const int64_t n = (int64_t)a.B * a.Sk * a.Hkv * (D / 8);
    hipLaunchKernelGGL((bwd_group_sum_kernel<T, D>), dim3((n + 255) / 256), dim3(256), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int nqt = (a.Sq + QCfg<D>::BM - 1) / QCfg<D>::BM;
  if ((stages & 8) && atomic_dq && nqt > 0) {
    const int64_t n = (int64_t)a.B * a.Sq * a.Hq * (D / 8);
    hipLaunchKernelGGL((bwd_dq_convert_kernel<T, D>), dim3((n + 255) / 256), dim3(256), 0, s, a);
    return hipGetLastError();
  }
  return hipSuccess;
}

template <typename T, int D>
hipError_t launch_d(const BwdArgs& a, int stages, hipStream_t s) {
  const int64_t rows = (int64_t)a.B * a.Sq * a.Hq;
  constexpr int LPR = D / 8;
  if ((stages & 1) && rows > 0 && a.dq_acc != nullptr) {  // the atomic-dQ schedule's Delta pass
    hipLaunchKernelGGL((bwd_delta_kernel<T, D>), dim3((rows * LPR + 255) / 256), dim3(256), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // bit 0 ALiBi, bit 1 softcap, bit 2 block-sparse lists (document ids only with these)
  const int mod = (a.alibi != nullptr ? 1 : 0) | (a.softcap > 0.0f ? 2 : 0) |
                  (a.tiles.kv_num_full != nullptr ? 4 : 0);
  switch (mod) {
    case 0: return launch_mod<T, D, 0>(a, stages, s);
    case 1: return launch_mod<T, D, 1>(a, stages, s);
    case 2: return launch_mod<T, D, 2>(a, stages, s);
    case 3: return launch_mod<T, D, 3>(a, stages, s);
    case 4: return launch_mod<T, D, 4>(a, stages, s);
    case 5: return launch_mod<T, D, 5>(a, stages, s);
    case 6: return launch_mod<T, D, 6>(a, stages, s);
    default: return launch_mod<T, D, 7>(a, stages, s);
  }
}

}  // namespace

size_t bwd_workspace_bytes(int B, int Hq, int Hkv, int Sq, int Sk, int D) {
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  size_t n = 2 * up((size_t)B * Hq * Sq * sizeof(float));  // Delta, lse2
  if (Hkv > 0 && Hq / Hkv > 1) n += 2 * up((size_t)B * Sk * Hq * D * sizeof(float));
  n += up((size_t)B * Sq * Hq * D * sizeof(float));  // non-deterministic dQ accumulator
  return n;
}

hipError_t launch_bwd_bf16(const BwdArgs& a, int stage_mask, hipStream_t s) {
  if (a.B == 0 || a.Hq == 0) return hipSuccess;
  if (a.f16) return a.D == 64 ? launch_d<F16T, 64>(a, stage_mask, s) : launch_d<F16T, 128>(a, stage_mask, s);
  if (a.D == 64) return launch_d<Bf16T, 64>(a, stage_mask, s);
  return launch_d<Bf16T, 128>(a, stage_mask, s);
}

}  // namespace attn
