// Forward attention, bf16 or fp16 inputs, MFMA (gfx950).
//
// Tiled exact attention with an online softmax ("Accelerating AI: A Deep
// Dive into Flash Attention", sections "Tiling the Computation",
// "2. Online Softmax" and "3. Weighted Sum of Values"): each workgroup owns
// 128 query rows of one (batch, query head), streams 64-key tiles of the
// matching key/value head through LDS, and keeps a running row maximum, row
// sum and unnormalised output in registers, so scores never reach HBM.
//
// Work split.  4 waves x 32 query rows.  Each wave computes the transposed
// score tile S^T = K Q^T (64 keys x 32 queries) with 32x32x16 MFMAs: K comes
// from LDS (A operand), the wave's Q rows stay in registers (B operand) for
// the whole key loop.  In the S^T accumulator a lane holds 16 keys of one
// query per 32-key half, so the row statistics are in-lane reductions plus
// one exchange with lane l^32.  The same accumulator registers, rounded to
// bf16, are exactly the B operand of O^T += V^T P^T; V^T comes from LDS via
// transposed reads (ds_read_b64_tr_b16), so P never leaves registers.
//
// Score modifiers and masks are the FlexAttention hooks of "Lightning Talk:
// FlexAttention + FlashAttention-4" (score_mod: ALiBi, tanh softcap;
// mask_mod: causal, sliding window, document) and flash_attn_func's
// causal / window_size / alibi_slopes / softcap arguments ("FlashAttention:
// Fast and Memory-Efficient Exact Attention", "Examples").  Masks are
// evaluated only on PARTIAL tiles; EMPTY tiles are never visited.
//
// The running maximum is rescaled lazily: the output and sum are only
// rescaled when a row's maximum grows by more than 2^8 (in exp2 units) over
// the maximum in use, so p = exp2(x - m_used) <= 256.  Sum and output use the
// same m_used, so the final O = acc / l and LSE = m_used + log2(l) are exact.

#include <type_traits>

#include "common.h"
#include "internal.h"

namespace attn {
namespace {

constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kRescaleThreshold = 8.0f;

template <int D, int NW = 4>
struct FwdCfg {
  static constexpr int BM = 32 * NW;       // query rows per workgroup (32 per wave)
  static constexpr int BN = kFwdBN;        // keys per tile
  static constexpr int NT = 64 * NW;       // threads
  using L = TileLayout<D>;                 // LDS image of a 64-key K or V tile
  static constexpr int TB = L::BYTES;      // bytes per tile buffer
  static constexpr int DSTEPS = D / 16;
  static constexpr int DBLK = D / 32;
};

struct Tile {
  int kt;
  bool full;
};

template <typename V>
__device__ __forceinline__ V zero_frag() {
  return __builtin_bit_cast(V, make_uint4(0, 0, 0, 0));
}

struct TileCtx {
  float scale_log2;   // |scale| * log2(e)
  float slope_log2;   // ALiBi slope * log2(e)
  float cap_k2;       // 2 log2(e) |scale| / softcap
  float cap_log2;     // softcap * log2(e)
  int qpos;           // query row + (Sk - Sq): position compared with keys
  int row_lo;         // first allowed key of this lane's row
  int row_span;       // number of allowed keys from row_lo (0: empty row)
  int doc;            // document id of this lane's row
  bool has_doc;
};

// Key offset (within a 64-key tile, relative to 4*g) of S^T register r of
// 32-key half kb: rows 8*(r/4) + r%4 of the 32x32 accumulator.
__device__ __forceinline__ constexpr int koff(int kb, int r) { return 32 * kb + 8 * (r >> 2) + (r & 3); }

// One 64-key tile: S^T = K Q^T, online softmax update, O^T += V^T P^T.
// MASKED evaluates the mask predicate per element (partial tiles only).
template <typename T, int D, int MOD, bool MASKED>
__device__ __forceinline__ void fwd_tile(const char* kb_base, const char* vb_base,
                                         const int* doc_t, const typename T::vec8 (&qf)[D / 16],
                                         f32x16 (&oacc)[D / 32], float& m_run, float& l_run,
                                         const TileCtx& cx, int key_base, int lane) {
  using C = FwdCfg<D>;
  constexpr bool kAlibi = MOD & 1;
  constexpr bool kSoftcap = MOD & 2;
  constexpr bool kScaled = kAlibi || kSoftcap;
  const int g = lane >> 5, c = lane & 31;

  // S^T for the two 32-key halves.  The two accumulators are updated in
  // alternation so consecutive MFMAs never depend on each other (a dependent
  // accumulation waits for the previous MFMA to drain).
  f32x16 sacc[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.0f;
#pragma unroll
  for (int ds = 0; ds < C::DSTEPS; ds += 2) {
    typename T::vec8 ka[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int u = 0; u < 2; ++u)
        ka[kb][u] = *reinterpret_cast<const typename T::vec8*>(kb_base + C::L::off(32 * kb + c, 2 * (ds + u) + g));
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) sacc[kb] = mfma32(ka[kb][u], qf[ds + u], sacc[kb]);
  }

  // Scores in the exp2 domain (raw dot products when no modifier: the
  // positive scale is then applied inside the exponent).
  if (kScaled) {
    const float dist_base = static_cast<float>(cx.qpos - key_base - 4 * g);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float x;
        if (kSoftcap) {
          // softcap * tanh(scale * s / softcap); tanh(y) = 1 - 2 / (e^{2y} + 1)
          const float e = fast_exp2(sacc[kb][r] * cx.cap_k2);
          x = cx.cap_log2 * (1.0f - 2.0f * fast_rcp(e + 1.0f));
        } else {
          x = sacc[kb][r] * cx.scale_log2;
        }
        if (kAlibi)
          x = __builtin_fmaf(-cx.slope_log2, fabsf(dist_base - static_cast<float>(koff(kb, r))), x);
        sacc[kb][r] = x;
      }
  }
  if (MASKED) {
    // allowed <=> 0 <= key - row_lo < row_span (unsigned compare), and the
    // same document when a document mask is given.
    const uint32_t span = static_cast<uint32_t>(cx.row_span);
    const int jb = key_base + 4 * g - cx.row_lo;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        int4 dk = make_int4(0, 0, 0, 0);
        if (cx.has_doc) dk = *reinterpret_cast<const int4*>(doc_t + 4 * g + 32 * kb + 8 * rr);
        const int dks[4] = {dk.x, dk.y, dk.z, dk.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * rr + e;
          bool ok = static_cast<uint32_t>(jb + koff(kb, r)) < span;
          if (cx.has_doc) ok = ok && dks[e] == cx.doc;
          sacc[kb][r] = ok ? sacc[kb][r] : kNegInf;
        }
      }
  }

  // Row maximum: tree over this lane's 32 values, then lane l ^ 32.
  float m4[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    m4[i] = fmaxf(fmaxf(fmaxf(sacc[0][i], sacc[0][i + 4]), fmaxf(sacc[0][i + 8], sacc[0][i + 12])),
                  fmaxf(fmaxf(sacc[1][i], sacc[1][i + 4]), fmaxf(sacc[1][i + 8], sacc[1][i + 12])));
  float mx = fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3]));
  mx = fmaxf(mx, wave_xor32(mx));
  const float mx2 = kScaled ? mx : mx * cx.scale_log2;  // -inf stays -inf
  if (__any(mx2 > m_run + kRescaleThreshold)) {
    const float m_new = fmaxf(m_run, mx2);
    const float alpha = (m_run == kNegInf) ? 0.0f : fast_exp2(m_run - m_new);
    l_run *= alpha;
#pragma unroll
    for (int db = 0; db < C::DBLK; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
    m_run = m_new;
  }
  const float msub = (m_run == kNegInf) ? 0.0f : m_run;

  // P = exp2(x - m), rounded to the input type as the B operand of O^T += V^T P^T.
  typename T::vec8 pf[2][2];
  float ls[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p = kScaled ? fast_exp2(sacc[kb][r] - msub)
                              : fast_exp2(__builtin_fmaf(sacc[kb][r], cx.scale_log2, -msub));
      ls[r & 3] += p;
      pf[kb][r >> 3][r & 7] = static_cast<typename T::elem>(p);
    }
  l_run += (ls[0] + ls[1]) + (ls[2] + ls[3]);

  // O^T += V^T P^T; V^T fragments by transposed LDS reads.  For each
  // 16-key step the D/32 output blocks are independent accumulators, issued
  // back to back.
  const int beta = lane >> 4, s16 = lane & 15;
  const int tr_row = 4 * (beta >> 1) + (s16 >> 2);
  const int tr_chunk = 2 * (beta & 1) + ((s16 & 3) >> 1);
  const int tr_half = 8 * (s16 & 1);
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    typename T::vec8 va[C::DBLK];
#pragma unroll
    for (int db = 0; db < C::DBLK; ++db) {
      const char* p0 = vb_base + C::L::off(16 * kk + tr_row, 4 * db + tr_chunk) + tr_half;
      const char* p1 = vb_base + C::L::off(16 * kk + 8 + tr_row, 4 * db + tr_chunk) + tr_half;
      va[db] = cat_frag<typename T::vec8>(lds_read_tr16(reinterpret_cast<const bf16_t*>(p0)),
                        lds_read_tr16(reinterpret_cast<const bf16_t*>(p1)));
    }
#pragma unroll
    for (int db = 0; db < C::DBLK; ++db) oacc[db] = mfma32(va[db], pf[kk >> 1][kk & 1], oacc[db]);
  }
}

// NW waves of 32 query rows: 4 (128 rows, two workgroups per CU) or 8 (256
// rows, one workgroup per CU; each K/V tile copied to LDS feeds twice the
// query rows, halving the L2-to-LDS traffic per flop).
template <typename T, int D, int MOD, int NW>  // MOD bit 0: ALiBi, bit 1: softcap
__global__ __launch_bounds__(64 * NW, 8 / NW) void fwd_bf16_kernel(FwdArgs a) {
  using C = FwdCfg<D, NW>;
  constexpr bool kAlibi = MOD & 1;
  constexpr bool kSoftcap = MOD & 2;

  // Two distinct LDS objects per operand (not one array indexed by the
  // buffer): alias analysis can then see that the direct global->LDS copy of
  // the next tile does not touch the buffer being read, and no wait for the
  // copy is placed before the reads of the current tile.
  __shared__ __attribute__((aligned(16))) char lds_k0[C::TB];
  __shared__ __attribute__((aligned(16))) char lds_k1[C::TB];
  __shared__ __attribute__((aligned(16))) char lds_v0[C::TB];
  __shared__ __attribute__((aligned(16))) char lds_v1[C::TB];
  __shared__ int lds_doc0[C::BN];
  __shared__ int lds_doc1[C::BN];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5;   // k-group of the MFMA operands
  const int c = lane & 31;   // column (query) of S^T / O^T

  // Heaviest query tiles first (causal work grows with the tile index); the
  // head index is permuted so that consecutive workgroups, which the
  // dispatcher places on different XCDs, keep one GQA group per XCD.
  const int nqt = (a.Sq + C::BM - 1) / C::BM;
  const int per_qt = a.Hq * a.B;
  const int bid = blockIdx.x;
  const int qt = nqt - 1 - bid / per_qt;
  const int rem = bid % per_qt;
  const int b = rem / a.Hq;
  int h = rem % a.Hq;
  if ((a.Hq & 7) == 0) h = (h & 7) * (a.Hq >> 3) + (h >> 3);
  const int G = a.Hq / a.Hkv;
  const int kvh = h / G;

  const bf16_t* qp = static_cast<const bf16_t*>(a.q) + b * a.q_sb + h * a.q_sh;
  const bf16_t* kp = static_cast<const bf16_t*>(a.k) + b * a.k_sb + kvh * a.k_sh;
  const bf16_t* vp = static_cast<const bf16_t*>(a.v) + b * a.v_sb + kvh * a.v_sh;

  const int my_q = qt * C::BM + wave * 32 + c;
  const bool q_ok = my_q < a.Sq;

  // Q fragments (B operand): column my_q, d = 16*ds + 8*g .. +7.  A negative
  // scale is folded into Q by an exact sign flip so the exponent scale is
  // positive and row maxima can be taken on the raw dot products.
  const float scale_abs = fabsf(a.scale);
  const uint32_t sign_flip = a.scale < 0.0f ? 0x80008000u : 0u;
  typename T::vec8 qf[C::DSTEPS];
#pragma unroll
  for (int ds = 0; ds < C::DSTEPS; ++ds) {
    if (q_ok) {
      uint4 raw = *reinterpret_cast<const uint4*>(qp + (int64_t)my_q * a.q_ss + 16 * ds + 8 * g);
      raw.x ^= sign_flip; raw.y ^= sign_flip; raw.z ^= sign_flip; raw.w ^= sign_flip;
      qf[ds] = __builtin_bit_cast(typename T::vec8, raw);
    } else {
      qf[ds] = zero_frag<typename T::vec8>();
    }
  }

  const float scale_log2 = scale_abs * kLog2e;
  float slope_log2 = 0.0f;
  if (kAlibi) slope_log2 = a.alibi[b * a.alibi_sb + h] * kLog2e;
  const float cap = a.softcap;
  const float cap_k2 = kSoftcap ? 2.0f * kLog2e * scale_abs / cap : 0.0f;
  const float cap_log2 = cap * kLog2e;

  // Tile schedule: dense (causal / window interval) or block-mask lists.
  const RowWindow win(a.Sq, a.Sk, a.mask.causal, a.mask.wl, a.mask.wr);
  const TileRange range(win, qt, C::BM, C::BN);
  const bool sparse = a.tiles.kv_num_full != nullptr;
  int n_full = 0, ntiles;
  const int32_t* idx_full = nullptr;
  const int32_t* idx_part = nullptr;
  if (sparse) {
    const int row = b * a.tiles.nQ + qt;
    n_full = a.tiles.kv_num_full[row];
    const int n_part = a.tiles.kv_num_partial[row];
    idx_full = a.tiles.kv_idx_full + (int64_t)row * a.tiles.nK;
    idx_part = a.tiles.kv_idx_partial + (int64_t)row * a.tiles.nK;
    ntiles = (n_full + n_part) * a.tiles.sub;
  } else {
    ntiles = range.kt_end - range.kt_begin;
  }
  // Tiles in processing order: all FULL tiles first, then the PARTIAL ones.
  const int nfull_tiles = sparse ? n_full * a.tiles.sub : range.n_full();
  auto tile_at = [&](int t) -> Tile {
    Tile r;
    if (!sparse) {
      r.kt = range.kt_at(t);
      r.full = t < nfull_tiles;
    } else {
      const int mt = t / a.tiles.sub, sb = t % a.tiles.sub;
      if (mt < n_full) {
        r.kt = idx_full[mt] * a.tiles.sub + sb;
        r.full = true;
      } else {
        r.kt = idx_part[mt - n_full] * a.tiles.sub + sb;
        r.full = false;
      }
    }
    return r;
  };

  const bool has_doc = a.mask.doc_q != nullptr;
  const int doc_mine = (has_doc && q_ok) ? a.mask.doc_q[(int64_t)b * a.Sq + my_q] : 0;
  const int delta = a.Sk - a.Sq;

  int doc_r = 0;
  // K and V of tile kt into buffer BUF (direct global->LDS), and this
  // thread's document id of the tile into a register.
  auto load_tile = [&](int kt, auto buf_tag) {
    constexpr int BUF = decltype(buf_tag)::value;
    char* kdst = BUF ? lds_k1 : lds_k0;
    char* vdst = BUF ? lds_v1 : lds_v0;
    tile_dma<D, NW>(reinterpret_cast<bf16_t*>(kdst), kp, a.k_ss, kt * C::BN, a.Sk, wave, lane);
    tile_dma<D, NW>(reinterpret_cast<bf16_t*>(vdst), vp, a.v_ss, kt * C::BN, a.Sk, wave, lane);
    if (has_doc && tid < C::BN) {
      const int key = kt * C::BN + tid;
      doc_r = key < a.Sk ? a.mask.doc_k[(int64_t)b * a.Sk + key] : -1;
    }
  };
  auto store_doc = [&](auto buf_tag) {
    constexpr int BUF = decltype(buf_tag)::value;
    if (has_doc && tid < C::BN) (BUF ? lds_doc1 : lds_doc0)[tid] = doc_r;
  };
  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;

  uint8_t* trace_row = nullptr;
  if (a.trace != nullptr && tid == 0)
    trace_row = a.trace + ((int64_t)(b * a.Hq + h) * a.nQt + qt) * a.nKt;

  float m_run = kNegInf;  // running max (exp2 domain), shared by lanes c, c+32
  float l_run = 0.0f;     // this lane's partial row sum
  f32x16 oacc[C::DBLK];
#pragma unroll
  for (int db = 0; db < C::DBLK; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.0f;

  if (ntiles > 0) {
    load_tile(tile_at(0).kt, B0{});
    store_doc(B0{});
  }
  wait_dma();
  __syncthreads();

  // Per-row allowed key interval [lo, lo + span) for partial tiles; an empty
  // row (or a row past Sq) has span 0.
  int row_lo = 0, row_span = 0;
  if (q_ok && win.row_nonempty(my_q)) {
    row_lo = win.lo(my_q);
    row_span = win.hi(my_q) - row_lo + 1;
  }
  const TileCtx ctx{scale_log2, slope_log2, cap_k2, cap_log2, my_q + delta, row_lo, row_span,
                    doc_mine, has_doc};

  // Tile t lives in buffer t % 2.  Loops are unrolled by two so the buffer
  // is a compile-time choice, and full and partial tiles have loops of their
  // own, so each loop body is one instantiation and the accumulators keep
  // their registers across iterations.
  auto step = [&](int t, auto buf_tag, auto masked) {
    constexpr int BUF = decltype(buf_tag)::value;
    using NEXT = std::integral_constant<int, 1 - BUF>;
    const Tile cur = tile_at(t);
    const bool has_next = t + 1 < ntiles;
    if (has_next) load_tile(tile_at(t + 1).kt, NEXT{});
    if (trace_row != nullptr) {
      if (!sparse) trace_row[cur.kt] = cur.full ? 2 : 1;
      else if (cur.kt % a.tiles.sub == 0) trace_row[cur.kt / a.tiles.sub] = cur.full ? 2 : 1;
    }
    fwd_tile<T, D, MOD, decltype(masked)::value>(BUF ? lds_k1 : lds_k0, BUF ? lds_v1 : lds_v0,
                                              BUF ? lds_doc1 : lds_doc0, qf, oacc, m_run, l_run,
                                              ctx, cur.kt * C::BN, lane);
    if (has_next) store_doc(NEXT{});
    wait_dma();
    __syncthreads();
  };
  using FULL = std::false_type;
  using PART = std::true_type;
  int t = 0;
  for (; t + 1 < nfull_tiles; t += 2) {
    step(t, B0{}, FULL{});
    step(t + 1, B1{}, FULL{});
  }
  if (t < nfull_tiles) step(t++, B0{}, FULL{});
  if (t < ntiles && (t & 1)) step(t++, B1{}, PART{});
  for (; t + 1 < ntiles; t += 2) {
    step(t, B0{}, PART{});
    step(t + 1, B1{}, PART{});
  }
  if (t < ntiles) step(t++, B0{}, PART{});

  // ---- epilogue: O = acc / l, LSE = (m + log2 l) ln 2
  const float l_tot = l_run + wave_xor32(l_run);
  if (q_ok) {
    const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
    bf16_t* op = static_cast<bf16_t*>(a.o) + b * a.o_sb + (int64_t)my_q * a.o_ss + h * a.o_sh;
#pragma unroll
    for (int db = 0; db < C::DBLK; ++db) {
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int d0 = 32 * db + 8 * rr + 4 * g;
        uint2 packed;
        packed.x = f32_to_elem<T>(oacc[db][4 * rr + 0] * inv) | (uint32_t)f32_to_elem<T>(oacc[db][4 * rr + 1] * inv) << 16;
        packed.y = f32_to_elem<T>(oacc[db][4 * rr + 2] * inv) | (uint32_t)f32_to_elem<T>(oacc[db][4 * rr + 3] * inv) << 16;
        *reinterpret_cast<uint2*>(op + d0) = packed;
      }
    }
    if (g == 0)
      a.lse[((int64_t)b * a.Hq + h) * a.Sq + my_q] =
          l_tot > 0.0f ? (m_run + fast_log2(l_tot)) * kLn2 : kNegInf;
  }
}

template <typename T, int D, int NW>
hipError_t launch_d(const FwdArgs& a, hipStream_t s) {
  const int bm = 32 * NW;
  const int nqt = (a.Sq + bm - 1) / bm;
  const dim3 grid(nqt * a.Hq * a.B), block(64 * NW);
  const int mod = (a.alibi != nullptr ? 1 : 0) | (a.softcap > 0.0f ? 2 : 0);
  switch (mod) {
    case 0: hipLaunchKernelGGL((fwd_bf16_kernel<T, D, 0, NW>), grid, block, 0, s, a); break;
    case 1: hipLaunchKernelGGL((fwd_bf16_kernel<T, D, 1, NW>), grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL((fwd_bf16_kernel<T, D, 2, NW>), grid, block, 0, s, a); break;
    default: hipLaunchKernelGGL((fwd_bf16_kernel<T, D, 3, NW>), grid, block, 0, s, a); break;
  }
  return hipGetLastError();
}

}  // namespace

int fwd_bf16_rows_per_block(int B, int Sq, int Hq, int causal, bool sparse) {
  if (sparse) return 128;
  const long wg256 = (long)((Sq + 255) / 256) * Hq * B;
  // 256-row workgroups fill the GPU with one workgroup per CU; with causal
  // masks per-tile work differs, so they are only used when there are enough
  // tiles to even it out.
  if (wg256 >= 256 && (!causal || wg256 >= 1024)) return 256;
  return 128;
}

hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t s) {
  if (a.Sq == 0 || a.B == 0 || a.Hq == 0) return hipSuccess;
  const bool sparse = a.tiles.kv_num_full != nullptr;
  const bool wide = fwd_bf16_rows_per_block(a.B, a.Sq, a.Hq, a.mask.causal, sparse) == 256;
  if (a.f16) {
    if (a.D == 64) return wide ? launch_d<F16T, 64, 8>(a, s) : launch_d<F16T, 64, 4>(a, s);
    return wide ? launch_d<F16T, 128, 8>(a, s) : launch_d<F16T, 128, 4>(a, s);
  }
  if (a.D == 64) return wide ? launch_d<Bf16T, 64, 8>(a, s) : launch_d<Bf16T, 64, 4>(a, s);
  return wide ? launch_d<Bf16T, 128, 8>(a, s) : launch_d<Bf16T, 128, 4>(a, s);
}

}  // namespace attn
