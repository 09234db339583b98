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

// NW waves in NG groups; each group owns all BM rows (32 per wave) and takes
// every NG-th key tile (in-workgroup split over the keys when NG = 2).
template <int D, int NW = 4, int NG = 1>
struct FwdCfg {
  static constexpr int WPG = NW / NG;      // waves per group
  static constexpr int BM = 32 * WPG;      // query rows per workgroup (32 per wave)
  static constexpr int BN = kFwdBN;        // keys per tile
  static constexpr int NT = 64 * NW;       // threads
  static constexpr int GT = 64 * WPG;      // threads per group
  // Workgroups per CU the register budget is sized for: three 4-wave
  // workgroups at D = 64 (at most 168 VGPRs, three waves per SIMD), else
  // 8 waves per CU.
  static constexpr int MINB = (D == 64 && NW == 4) ? 3 : 8 / NW;
  using L = TileLayout<D>;                 // LDS image of a 64-key K or V tile
  static constexpr int TB = L::BYTES;      // bytes per tile buffer
  static constexpr int DSTEPS = D / 16;
  static constexpr int DBLK = D / 32;
};

struct Tile {
  int kt;
  bool full;
};


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
// LEAN: the kernel runs at the 168-register budget (three workgroups per
// CU), so fewer LDS fragments are read ahead.
template <typename T, int D, int MOD, bool MASKED, bool LEAN>
__device__ __forceinline__ void fwd_tile(const char* kb_base, const char* vb_base,
                                         const int* doc_t, const typename T::vec8 (&qf)[D / 16],
                                         f32x16 (&oacc)[D / 32], float& m_run, float& l_run,
                                         const TileCtx& cx, int key_base, int lane) {
  using C = FwdCfg<D>;
  constexpr bool kAlibi = MOD & 1;
  constexpr bool kSoftcap = MOD & 2;
  constexpr bool kScaled = kAlibi || kSoftcap;
  const int g = lane >> 5, c = lane & 31;

  // S^T for the two 32-key halves.  MFMA i (i = 2*ds + kb) takes K fragment
  // (key half kb, d-step ds); the two accumulators alternate so consecutive
  // MFMAs never depend on each other.  The K fragments are read from LDS
  // kSPF MFMAs ahead: the scheduling groups below fix the order "kSPF reads,
  // then (one MFMA, one read) pairs, then the last MFMAs", so each MFMA waits
  // only for a read issued kSPF MFMAs earlier instead of one round trip per
  // MFMA.
  constexpr int kNS = 2 * C::DSTEPS;            // S MFMAs per tile
  constexpr int kSPF = kNS < 8 ? kNS : 8;       // K reads in flight
  f32x16 sacc[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.0f;
  typename T::vec8 kf[kNS];
#pragma unroll
  for (int i = 0; i < kNS; ++i)
    kf[i] = *reinterpret_cast<const typename T::vec8*>(kb_base + C::L::off(32 * (i & 1) + c, 2 * (i >> 1) + g));
#pragma unroll
  for (int i = 0; i < kNS; ++i) sacc[i & 1] = mfma32(kf[i], qf[i >> 1], sacc[i & 1]);

  // V^T fragments of the first PV steps are read now, behind the K reads:
  // they do not depend on the softmax, so they land while it runs.
  // Fragment f = kk * DBLK + db: keys 16*kk.., output block db.
  constexpr int kNV = 4 * C::DBLK;              // PV MFMAs per tile
  constexpr int kVPF = LEAN ? 0 : C::DBLK;      // V fragments read ahead
  const int beta = lane >> 4, s16 = lane & 15;
  const int tr_row = 4 * (beta >> 1) + (s16 >> 2);
  const int tr_chunk = 2 * (beta & 1) + ((s16 & 3) >> 1);
  const int tr_half = 8 * (s16 & 1);
  auto vfrag = [&](int f) __attribute__((always_inline)) {
    const int kk = f / C::DBLK, db = f % C::DBLK;
    const char* p0 = vb_base + C::L::off(16 * kk + tr_row, 4 * db + tr_chunk) + tr_half;
    const char* p1 = vb_base + C::L::off(16 * kk + 8 + tr_row, 4 * db + tr_chunk) + tr_half;
    return cat_frag<typename T::vec8>(lds_read_tr16(reinterpret_cast<const bf16_t*>(p0)),
                                      lds_read_tr16(reinterpret_cast<const bf16_t*>(p1)));
  };
  typename T::vec8 vf[kNV];
#pragma unroll
  for (int f = 0; f < kVPF; ++f) vf[f] = vfrag(f);

  // (At the 168-register budget the compiler's own order is kept: reads
  // ahead cost registers there, and spills cost more than the waits.)
  if constexpr (!LEAN) {
    __builtin_amdgcn_sched_group_barrier(0x100, kSPF, 0);
#pragma unroll
    for (int i = 0; i < kNS - kSPF; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, kSPF, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * kVPF, 0);
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
    // same document.  Without a document mask every key and row carries
    // document 0, so the test is the same straight-line select either way
    // (a test guarded by has_doc was compiled as a branch per element).
    const uint32_t span = static_cast<uint32_t>(cx.row_span);
    const int jb = key_base + 4 * g - cx.row_lo;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int4 dk = *reinterpret_cast<const int4*>(doc_t + 4 * g + 32 * kb + 8 * rr);
        const int dks[4] = {dk.x, dk.y, dk.z, dk.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * rr + e;
          const bool ok = (static_cast<uint32_t>(jb + koff(kb, r)) < span) & (dks[e] == cx.doc);
          sacc[kb][r] = ok ? sacc[kb][r] : kNegInf;
        }
      }
  }

  // Row maximum over this lane's 32 values, then lane l ^ 32.  The first
  // read of the accumulators is a compiled fmaxf, which carries the wait
  // states after the MFMAs that wrote them; every three-input max in
  // assembly after it depends on its result, so none is placed before it.
  // (Compiled fmaxf in IEEE mode also quiets every operand first: 18
  // instructions here against about 47.)
  float v[32];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    v[r] = sacc[0][r];
    v[16 + r] = sacc[1][r];
  }
  float mc[4];
  mc[0] = fmaxf(v[0], v[16]);
  mc[1] = max3_nc(mc[0], v[1], v[2]);
  mc[2] = max3_nc(mc[0], v[3], v[4]);
  mc[3] = max3_nc(mc[0], v[5], v[6]);
  // the other 24 values (7..15, 17..31) in pairs over the four chains
#pragma unroll
  for (int j = 0; j < 12; ++j) {
    const int i0 = 7 + 2 * j < 16 ? 7 + 2 * j : 8 + 2 * j;   // 7, 9, 11, 13, 15, 17, ...
    const int i1 = 7 + 2 * j + 1 < 16 ? 7 + 2 * j + 1 : 8 + 2 * j + 1;
    mc[j & 3] = max3_nc(mc[j & 3], v[i0], v[i1]);
  }
  float mx = max_nc(max3_nc(mc[0], mc[1], mc[2]), mc[3]);
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

  // O^T += V^T P^T; V^T fragments by transposed LDS reads, kVPF fragments
  // ahead of their MFMA (the first kVPF were read before the softmax).  For
  // each 16-key step the D/32 output blocks are independent accumulators,
  // issued back to back.
#pragma unroll
  for (int f = kVPF; f < kNV; ++f) vf[f] = vfrag(f);
#pragma unroll
  for (int f = 0; f < kNV; ++f) {
    const int kk = f / C::DBLK, db = f % C::DBLK;
    oacc[db] = mfma32(vf[f], pf[kk >> 1][kk & 1], oacc[db]);
  }
  if constexpr (!LEAN) {
#pragma unroll
    for (int f = 0; f < kNV - kVPF; ++f) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, kVPF, 1);
  }
}

// NW waves of 32 query rows: 4 (128 rows, two workgroups per CU), 8 in one
// group (256 rows, one workgroup per CU; each K/V tile copied to LDS feeds
// twice the query rows, halving the L2-to-LDS traffic per flop), or 8 in two
// groups (NG = 2: 128 rows, the two groups take alternate key tiles and merge
// their softmax states through LDS at the end).  With one workgroup per CU
// the dispatcher hands out workgroups as CUs free up, so heaviest-first
// order balances causal work; two 4-wave workgroups per CU are all placed at
// once, pairing fixed tiles on a CU.
template <typename T, int D, int MOD, int NW, int NG>  // MOD bit 0: ALiBi, bit 1: softcap
__global__ __launch_bounds__(64 * NW, (FwdCfg<D, NW, NG>::MINB)) void fwd_bf16_kernel(FwdArgs a) {
  using C = FwdCfg<D, NW, NG>;
  constexpr bool kAlibi = MOD & 1;
  constexpr bool kSoftcap = MOD & 2;

  // Two distinct LDS objects per operand (not one array indexed by the
  // buffer): alias analysis can then see that the direct global->LDS copy of
  // the next tile does not touch the buffer being read, and no wait for the
  // copy is placed before the reads of the current tile.
  // (One slice of TB bytes per group in each.)
  __shared__ __attribute__((aligned(16))) char lds_k0_[NG * C::TB];
  __shared__ __attribute__((aligned(16))) char lds_k1_[NG * C::TB];
  __shared__ __attribute__((aligned(16))) char lds_v0_[NG * C::TB];
  __shared__ __attribute__((aligned(16))) char lds_v1_[NG * C::TB];
  __shared__ int lds_doc0_[NG * C::BN];
  __shared__ int lds_doc1_[NG * C::BN];
  __shared__ int lds_gsync_[NG];  // arrivals of each group's waves at its step barriers
  __shared__ int lds_broken_;     // a step barrier wait expired (results are poisoned)

  const int tid_wg = threadIdx.x;
  const int wave_wg = __builtin_amdgcn_readfirstlane(tid_wg >> 6);
  const int grp = NG > 1 ? wave_wg / C::WPG : 0;  // key-tile group
  const int tid = tid_wg - grp * C::GT;           // thread / wave index within the group
  const int wave = wave_wg - grp * C::WPG;
  const int lane = tid & 63;
  const int g = lane >> 5;   // k-group of the MFMA operands
  const int c = lane & 31;   // column (query) of S^T / O^T
  char* const lds_k0 = lds_k0_ + grp * C::TB;
  char* const lds_k1 = lds_k1_ + grp * C::TB;
  char* const lds_v0 = lds_v0_ + grp * C::TB;
  char* const lds_v1 = lds_v1_ + grp * C::TB;
  int* const lds_doc0 = lds_doc0_ + grp * C::BN;
  int* const lds_doc1 = lds_doc1_ + grp * C::BN;

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
  uint4 raw[C::DSTEPS];
  const int q_row = q_ok ? my_q : a.Sq - 1;
#pragma unroll
  for (int ds = 0; ds < C::DSTEPS; ++ds) {
    // All loads first, unconditionally (a row past Sq reads row Sq - 1 and
    // is zeroed below): loads guarded one by one were issued as a chain of
    // round trips, each waited for before the next.
    raw[ds] = *reinterpret_cast<const uint4*>(qp + (int64_t)q_row * a.q_ss + 16 * ds + 8 * g);
  }
#pragma unroll
  for (int ds = 0; ds < C::DSTEPS; ++ds) {
    uint4 r = raw[ds];
    r.x = q_ok ? r.x ^ sign_flip : 0u;
    r.y = q_ok ? r.y ^ sign_flip : 0u;
    r.z = q_ok ? r.z ^ sign_flip : 0u;
    r.w = q_ok ? r.w ^ sign_flip : 0u;
    qf[ds] = __builtin_bit_cast(typename T::vec8, r);
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
  // Copies issued from inline assembly: with the builtin, the compiler counts
  // the pending copies as LDS traffic of unknown order and waits for every
  // LDS read in full (lgkmcnt(0)), which serialises the fragment reads.
  // (Not at the 168-register budget, where the copies' 64-bit addresses,
  // which the builtin folds into its offset field, cost registers.)
  constexpr bool kAsmCopy = C::MINB < 3;
  const TileCopy<D, C::WPG, kAsmCopy> kcopy(kp, a.k_ss, a.Sk, wave, lane);
  const TileCopy<D, C::WPG, kAsmCopy> vcopy(vp, a.v_ss, a.Sk, wave, lane);
  // K and V of tile kt into buffer BUF (direct global->LDS), and this
  // thread's document id of the tile into a register.
  auto load_tile = [&](int kt, auto buf_tag) {
    constexpr int BUF = decltype(buf_tag)::value;
    char* kdst = BUF ? lds_k1 : lds_k0;
    char* vdst = BUF ? lds_v1 : lds_v0;
    kcopy(reinterpret_cast<bf16_t*>(kdst), kt * C::BN);
    vcopy(reinterpret_cast<bf16_t*>(vdst), kt * C::BN);
    if (has_doc && tid < C::BN) {
      const int key = kt * C::BN + tid;
      doc_r = key < a.Sk ? a.mask.doc_k[(int64_t)b * a.Sk + key] : -1;
    }
  };
  auto store_doc = [&](auto buf_tag) {
    constexpr int BUF = decltype(buf_tag)::value;
    if (tid < C::BN) (BUF ? lds_doc1 : lds_doc0)[tid] = doc_r;  // 0 without documents
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

  // Group grp takes tiles grp, grp + NG, ...: step s of the group is tile
  // NG * s + grp.  Both groups run the same number of steps (one barrier
  // each); a group past its last tile only takes part in the barriers.
  if (grp < ntiles) {
    load_tile(tile_at(grp).kt, B0{});
    store_doc(B0{});
  }
  if (tid_wg < NG) lds_gsync_[tid_wg] = 0;
  if (tid_wg == 0) lds_broken_ = 0;
  wait_dma();
  __syncthreads();

  // With two groups, each group ends its steps with a barrier of its own
  // four waves (an arrival count in LDS, bounded spin), so the groups do not
  // run in lockstep and one group's softmax can overlap the other's matrix
  // work on the same SIMD.  The tile buffers are per group, so a group
  // barrier orders everything a step needs: copies landed before reads, and
  // reads of a buffer done before the next copy into it.
  // The wait is bounded (a.spin_limit sleeps); if it expires the tiles may
  // not have landed, so the workgroup's rows are written as NaN at the end.
  int nsync = 0;
  bool broken = false;
  auto step_sync = [&]() __attribute__((always_inline)) {
    if constexpr (NG == 1) {
      __syncthreads();
    } else {
      ++nsync;
      if (lane == 0) __hip_atomic_fetch_add(&lds_gsync_[grp], 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
      const int target = C::WPG * nsync;
      for (int n = 0;; ++n) {
        const int v = __builtin_amdgcn_readfirstlane(
            __hip_atomic_load(&lds_gsync_[grp], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP));
        if (v >= target) break;
        if (n >= a.spin_limit) {
          broken = true;
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
    }
  };

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
  auto step = [&](int s, auto buf_tag, auto masked) {
    constexpr int BUF = decltype(buf_tag)::value;
    using NEXT = std::integral_constant<int, 1 - BUF>;
    const int t = NG * s + grp;
    const bool has_next = t + NG < ntiles;
    if (has_next) load_tile(tile_at(t + NG).kt, NEXT{});
    if (NG == 1 || t < ntiles) {
      const Tile cur = tile_at(t);
      if (trace_row != nullptr) {
        if (!sparse) trace_row[cur.kt] = cur.full ? 2 : 1;
        else if (cur.kt % a.tiles.sub == 0) trace_row[cur.kt / a.tiles.sub] = cur.full ? 2 : 1;
      }
      fwd_tile<T, D, MOD, decltype(masked)::value, C::MINB >= 3>(BUF ? lds_k1 : lds_k0, BUF ? lds_v1 : lds_v0,
                                                BUF ? lds_doc1 : lds_doc0, qf, oacc, m_run, l_run,
                                                ctx, cur.kt * C::BN, lane);
    }
    if (has_next) store_doc(NEXT{});
    wait_dma();
    step_sync();
  };
  using FULL = std::false_type;
  using PART = std::true_type;
  // Steps of this group: nsteps in all, the first nfull_steps on FULL tiles.
  const int nsteps = (ntiles + NG - 1) / NG;
  const int nfull_steps = nfull_tiles > grp ? (nfull_tiles - grp + NG - 1) / NG : 0;
  int t = 0;
  for (; t + 1 < nfull_steps; t += 2) {
    step(t, B0{}, FULL{});
    step(t + 1, B1{}, FULL{});
  }
  if (t < nfull_steps) step(t++, B0{}, FULL{});
  if (t < nsteps && (t & 1)) step(t++, B1{}, PART{});
  for (; t + 1 < nsteps; t += 2) {
    step(t, B0{}, PART{});
    step(t + 1, B1{}, PART{});
  }
  if (t < nsteps) step(t++, B0{}, PART{});

  if constexpr (NG == 2) {
    // Group 1 hands its running state (max, partial sums, unnormalised O)
    // to group 0 through LDS; wave w of each group owns the same 32 rows.
    // The slots overlap group 0's tile buffers, and the step barriers are per
    // group, so first both groups must be past their last step.
    if (broken) lds_broken_ = 1;
    __syncthreads();
    constexpr int SLOT = 64 * (16 * C::DBLK + 2);  // floats per wave
    static_assert(SLOT * 4 <= C::TB, "state slot fits one tile buffer");
    float* st = reinterpret_cast<float*>((wave < 2 ? lds_k0_ : lds_k1_) + (wave & 1) * C::TB);
    if (grp == 1) {
#pragma unroll
      for (int db = 0; db < C::DBLK; ++db)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
          *reinterpret_cast<float4*>(st + ((db * 4 + rr) * 64 + lane) * 4) =
              make_float4(oacc[db][4 * rr], oacc[db][4 * rr + 1], oacc[db][4 * rr + 2], oacc[db][4 * rr + 3]);
      st[16 * C::DBLK * 64 + lane] = m_run;
      st[16 * C::DBLK * 64 + 64 + lane] = l_run;
    }
    __syncthreads();  // group 1's state is in LDS
    if (grp == 1) return;
    broken = lds_broken_ != 0;
    const float mo = st[16 * C::DBLK * 64 + lane];
    const float lo = st[16 * C::DBLK * 64 + 64 + lane];
    const float M = fmaxf(m_run, mo);
    const float a0 = m_run == kNegInf ? 0.0f : fast_exp2(m_run - M);
    const float a1 = mo == kNegInf ? 0.0f : fast_exp2(mo - M);
    l_run = l_run * a0 + lo * a1;
#pragma unroll
    for (int db = 0; db < C::DBLK; ++db)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const float4 x = *reinterpret_cast<const float4*>(st + ((db * 4 + rr) * 64 + lane) * 4);
        oacc[db][4 * rr] = oacc[db][4 * rr] * a0 + x.x * a1;
        oacc[db][4 * rr + 1] = oacc[db][4 * rr + 1] * a0 + x.y * a1;
        oacc[db][4 * rr + 2] = oacc[db][4 * rr + 2] * a0 + x.z * a1;
        oacc[db][4 * rr + 3] = oacc[db][4 * rr + 3] * a0 + x.w * a1;
      }
    m_run = M;
  }

  // ---- epilogue: O = acc / l, LSE = (m + log2 l) ln 2.  Poisoned rows get
  // NaN bit patterns written as integers.
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
        if (broken) packed = make_uint2(T::kNan2, T::kNan2);
        *reinterpret_cast<uint2*>(op + d0) = packed;
      }
    }
    if (g == 0) {
      const float lse = l_tot > 0.0f ? (m_run + fast_log2(l_tot)) * kLn2 : kNegInf;
      reinterpret_cast<uint32_t*>(a.lse)[((int64_t)b * a.Hq + h) * a.Sq + my_q] =
          broken ? 0x7FC00000u : __float_as_uint(lse);
    }
  }
}

template <typename T, int D, int NW, int NG = 1>
hipError_t launch_d(const FwdArgs& a, hipStream_t s) {
  const int bm = 32 * NW / NG;
  const int nqt = (a.Sq + bm - 1) / bm;
  const dim3 grid(nqt * a.Hq * a.B), block(64 * NW);
  const int mod = (a.alibi != nullptr ? 1 : 0) | (a.softcap > 0.0f ? 2 : 0);
  switch (mod) {
    case 0: hipLaunchKernelGGL((fwd_bf16_kernel<T, D, 0, NW, NG>), grid, block, 0, s, a); break;
    case 1: hipLaunchKernelGGL((fwd_bf16_kernel<T, D, 1, NW, NG>), grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL((fwd_bf16_kernel<T, D, 2, NW, NG>), grid, block, 0, s, a); break;
    default: hipLaunchKernelGGL((fwd_bf16_kernel<T, D, 3, NW, NG>), grid, block, 0, s, a); break;
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

template <typename T, int D>
hipError_t launch_t(const FwdArgs& a, hipStream_t s, bool wide, bool split) {
  if (wide) return launch_d<T, D, 8, 1>(a, s);
  if (split) return launch_d<T, D, 8, 2>(a, s);
  return launch_d<T, D, 4, 1>(a, s);
}

hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t s) {
  if (a.Sq == 0 || a.B == 0 || a.Hq == 0) return hipSuccess;
  const bool sparse = a.tiles.kv_num_full != nullptr;
  const bool wide = fwd_bf16_rows_per_block(a.B, a.Sq, a.Hq, a.mask.causal, sparse) == 256;
  // 128-row tiles split over the keys in the workgroup when the grid is small
  // (up to about 8 tiles per CU): placed two per CU, 4-wave workgroups would
  // all be dispatched at once with fixed pairs of uneven causal tiles.
  const long wg128 = (long)((a.Sq + 127) / 128) * a.Hq * a.B;
  const bool split = !wide && !sparse && wg128 <= 2048;
  if (a.f16) return a.D == 64 ? launch_t<F16T, 64>(a, s, wide, split) : launch_t<F16T, 128>(a, s, wide, split);
  return a.D == 64 ? launch_t<Bf16T, 64>(a, s, wide, split) : launch_t<Bf16T, 128>(a, s, wide, split);
}

}  // namespace attn
