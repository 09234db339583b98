// Split-K decode over a KV cache, bf16 or fp16 (gfx950).
//
// flash_attn_with_kvcache ("FlashAttention: Fast and Memory-Efficient Exact
// Attention", "Examples") attends the new queries of each sequence (one, or a
// few for chunked prefill and speculative decoding) to the first
// cache_seqlens[b] rows of that sequence's cache; with several queries they
// are the last positions of the sequence, so causal masking (bottom-right
// aligned) limits query t of Sq to the first L - Sq + 1 + t keys.  The key
// work is split and
// merged with the LSE-weighted combine
//   lse = log sum_s exp(lse_s),   O = sum_s exp(lse_s - lse) O_s
// (the chunk-level form of the online softmax of "Accelerating AI: A Deep
// Dive into Flash Attention", "2. Online Softmax").
//
// Work decomposition.  A job is one (sequence b, kv head, group of up to 128
// rows of that kv head), a row being a (query t, query head) pair numbered
// t * G + head (G query heads per kv head); its keys are cut into 32-key
// steps.  All jobs, in job order, form one list of S units -- each job SEG
// units of segment weight (its query load, state merge and partial write)
// followed by its steps -- that is cut into Pe = min(P, S) equal contiguous
// ranges, one per workgroup (P = one per compute unit by default), so every
// workgroup gets the same work whatever the mix of cache lengths, a
// workgroup that starts a job taking fewer key steps.  A range that spans several jobs
// produces one partial result per job; the partial of job j from workgroup w
// goes to slot w + j (unique, since ranges are ordered).  The workgroups that
// start and end a job record their index for the combine kernel.
//
// Inside a workgroup, 8 consumer waves: head block hb = wave % 4 (32 query
// heads, so each K/V byte read from HBM serves all 128 heads of the job) and
// step parity wave / 4 (the two waves of a head block share a SIMD, take
// alternate 32-key steps and merge their running softmax states through LDS
// at the end of the job's segment).  The query heads play the role of query
// rows of the forward kernel: S^T = K Q^T on the 32x32x16 matrix core.  K/V
// tiles stream through an NS-deep LDS ring filled by direct global->LDS copies
// that 4 producer waves issue and wait for, so the consumers never stall on
// the memory pipeline; each query block is itself a ring item, so the ring
// never drains at a job change.  The hand-over uses LDS counters, not
// barriers: producers and consumers each run at their own pace.

#include <type_traits>

#include "common.h"
#include "internal.h"

namespace attn {
namespace {

constexpr float kNegInf = -__builtin_huge_valf();

template <int D, bool W = false>
struct DecCfg {
  // rows (query, head) per job; W: wide jobs, one 32-row block per consumer
  static constexpr int ROWS = W ? kDecodeRowsWide : kDecodeRows;
  static constexpr int NWC = 8;                       // consumers: 4 head blocks x 2 step parities, or 8 blocks (W)
  static constexpr int NWP = 4;                       // producer waves (copies only)
  static constexpr int NWT = NWC + NWP;
  static constexpr int NT = 64 * NWT;
  static constexpr int BN = 32;                       // keys per ring item
  using L = TileLayout<D>;
  static constexpr int GROUPS = BN / L::RG;           // 1 KB copy groups per 32-row tile
  static constexpr int TB = GROUPS * L::GS;           // bytes of one 32-row tile image
  static constexpr int SB = 2 * TB;                   // ring item: K then V, or 2 query blocks
  static constexpr int NS = D == 128 ? 7 : 15;        // ring depth
  static constexpr int DEPTH = NS - 1;                // items a producer keeps unpublished in flight
  static constexpr int PER = 2 * GROUPS / NWP;        // copies per producer lane per ring item
  // Schedule weight of a job segment (query load, state merge, partial
  // write) in 32-key steps: each job counts SEG extra units in the split, so
  // a workgroup that starts a job takes that many fewer key steps.
  static constexpr int SEG = 4;
  static constexpr int DSTEPS = D / 16;
  static constexpr int DBLK = D / 32;
  // One wave's softmax state handed over at a segment end: the unnormalised
  // output rounded to bf16 (16 * DBLK values per lane, lane-major pairs)
  // and the fp32 row maximum and sum.
  static constexpr int MSLOT = 64 * (16 * DBLK * 2 + 8);  // bytes
};

// Bounded spin on an LDS flag: the waves of a workgroup hand items over with
// counters instead of barriers.  The bound (spin_limit sleeps, about 2^22 by
// default) only matters if the protocol were broken; it keeps every wave
// finite.  Returns false when the bound was reached with the condition still
// false: the caller then marks its results as poisoned.
template <typename Pred>
__device__ __forceinline__ bool spin_until(Pred pred, int limit) {
  for (int n = 0; n < limit; ++n) {
    if (pred()) return true;
    __builtin_amdgcn_s_sleep(1);
  }
  return pred();
}
__device__ __forceinline__ int lds_acquire(const int* p) {
  return __hip_atomic_load(p, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void publish(int* p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ bool spin_until_ge(const int* p, int v, int limit) {
  return spin_until([&] { return lds_acquire(p) >= v; }, limit);
}
// Set bits of the sticky status word (a device-scope vector atomic).
__device__ __forceinline__ void status_or(uint32_t* status, uint32_t bits) {
  __hip_atomic_fetch_or(status, bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ int clamp_len(int L, int smax) { return L < 0 ? 0 : (L > smax ? smax : L); }

// Keys sequence b attends to: its cache length (clamped so that the appended
// rows fit the capacity) plus the appended rows.
__device__ __forceinline__ int seq_len(const DecodeArgs& a, int b) {
  return clamp_len(a.seqlens[b], a.Smax - a.len_add) + a.len_add;
}

// One int32 through the scalar cache (p must be wave-uniform).  Used by the
// producer waves for page and batch-row lookups: a vector load would make
// the compiler wait for all of their outstanding copies.
__device__ __forceinline__ int sload_i32(const int32_t* p) {
  int v;
  asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(p) : "memory");
  return v;
}

// Wait until at most PER * k copies of this lane are outstanding.
template <int PER, int K>
__device__ __forceinline__ void vm_wait_imm() {
  asm volatile("s_waitcnt vmcnt(%0)" :: "n"(PER * K) : "memory");
}
template <int PER, int KMAX>
__device__ __forceinline__ void wait_items(int k) {
  static_assert(PER * KMAX <= 63 && KMAX <= 15, "vmcnt range");
#define ATTN_WAIT_CASE(n) \
  case n: if constexpr (KMAX >= n) { vm_wait_imm<PER, n>(); break; } [[fallthrough]];
  switch (k) {
    ATTN_WAIT_CASE(15)
    ATTN_WAIT_CASE(14)
    ATTN_WAIT_CASE(13)
    ATTN_WAIT_CASE(12)
    ATTN_WAIT_CASE(11)
    ATTN_WAIT_CASE(10)
    ATTN_WAIT_CASE(9)
    ATTN_WAIT_CASE(8)
    ATTN_WAIT_CASE(7)
    ATTN_WAIT_CASE(6)
    ATTN_WAIT_CASE(5)
    ATTN_WAIT_CASE(4)
    ATTN_WAIT_CASE(3)
    ATTN_WAIT_CASE(2)
    ATTN_WAIT_CASE(1)
    default: vm_wait_imm<PER, 0>(); break;
  }
#undef ATTN_WAIT_CASE
}

// Wave-wide sum and inclusive prefix sum of one value per lane.
__device__ __forceinline__ long long wave_sum64(long long v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
// A wave-uniform 64-bit value moved to scalar registers (the compiler cannot
// see that a cross-lane reduction gives every lane the same value).
__device__ __forceinline__ long long uniform64(long long v) {
  const uint64_t u = static_cast<uint64_t>(v);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(u));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(u >> 32));
  return static_cast<long long>((static_cast<uint64_t>(hi) << 32) | lo);
}
__device__ __forceinline__ long long wave_incl_scan64(long long x, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const long long y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  return x;
}

// Position in one workgroup's sequence of ring items: job (hg, b, jb) with
// head group hg, sequence b and kv head jb, key step `step` of that job; `phase` < nq
// for the query-block items that open a job's segment, == nq for K/V items.
struct Cursor {
  int b, jb, step, phase;
  int n, Lb, nq, rows, g_kv, hg;  // of the current job
  int left;                       // K/V steps left in this workgroup's range
};

template <typename T, int D, bool kSoftcap, bool kMulti, bool kWide>
__global__ __launch_bounds__(DecCfg<D>::NT, 1) void decode_split_kernel(DecodeArgs a) {
  using C = DecCfg<D, kWide>;
  using L = typename C::L;
  __shared__ __attribute__((aligned(16))) char ring[C::NS * C::SB];
  __shared__ __attribute__((aligned(16))) char mrg[kWide ? 16 : 4 * C::MSLOT];  // (unused when wide)
  __shared__ int landed[C::NWP];       // items whose copies by producer p have landed
  __shared__ int consumed[C::NWC];     // items consumer wave w is done with
  __shared__ int mrg_written[4], mrg_read[4];  // merge handshakes per head block
  __shared__ int ring_broken;          // some wave's wait expired (its data may be stale)

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool producer = wave >= C::NWC;
  const int hb = wave & 3, par = (wave >> 2) & 1;  // consumer head block and step parity
  // Consumer's 32-row block of the job: wide jobs give each consumer wave a
  // block of its own and every K/V step, so the steps are read once for twice
  // the rows; otherwise the two waves of a head block split the steps.
  const int rb = kWide ? wave : hb;
  const int g = lane >> 5, c = lane & 31;
  const int G = a.Hq / a.Hkv;
  const int R = a.Sq * G;         // rows per kv head
  const int P = gridDim.x;
  const int w_id = blockIdx.x;

  // ---- counters first (zero before anyone publishes), then every wave
  // finds this workgroup's step range [lo, hi) and first job by itself:
  // wave-wide sums and prefix sums over the sequences, 64 at a time, so no
  // workgroup barrier stands between the cache lengths and the first copies.
  if (tid < C::NWP) landed[tid] = 0;
  if (tid < C::NWC) consumed[tid] = 0;
  if (tid < 4) mrg_written[tid] = mrg_read[tid] = 0;
  if (tid == 0) ring_broken = 0;
  __syncthreads();
  // Lengths of sequences c*64 .. c*64 + 63 for chunk c, one per lane; chunk
  // 0 is loaded once and kept (a workgroup's range rarely goes past it).
  auto lens_chunk = [&](int c) -> int { return c * 64 + lane < a.B ? seq_len(a, c * 64 + lane) : 0; };
  const int len0 = lens_chunk(0);
  // Jobs are listed head group first (all sequences' jobs of head group 0,
  // then of group 1, ...), so with P a multiple of the group count the
  // workgroups w, w + P/nhg, ... cover the same keys of the same sequence for
  // the different query heads at the same time (one pass over the keys from
  // memory, the others from cache).  Units of a sequence within one head
  // group: Hkv jobs of (steps + SEG).
  auto units_of = [&](int L) -> long long {
    const int n = (L + C::BN - 1) / C::BN;
    return n > 0 ? (long long)(n + C::SEG) * a.Hkv : 0;
  };
  long long S1 = wave_sum64(units_of(len0));
  for (int c = 1; c * 64 < a.B; ++c) S1 += wave_sum64(units_of(lens_chunk(c)));
  S1 = uniform64(S1);
  const long long S = S1 * a.nhg;
  const int Pe = S < P ? (int)S : P;
  if (w_id >= Pe) return;  // the same for every wave of the workgroup
  const long long lo = (long long)w_id * S / Pe;
  const long long hi = (long long)(w_id + 1) * S / Pe;
  // The head group, the sequence whose units contain lo, and the offset of
  // lo inside them.
  const int hg0 = static_cast<int>(lo / S1);
  const long long lo1 = lo - hg0 * S1;
  int b0 = 0;
  long long off0 = 0;
  {
    long long carry = 0;
    for (int c = 0; c * 64 < a.B; ++c) {
      const long long u = units_of(c == 0 ? len0 : lens_chunk(c));
      const long long incl = carry + wave_incl_scan64(u, lane);
      const uint64_t hit = __ballot(u > 0 && incl - u <= lo1 && lo1 < incl);
      if (hit != 0) {
        const int src = __builtin_ctzll(hit);
        b0 = c * 64 + src;
        const long long excl = __shfl(incl, src, 64) - __shfl(u, src, 64);
        // (wave-uniform; readfirstlane tells the compiler so, keeping the
        // cursor in scalar registers)
        off0 = __builtin_amdgcn_readfirstlane(static_cast<int>(lo1 - excl));
        break;
      }
      carry = __shfl(incl, 63, 64);
    }
  }
  b0 = __builtin_amdgcn_readfirstlane(b0);
  // A wait of this wave that expired: its data may be stale, so the rows it
  // contributes to are written as NaN and the status word records it.
  bool broken = false;
  auto note = [&](bool ok) {
    if (!ok) {
      broken = true;
      ring_broken = 1;
    }
  };
  // Minimum of a group of counters: relaxed loads issued together, then one
  // acquire fence (an acquire per load would serialise the LDS round trips).
  auto counters_min = [&](const int* cnt, auto n_tag) {
    constexpr int N = decltype(n_tag)::value;
    int v[N];
#pragma unroll
    for (int q = 0; q < N; ++q) v[q] = __hip_atomic_load(&cnt[q], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    int m = v[0];
#pragma unroll
    for (int q = 1; q < N; ++q) m = min(m, v[q]);
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    return m;
  };
  auto landed_min = [&]() { return counters_min(landed, std::integral_constant<int, C::NWP>{}); };
  auto consumed_min = [&]() { return counters_min(consumed, std::integral_constant<int, C::NWC>{}); };

  auto len_of = [&](int b) -> int {
    return __builtin_amdgcn_readfirstlane(b < 64 ? __shfl(len0, b, 64) : seq_len(a, b));
  };
  auto set_job = [&](Cursor& cu) {
    cu.g_kv = cu.jb;
    cu.rows = min(C::ROWS, R - cu.hg * C::ROWS);
    cu.nq = (cu.rows + 63) / 64;
  };
  // Position of the cursor's job in the list (it orders the partial slots).
  auto job_index = [&](const Cursor& cu) -> int64_t {
    return ((int64_t)cu.hg * a.B + cu.b) * a.Hkv + cu.jb;
  };
  auto start = [&](Cursor& cu) {
    cu.hg = hg0;
    cu.b = b0;
    cu.Lb = len_of(b0);
    cu.n = (cu.Lb + C::BN - 1) / C::BN;
    // The range starts in job jb at unit pos; a job's first SEG units are
    // its segment weight, so a start inside them means the job's first step
    // (and the rest of those units come out of the range).
    const int off = (int)off0;
    const int per_job = cu.n + C::SEG;
    cu.jb = off / per_job;
    const int pos = off - cu.jb * per_job;
    cu.step = pos < C::SEG ? 0 : pos - C::SEG;
    cu.phase = 0;
    cu.left = (int)(hi - lo) - (pos < C::SEG ? C::SEG - pos : 0);  // <= 0: no key step here
    set_job(cu);
  };
  auto advance = [&](Cursor& cu) {
    if (cu.phase < cu.nq) {
      ++cu.phase;
      return;
    }
    --cu.left;
    ++cu.step;
    if (cu.left == 0 || cu.step < cu.n) return;
    // the next job's segment weight comes first; a range that ends inside
    // it has no key step of that job
    if (cu.left <= C::SEG) {
      cu.left = 0;
      return;
    }
    cu.left -= C::SEG;
    cu.step = 0;
    cu.phase = 0;
    if (++cu.jb == a.Hkv) {
      cu.jb = 0;
      do {
        if (++cu.b == a.B) {  // on to the next head group's list
          cu.b = 0;
          ++cu.hg;
        }
        cu.Lb = len_of(cu.b);
        cu.n = (cu.Lb + C::BN - 1) / C::BN;
      } while (cu.n == 0);
    }
    set_job(cu);
  };

  // ---- producer waves: copy u is copy cpy = p + NWP * u of the item: tile
  // cpy / GROUPS (0: first tile of the item, 1: second), 1 KB group
  // cpy % GROUPS; lane l of a group copies row RG * group + l % RG, 16-byte
  // chunk l / RG.
  const int pw = producer ? wave - C::NWC : 0;

  int pg_b = -1, pg_blk = -1, pg_page = 0;  // last page lookup (producers)
  int cb_b = -1, cb_row = 0;                // last batch-row lookup (producers)
  // Byte offset of copy u of this lane from its matrix's first row of a full
  // K/V item (set by the producer waves before their loop, so that a full
  // item costs one 64-bit add per copy).
  int64_t poff[C::PER];
  auto issue = [&](const Cursor& pc, int slot) {
    // (Lane constants are recomputed here so that they do not occupy
    // registers in the consumer waves.)
    const int lrow = lane % L::RG, cp_chunk = lane / L::RG;
    char* item = ring + slot * C::SB;
    if (pc.phase < pc.nq) {  // rows [64 phase, 64 phase + 64) of the job
      const char* qb = static_cast<const char*>(a.q) + ((int64_t)pc.b * a.q_sb + (int64_t)pc.g_kv * G * a.q_sh) * 2;
#pragma unroll
      for (int u = 0; u < C::PER; ++u) {
        const int cpy = pw + C::NWP * u, mat = cpy / C::GROUPS, grp = cpy % C::GROUPS;
        int r = 64 * pc.phase + 32 * mat + grp * L::RG + lrow;
        r = pc.hg * C::ROWS + (r < pc.rows ? r : pc.rows - 1);  // rows past the job's last repeat it (unused)
        const int t = kMulti || a.Sq > 1 ? r / G : 0;
        const int64_t roff = (int64_t)t * a.q_ss + (int64_t)(r - t * G) * a.q_sh;
        dma16(qb + (roff + cp_chunk * 8) * 2, lds_addr(item + mat * C::TB + grp * L::GS));
      }
    } else {
      const int row0 = pc.step * C::BN;
      int64_t koff, voff;  // element offsets of the item's first row
      if (a.block_table != nullptr) {  // an item never straddles pages (page_size % 32 == 0)
        const int blk = row0 / a.page_size;
        if (pc.b != pg_b || blk != pg_blk) {
          pg_b = pc.b;
          pg_blk = blk;
          pg_page = clamp_len(sload_i32(a.block_table + (int64_t)pc.b * a.max_blocks + blk), a.num_pages - 1);
        }
        const int prow = row0 - blk * a.page_size;
        koff = (int64_t)pg_page * a.k_pg + (int64_t)prow * a.k_ss;
        voff = (int64_t)pg_page * a.v_pg + (int64_t)prow * a.v_ss;
      } else {
        if (pc.b != cb_b) {
          cb_b = pc.b;
          cb_row = a.batch_idx != nullptr ? clamp_len(sload_i32(a.batch_idx + pc.b), a.cache_batch - 1) : pc.b;
        }
        koff = (int64_t)cb_row * a.k_sb + (int64_t)row0 * a.k_ss;
        voff = (int64_t)cb_row * a.v_sb + (int64_t)row0 * a.v_ss;
      }
      const char* kb = static_cast<const char*>(a.k) + (koff + (int64_t)pc.g_kv * a.k_sh) * 2;
      const char* vb = static_cast<const char*>(a.v) + (voff + (int64_t)pc.g_kv * a.v_sh) * 2;
      if (row0 + C::BN <= pc.Lb) {
#pragma unroll
        for (int u = 0; u < C::PER; ++u) {
          const int cpy = pw + C::NWP * u, mat = cpy / C::GROUPS, grp = cpy % C::GROUPS;
          dma16((mat ? vb : kb) + poff[u], lds_addr(item + mat * C::TB + grp * L::GS));
        }
      } else {  // the job's last step: rows past the cache length repeat the last one
#pragma unroll
        for (int u = 0; u < C::PER; ++u) {
          const int cpy = pw + C::NWP * u, mat = cpy / C::GROUPS, grp = cpy % C::GROUPS;
          int r = grp * L::RG + lrow;
          r = row0 + r < pc.Lb ? r : pc.Lb - 1 - row0;
          const int64_t ld = mat ? a.v_ss : a.k_ss;
          dma16((mat ? vb : kb) + ((int64_t)r * ld + cp_chunk * 8) * 2, lds_addr(item + mat * C::TB + grp * L::GS));
        }
      }
    }
  };

  // ---- consumer state: this wave's 32 heads over its parity's steps ----
  // Scores are raw dot products; the scale is applied inside exp2 (the query
  // is negated for a negative scale, so the applied scale is positive).
  const float scl = fabsf(a.scale) * kLog2e;
  const uint32_t qsign = a.scale < 0.0f ? 0x80008000u : 0u;
  const float cap_k2 = kSoftcap ? 2.0f * kLog2e * fabsf(a.scale) / a.softcap : 0.0f;
  const float cap_log2 = a.softcap * kLog2e;
  const int beta = lane >> 4, s16 = lane & 15;
  const int tr_row = 4 * (beta >> 1) + (s16 >> 2);
  const int tr_chunk = 2 * (beta & 1) + ((s16 & 3) >> 1);
  const int tr_half = 8 * (s16 & 1);

  typename T::vec8 qf[C::DSTEPS];
  float m_run = kNegInf, l_run = 0.0f;  // m_run in exp2 units
  // kMulti (causal, several queries): keys this lane's row may see, and the
  // smallest such count in the wave (steps below it need no mask).
  int lim_row = 0, lim_wave = 0;
  f32x16 oacc[C::DBLK];
#pragma unroll
  for (int ds = 0; ds < C::DSTEPS; ++ds) qf[ds] = __builtin_bit_cast(typename T::vec8, make_uint4(0, 0, 0, 0));
#pragma unroll
  for (int db = 0; db < C::DBLK; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.0f;

  // One group of NI (1 or 2) consecutive K/V steps of the job for this
  // wave's 32 heads; the steps' score tiles are independent matrix-core
  // chains and share one max / rescale.
  auto kv_group = [&](auto ni_tag, int i0, int step, int Lb) {
    constexpr int NI = decltype(ni_tag)::value;
    f32x16 sacc[NI];
#pragma unroll
    for (int t = 0; t < NI; ++t) {
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[t][r] = 0.0f;
    }
#pragma unroll
    for (int t = 0; t < NI; ++t) {
      const char* kt = ring + ((i0 + t) % C::NS) * C::SB;
      typename T::vec8 ka[C::DSTEPS];
#pragma unroll
      for (int ds = 0; ds < C::DSTEPS; ++ds)
        ka[ds] = *reinterpret_cast<const typename T::vec8*>(kt + L::off(c, 2 * ds + g));
#pragma unroll
      for (int ds = 0; ds < C::DSTEPS; ++ds) sacc[t] = mfma32(ka[ds], qf[ds], sacc[t]);
    }
    // sacc[t][r]: key 8*(r/4) + 4*g + r%4 of step step + t, head c.  Keys
    // past the cache length hold copies of the last key, so they never
    // raise the max.
    if (kSoftcap) {
#pragma unroll
      for (int t = 0; t < NI; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float e = fast_exp2(sacc[t][r] * cap_k2);
          sacc[t][r] = cap_log2 * (1.0f - 2.0f * fast_rcp(e + 1.0f));
        }
    }
    // Causal rows: keys at or past the row's own count are real keys of later
    // positions, so they are removed before the max.
    if constexpr (kMulti) {
#pragma unroll
      for (int t = 0; t < NI; ++t) {
        if ((step + t + 1) * C::BN > lim_wave) {
          const int key0 = (step + t) * C::BN + 4 * g;
#pragma unroll
          for (int r = 0; r < 16; ++r)
            sacc[t][r] = key0 + 8 * (r >> 2) + (r & 3) < lim_row ? sacc[t][r] : kNegInf;
        }
      }
    }
    // (Plain fmaxf here: the matrix-core results must be read by compiled
    // instructions, which get the MFMA -> VALU wait states.)
    float mt[NI];
#pragma unroll
    for (int t = 0; t < NI; ++t) {
      float m4[4];
#pragma unroll
      for (int q = 0; q < 4; ++q)
        m4[q] = fmaxf(fmaxf(sacc[t][4 * q], sacc[t][4 * q + 1]), fmaxf(sacc[t][4 * q + 2], sacc[t][4 * q + 3]));
      mt[t] = fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3]));
    }
    float mx = NI == 2 ? fmaxf(mt[0], mt[NI - 1]) : mt[0];
    mx = pair_max32(mx);
    if (!kSoftcap) mx *= scl;
    if (__any(mx > m_run + 8.0f)) {
      const float m_new = max_nc(m_run, mx);
      const float alpha = (m_run == kNegInf) ? 0.0f : fast_exp2(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < C::DBLK; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
      m_run = m_new;
    }
    typename T::vec8 pf[NI][2];
    float ls[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    // (A row with no visible key yet keeps m_run = -inf; all its scores are
    // -inf then, and a zero reference keeps exp2 at 0 instead of NaN.)
    const float m_use = kMulti && m_run == kNegInf ? 0.0f : m_run;
#pragma unroll
    for (int t = 0; t < NI; ++t) {
      float p[16];
#pragma unroll
      for (int r = 0; r < 16; ++r)
        p[r] = kSoftcap ? fast_exp2(sacc[t][r] - m_use) : fast_exp2(__builtin_fmaf(sacc[t][r], scl, -m_use));
      if (!kMulti && (step + t + 1) * C::BN > Lb) {
        const int key0 = (step + t) * C::BN + 4 * g;
#pragma unroll
        for (int r = 0; r < 16; ++r) p[r] = key0 + 8 * (r >> 2) + (r & 3) < Lb ? p[r] : 0.0f;
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        ls[r & 3] += p[r];
        pf[t][r >> 3][r & 7] = static_cast<typename T::elem>(p[r]);
      }
    }
    l_run += (ls[0] + ls[1]) + (ls[2] + ls[3]);
    // O^T += V^T P^T
#pragma unroll
    for (int t = 0; t < NI; ++t) {
      const char* vt = ring + ((i0 + t) % C::NS) * C::SB + C::TB;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        typename T::vec8 va[C::DBLK];
#pragma unroll
        for (int db = 0; db < C::DBLK; ++db) {
          const char* p0 = vt + L::off(16 * ks + tr_row, 4 * db + tr_chunk) + tr_half;
          const char* p1 = vt + L::off(16 * ks + 8 + tr_row, 4 * db + tr_chunk) + tr_half;
          va[db] = cat_frag<typename T::vec8>(lds_read_tr16(reinterpret_cast<const bf16_t*>(p0)),
                            lds_read_tr16(reinterpret_cast<const bf16_t*>(p1)));
        }
#pragma unroll
        for (int db = 0; db < C::DBLK; ++db) oacc[db] = mfma32(va[db], pf[t][ks], oacc[db]);
      }
    }
  };

  // End of this wave's segment of job (cc.b, cc.jb), number `seg` of this
  // workgroup: the parity-1 wave of each head block hands its softmax state
  // to the parity-0 wave through its LDS slot (sequence flags, no barrier),
  // and the parity-0 wave writes the merged partial result (normalised O,
  // rounded to the input type: it is a convex combination of value rows, so
  // it fits their range, and the combine reads half the bytes of fp32;
  // natural-log LSE in fp32) to slot w + j.  Waves whose head block has no
  // query heads in this job still step the flags.
  auto finish_segment = [&](const Cursor& cc, bool job_end, int seg) {
    const bool active = rb * 32 < cc.rows;
    const int64_t j = job_index(cc);
    const int64_t slot = w_id + j;
    if constexpr (kWide) {  // the wave holds its rows' whole state: write it
      const bool poison = broken || __hip_atomic_load(&ring_broken, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      if (active) {
        const float l_tot = pair_sum32(l_run);
        const int row = rb * 32 + c;
        const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
        uint16_t* op = a.part_o + (slot * C::ROWS + row) * D;
#pragma unroll
        for (int db = 0; db < C::DBLK; ++db)
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            const uint2 w2 = make_uint2(
                f32_to_elem<T>(oacc[db][4 * rr] * inv) | (uint32_t)f32_to_elem<T>(oacc[db][4 * rr + 1] * inv) << 16,
                f32_to_elem<T>(oacc[db][4 * rr + 2] * inv) | (uint32_t)f32_to_elem<T>(oacc[db][4 * rr + 3] * inv) << 16);
            if (row < cc.rows) *reinterpret_cast<uint2*>(op + 32 * db + 8 * rr + 4 * g) = w2;
          }
        if (g == 0 && row < cc.rows)
          a.part_lse[slot * C::ROWS + row] =
              poison ? __builtin_nanf("") : (l_tot > 0.0f ? (m_run + fast_log2(l_tot)) * kLn2 : kNegInf);
      }
      if (lane == 0 && wave == 0 && job_end) a.job_seg[2 * j + 1] = w_id;  // this workgroup ends the job
      return;
    }
    char* ms = mrg + hb * C::MSLOT;
    uint2* ms_o = reinterpret_cast<uint2*>(ms);                       // [DBLK * 4][64] pairs of pairs
    float* ms_ml = reinterpret_cast<float*>(ms + 64 * 16 * C::DBLK * 2);  // m [64], l [64]
    if (par == 1) {
      note(spin_until_ge(&mrg_read[hb], seg, a.spin_limit));  // the previous segment's state has been taken
      if (active) {
        // bf16 is enough here: the merged partial is itself stored rounded
        // to the input type, and the state's relative rounding (2^-9) adds
        // to that once
#pragma unroll
        for (int db = 0; db < C::DBLK; ++db)
#pragma unroll
          for (int rr = 0; rr < 4; ++rr)
            ms_o[(db * 4 + rr) * 64 + lane] =
                make_uint2(f32_to_elem<Bf16T>(oacc[db][4 * rr]) | (uint32_t)f32_to_elem<Bf16T>(oacc[db][4 * rr + 1]) << 16,
                           f32_to_elem<Bf16T>(oacc[db][4 * rr + 2]) | (uint32_t)f32_to_elem<Bf16T>(oacc[db][4 * rr + 3]) << 16);
        ms_ml[lane] = m_run;
        ms_ml[64 + lane] = l_run;
      }
      if (lane == 0) publish(&mrg_written[hb], seg + 1);
      return;
    }
    note(spin_until_ge(&mrg_written[hb], seg + 1, a.spin_limit));
    const bool poison = broken || __hip_atomic_load(&ring_broken, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    if (active) {
      const float mo = ms_ml[lane];
      const float lo1 = ms_ml[64 + lane];
      const float M = fmaxf(m_run, mo);
      const float a0 = m_run == kNegInf ? 0.0f : fast_exp2(m_run - M);
      const float a1 = mo == kNegInf ? 0.0f : fast_exp2(mo - M);
      const float l_tot = pair_sum32(l_run * a0 + lo1 * a1);
      const int row = hb * 32 + c;
      const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
      const float s0 = a0 * inv, s1 = a1 * inv;
      uint16_t* op = a.part_o + (slot * C::ROWS + row) * D;
#pragma unroll
      for (int db = 0; db < C::DBLK; ++db)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const uint2 xp = ms_o[(db * 4 + rr) * 64 + lane];
          const float4 x = make_float4(Bf16T::to_f32(xp.x & 0xffffu), Bf16T::to_f32(xp.x >> 16),
                                       Bf16T::to_f32(xp.y & 0xffffu), Bf16T::to_f32(xp.y >> 16));
          const float o0 = oacc[db][4 * rr] * s0 + x.x * s1, o1 = oacc[db][4 * rr + 1] * s0 + x.y * s1;
          const float o2 = oacc[db][4 * rr + 2] * s0 + x.z * s1, o3 = oacc[db][4 * rr + 3] * s0 + x.w * s1;
          const uint2 w2 = make_uint2(f32_to_elem<T>(o0) | (uint32_t)f32_to_elem<T>(o1) << 16,
                                      f32_to_elem<T>(o2) | (uint32_t)f32_to_elem<T>(o3) << 16);
          if (row < cc.rows) *reinterpret_cast<uint2*>(op + 32 * db + 8 * rr + 4 * g) = w2;
        }
      if (g == 0 && row < cc.rows)
        a.part_lse[slot * C::ROWS + row] =
            poison ? __builtin_nanf("") : (l_tot > 0.0f ? (M + fast_log2(l_tot)) * kLn2 : kNegInf);
    }
    if (lane == 0) publish(&mrg_read[hb], seg + 1);  // the slot may be refilled
    if (lane == 0 && hb == 0 && job_end) a.job_seg[2 * j + 1] = w_id;  // this workgroup ends the job
  };

  // ---- the ring: item i lives in slot i % NS.  No barriers: the producer
  // waves publish how many items have landed, each consumer wave publishes
  // how many items it is done with, and a slot is refilled once every
  // consumer wave is past its previous item. ----
  using One = std::integral_constant<int, 1>;
  Cursor cc;
  start(cc);
  if (producer) {
    // The producer shares its SIMD with consumer waves; a higher issue
    // priority keeps its copies flowing while they compute.
    __builtin_amdgcn_s_setprio(3);
    {
      const int lrow = lane % L::RG, cp_chunk = lane / L::RG;
#pragma unroll
      for (int u = 0; u < C::PER; ++u) {
        const int cpy = pw + C::NWP * u, mat = cpy / C::GROUPS, grp = cpy % C::GROUPS;
        poff[u] = ((int64_t)(grp * L::RG + lrow) * (mat ? a.v_ss : a.k_ss) + cp_chunk * 8) * 2;
      }
    }
    Cursor pc = cc;
    int issued = 0, published = 0;
    auto publish_all = [&]() {
      if (published < issued) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        published = issued;
        if (lane == 0) publish(&landed[pw], published);
      }
    };
    int seen = 0;  // a lower bound of every consumer's count (they only grow)
    while (pc.left > 0) {
      const int need = issued - C::NS + 1;  // the slot's previous item must be done
      // While the slot is busy, publish the oldest unpublished item one at a
      // time (the consumers may be waiting for it), else sleep.
      for (int n = 0; seen < need; ++n) {
        if ((seen = consumed_min()) >= need) break;
        if (n >= a.spin_limit) {  // the slot may still be read: stale data for a consumer
          note(false);
          break;
        }
        if (published < issued) {
          wait_items<C::PER, C::NS - 1>(issued - published - 1);
          ++published;
          if (lane == 0) publish(&landed[pw], published);
        } else {
          __builtin_amdgcn_s_sleep(1);
        }
      }
      issue(pc, issued % C::NS);
      advance(pc);
      ++issued;
      if (issued - published > C::DEPTH) {  // keep DEPTH items in flight, publish the rest
        vm_wait_imm<C::PER, C::DEPTH>();
        published = issued - C::DEPTH;
        if (lane == 0) publish(&landed[pw], published);
      }
    }
    publish_all();
    if (broken) status_or(a.status, kDecodeStatusWait);
    return;
  }
  int seg = 0, have = 0;  // have: a lower bound of the landed count
  auto wait_landed = [&](int v) {
    if (have < v) note(spin_until(([&] { return (have = landed_min()) >= v; }), a.spin_limit));
  };
  for (int i = 0; cc.left > 0;) {
    // The next group: a job's query items (read by every consumer wave), or
    // one K/V step per parity.
    const bool qgrp = cc.phase < cc.nq;
    const int gsz = qgrp ? cc.nq : ((!kWide && cc.left >= 2 && cc.step + 1 < cc.n) ? 2 : 1);
    if (qgrp) {
      wait_landed(i + gsz);
      if (lane == 0 && wave == 0 && cc.step == 0)  // this workgroup starts the job
        a.job_seg[2 * job_index(cc)] = w_id;
      m_run = kNegInf;
      l_run = 0.0f;
#pragma unroll
      for (int db = 0; db < C::DBLK; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] = 0.0f;
      if constexpr (kMulti) {
        const int r0 = cc.hg * C::ROWS + rb * 32;
        lim_row = cc.Lb - a.Sq + 1 + min(r0 + c, R - 1) / G;
        lim_wave = cc.Lb - a.Sq + 1 + r0 / G;
      }
      if (rb * 32 < cc.rows) {
        const char* qt = ring + ((i + (rb >> 1)) % C::NS) * C::SB + (rb & 1) * C::TB;
#pragma unroll
        for (int ds = 0; ds < C::DSTEPS; ++ds) {
          uint4 raw = *reinterpret_cast<const uint4*>(qt + L::off(c, 2 * ds + g));
          raw.x ^= qsign;
          raw.y ^= qsign;
          raw.z ^= qsign;
          raw.w ^= qsign;
          qf[ds] = __builtin_bit_cast(typename T::vec8, raw);
        }
      }
      if (lane == 0) publish(&consumed[wave], i + gsz);
    } else if constexpr (kWide) {  // one K/V step, read by every consumer wave
      if (rb * 32 < cc.rows) {
        wait_landed(i + 1);
        kv_group(One{}, i, cc.step, cc.Lb);
      }
      if (lane == 0) publish(&consumed[wave], i + 1);
      const bool job_end = cc.step + 1 == cc.n;
      if (job_end || cc.left == 1) finish_segment(cc, job_end, seg++);
    } else {
      const bool mine = par < gsz && hb * 32 < cc.rows;
      // A parity-1 wave never reads item i of the group, so it is done with
      // every item before i + 1 already; saying so at once lets the slot of
      // item i be refilled as soon as the parity-0 waves are past it.
      if (par == 1 && lane == 0) publish(&consumed[wave], i + 1);
      if (mine) {
        wait_landed(i + par + 1);
        kv_group(One{}, i + par, cc.step + par, cc.Lb);
      }
      if (lane == 0) publish(&consumed[wave], i + gsz);
      const bool job_end = cc.step + gsz == cc.n;
      if (job_end || cc.left == gsz) finish_segment(cc, job_end, seg++);
    }
    for (int t = 0; t < gsz; ++t) advance(cc);
    i += gsz;
  }
  if (broken) status_or(a.status, kDecodeStatusWait);
}

// Merge the partial results of one job: one thread per (head row, 4 columns).
// The job's partials are in slots w + j for w from its first to its last
// workgroup, as recorded by the split kernel.
template <typename T, int D, int ROWS>
__global__ __launch_bounds__(256) void decode_combine_kernel(DecodeArgs a) {
  constexpr int TPH = D / 4;      // threads per head
  constexpr int HPB = 256 / TPH;  // heads per workgroup
  constexpr int U = 8;            // partials loaded per round
  const int j = blockIdx.x;
  // job j of the split kernel's list: head group first, then sequence, kv head
  const int hg = j / (a.B * a.Hkv);
  const int b = (j / a.Hkv) % a.B, g_kv = j % a.Hkv;
  const int G = a.Hq / a.Hkv;
  const int rows = min(ROWS, a.Sq * G - hg * ROWS);
  const int r = blockIdx.y * HPB + threadIdx.x / TPH;
  if (r >= rows) return;
  const int d4 = threadIdx.x % TPH;
  const int jr = hg * ROWS + r;  // row = query t * G + head
  const int t = jr / G;
  const int h = g_kv * G + (jr - t * G);
  // The job's first and last workgroup are loaded beside its length, not
  // after it: two dependent round trips become one.  (For an empty sequence
  // they were never written and are not used.)
  const int w0 = a.job_seg[2 * j], w1 = a.job_seg[2 * j + 1];
  const int Lb = seq_len(a, b);
  asm volatile("" :: "v"(w0), "v"(w1), "v"(Lb));
  if (blockIdx.y == 0 && threadIdx.x == 0) {
    const int raw = a.seqlens[b];
    if (raw < 0 || raw > a.Smax - a.len_add) status_or(a.status, kDecodeStatusLength);
  }
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  float m = kNegInf, tot = 0.0f;
  bool poisoned = false;  // a partial was written as NaN (an expired wait)
  if (Lb > 0) {
    const float* pl = a.part_lse + ((int64_t)w0 + j) * ROWS + r;
    const uint16_t* po = a.part_o + (((int64_t)w0 + j) * ROWS + r) * D + 4 * d4;
    const int ns = w1 - w0 + 1;
    for (int s0 = 0; s0 < ns; s0 += U) {
      float ls[U];
      float4 ov[U];
#pragma unroll
      for (int e = 0; e < U; ++e) {
        const bool ok = s0 + e < ns;
        ls[e] = ok ? pl[(int64_t)(s0 + e) * ROWS] : kNegInf;
        const uint2 w2 = ok ? *reinterpret_cast<const uint2*>(po + (int64_t)(s0 + e) * ROWS * D) : make_uint2(0, 0);
        ov[e] = make_float4(T::to_f32(w2.x & 0xffffu), T::to_f32(w2.x >> 16), T::to_f32(w2.y & 0xffffu),
                            T::to_f32(w2.y >> 16));
      }
      float mr = m;
#pragma unroll
      for (int e = 0; e < U; ++e) {
        poisoned |= ls[e] != ls[e];
        mr = fmaxf(mr, ls[e]);
      }
      if (mr == kNegInf) continue;
      const float sc = m == kNegInf ? 0.0f : fast_exp2((m - mr) * kLog2e);
      tot *= sc;
      acc.x *= sc;
      acc.y *= sc;
      acc.z *= sc;
      acc.w *= sc;
#pragma unroll
      for (int e = 0; e < U; ++e) {
        const float wgt = ls[e] == kNegInf ? 0.0f : fast_exp2((ls[e] - mr) * kLog2e);
        tot += wgt;
        acc.x = __builtin_fmaf(wgt, ov[e].x, acc.x);
        acc.y = __builtin_fmaf(wgt, ov[e].y, acc.y);
        acc.z = __builtin_fmaf(wgt, ov[e].z, acc.z);
        acc.w = __builtin_fmaf(wgt, ov[e].w, acc.w);
      }
      m = mr;
    }
  }
  float inv = tot > 0.0f ? 1.0f / tot : 0.0f;
  if (poisoned) {
    inv = __builtin_nanf("");
    m = __builtin_nanf("");
  }
  bf16_t* op = static_cast<bf16_t*>(a.o) + b * a.o_sb + (int64_t)t * a.o_ss + (int64_t)h * a.o_sh + 4 * d4;
  const uint32_t lo2 = (uint32_t)(f32_to_elem<T>(acc.x * inv)) |
                       ((uint32_t)(f32_to_elem<T>(acc.y * inv)) << 16);
  const uint32_t hi2 = (uint32_t)(f32_to_elem<T>(acc.z * inv)) |
                       ((uint32_t)(f32_to_elem<T>(acc.w * inv)) << 16);
  *reinterpret_cast<uint2*>(op) = make_uint2(lo2, hi2);
  if (d4 == 0)
    a.lse[((int64_t)b * a.Hq + h) * a.Sq + t] = (tot > 0.0f || poisoned) ? m + fast_log2(tot) * kLn2 : kNegInf;
}

// In-place append: rows [L_b, L_b + len_add) of sequence b's cache (paged or
// contiguous) receive k_new / v_new.  One thread per 16-byte chunk.
template <int D>
__global__ __launch_bounds__(256) void kvcache_append_kernel(DecodeArgs a) {
  constexpr int CH = D / 8;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t total = (int64_t)a.B * a.len_add * a.Hkv * CH;
  if (idx >= total) return;
  const int ch = (int)(idx % CH);
  int64_t rest = idx / CH;
  const int g = (int)(rest % a.Hkv);
  rest /= a.Hkv;
  const int t = (int)(rest % a.len_add);
  const int b = (int)(rest / a.len_add);
  const int r = clamp_len(a.seqlens[b], a.Smax - a.len_add) + t;
  int64_t koff, voff;
  if (a.block_table != nullptr) {
    const int blk = r / a.page_size;
    const int page = clamp_len(a.block_table[(int64_t)b * a.max_blocks + blk], a.num_pages - 1);
    koff = (int64_t)page * a.k_pg + (int64_t)(r - blk * a.page_size) * a.k_ss;
    voff = (int64_t)page * a.v_pg + (int64_t)(r - blk * a.page_size) * a.v_ss;
  } else {
    const int row = a.batch_idx != nullptr ? clamp_len(a.batch_idx[b], a.cache_batch - 1) : b;
    koff = (int64_t)row * a.k_sb + (int64_t)r * a.k_ss;
    voff = (int64_t)row * a.v_sb + (int64_t)r * a.v_ss;
  }
  bf16_t* kd = static_cast<bf16_t*>(const_cast<void*>(a.k)) + koff + (int64_t)g * a.k_sh + 8 * ch;
  bf16_t* vd = static_cast<bf16_t*>(const_cast<void*>(a.v)) + voff + (int64_t)g * a.v_sh + 8 * ch;
  const bf16_t* ks = static_cast<const bf16_t*>(a.k_new) + b * a.kn_sb + (int64_t)t * a.kn_ss + g * a.kn_sh + 8 * ch;
  const bf16_t* vs = static_cast<const bf16_t*>(a.v_new) + b * a.vn_sb + (int64_t)t * a.vn_ss + g * a.vn_sh + 8 * ch;
  *reinterpret_cast<uint4*>(kd) = *reinterpret_cast<const uint4*>(ks);
  *reinterpret_cast<uint4*>(vd) = *reinterpret_cast<const uint4*>(vs);
}

template <typename T, int D, bool W>
hipError_t launch_split(const DecodeArgs& a, hipStream_t s) {
  const dim3 block(DecCfg<D, W>::NT);
  const bool multi = a.causal && a.Sq > 1;
  if (a.softcap > 0.0f) {
    if (multi) hipLaunchKernelGGL((decode_split_kernel<T, D, true, true, W>), dim3(a.parts), block, 0, s, a);
    else hipLaunchKernelGGL((decode_split_kernel<T, D, true, false, W>), dim3(a.parts), block, 0, s, a);
  } else {
    if (multi) hipLaunchKernelGGL((decode_split_kernel<T, D, false, true, W>), dim3(a.parts), block, 0, s, a);
    else hipLaunchKernelGGL((decode_split_kernel<T, D, false, false, W>), dim3(a.parts), block, 0, s, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  constexpr int ROWS = DecCfg<D, W>::ROWS;
  constexpr int HPB = 256 / (D / 4);
  const int jobs = a.B * a.Hkv * a.nhg;
  hipLaunchKernelGGL((decode_combine_kernel<T, D, ROWS>), dim3(jobs, (ROWS + HPB - 1) / HPB), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_d(const DecodeArgs& a, hipStream_t s) {
  if (a.len_add > 0) {
    const int64_t total = (int64_t)a.B * a.len_add * a.Hkv * (D / 8);
    hipLaunchKernelGGL(kvcache_append_kernel<D>, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.rows_job == kDecodeRowsWide) return launch_split<T, D, true>(a, s);
  if (a.rows_job == kDecodeRows) return launch_split<T, D, false>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace

// A kv head with more than 128 rows takes 256-row jobs: its keys are then
// streamed once per 256 rows instead of once per 128.
int decode_job_rows(int Hq, int Hkv, int Sq) {
  return (int64_t)Sq * (Hq / Hkv) > kDecodeRows ? kDecodeRowsWide : kDecodeRows;
}

int decode_head_groups(int Hq, int Hkv, int Sq) {
  const int rows = decode_job_rows(Hq, Hkv, Sq);
  return (int)(((int64_t)Sq * (Hq / Hkv) + rows - 1) / rows);
}

int device_cu_count() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cus[dev] = n;
  }
  return cus[dev];
}

int decode_parts(int num_splits) { return num_splits > 0 ? num_splits : device_cu_count(); }

DecodeWorkspace decode_workspace(int B, int Hq, int Hkv, int Sq, int D, int parts) {
  DecodeWorkspace w;
  const size_t jobs = (size_t)B * Hkv * decode_head_groups(Hq, Hkv, Sq);
  const size_t slots = (size_t)parts + jobs;
  const size_t rows = decode_job_rows(Hq, Hkv, Sq);
  w.status_off = 0;  // the status word; 256 bytes keep the rest aligned
  w.o_off = 256;
  w.lse_off = w.o_off + (slots * rows * D * sizeof(uint16_t) + 255) / 256 * 256;
  w.seg_off = w.lse_off + (slots * rows * sizeof(float) + 255) / 256 * 256;
  w.bytes = w.seg_off + (jobs * 2 * sizeof(int32_t) + 255) / 256 * 256;
  return w;
}

hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t s) {
  if (a.B == 0) return hipSuccess;
  if (a.f16) return a.D == 64 ? launch_d<F16T, 64>(a, s) : launch_d<F16T, 128>(a, s);
  if (a.D == 64) return launch_d<Bf16T, 64>(a, s);
  return launch_d<Bf16T, 128>(a, s);
}

}  // namespace attn
