// Internal launch interfaces between the C-ABI layer (api.hip) and the
// kernel translation units.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

// Mask predicate evaluated on partial tiles (causal / window / document).
struct MaskArgs {
  int causal, wl, wr;        // wl/wr < 0: unbounded side
  const int32_t* doc_q;      // [B, Sq] or nullptr
  const int32_t* doc_k;      // [B, Sk] or nullptr
};

// Block-sparse tile lists (nullptr kv_num_* = dense iteration).
struct TileLists {
  const int32_t* kv_num_full;
  const int32_t* kv_idx_full;
  const int32_t* kv_num_partial;
  const int32_t* kv_idx_partial;
  int nQ, nK;                // mask tile grid per batch row
  int block_m;               // mask tile rows (a multiple of the kernel's)
  int sub;                   // kernel key tiles per mask key tile
};

struct FwdArgs {
  const void* q; const void* k; const void* v; void* o;
  bool f16;                  // 16-bit inputs are fp16 (else bf16); the fp32 kernel ignores it
  float* lse;
  uint8_t* trace;
  int64_t q_sb, q_ss, q_sh;
  int64_t k_sb, k_ss, k_sh;
  int64_t v_sb, v_ss, v_sh;
  int64_t o_sb, o_ss, o_sh;
  int B, Sq, Sk, Hq, Hkv, D;
  int nQt, nKt;              // trace grid (kernel tiles, or mask tiles)
  float scale;               // softmax scale (any sign)
  const float* alibi;        // nullptr = off
  int64_t alibi_sb;
  float softcap;             // 0 = off
  MaskArgs mask;
  TileLists tiles;
  int spin_limit;            // bound of the in-kernel waits (sleeps); see attn_debug_set_spin_limit
};

// Bound on every in-kernel spin wait, in s_sleep rounds: the default (about
// 2^22) only matters if a hand-over protocol were broken; a wait that
// expires poisons its outputs (NaN) and, in the decode path, sets a status
// bit.  Tests lower it through attn_debug_set_spin_limit.
constexpr int kDefaultSpinLimit = 1 << 22;
int spin_limit();

// Whether the dK/dV kernel loops the grouped-query heads of a kv head inside
// one workgroup (kv_grid: its workgroups then) rather than writing per-head
// partials; attn_set_bwd_gqa_schedule can force either.
bool bwd_group_loop_choice(long kv_grid, int cus);

// bf16 MFMA forward.  Tiles of 128 or 256 query rows x 64 keys (block-sparse
// masks use 128-row tiles).
constexpr int kFwdBM = 128;
constexpr int kFwdBN = 64;
int fwd_bf16_rows_per_block(int B, int Sq, int Hq, int causal, bool sparse);
hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t s);

// fp32 vector-ALU forward.  Tile 64 x 64.
constexpr int kFwdF32BM = 64;
constexpr int kFwdF32BN = 64;
hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t s);

// Block-sparse tile lists for the backward: per query block the key blocks
// (dQ), per key block the query blocks (dK/dV); mask tiles of 128 query rows
// by block_n keys, block_n a multiple of 128.
struct BwdTiles {
  const int32_t* kv_num_full; const int32_t* kv_idx_full;
  const int32_t* kv_num_partial; const int32_t* kv_idx_partial;
  const int32_t* q_num_full; const int32_t* q_idx_full;
  const int32_t* q_num_partial; const int32_t* q_idx_partial;
  int nQ, nK, block_n;
};

struct BwdArgs {
  const void* q; const void* k; const void* v; const void* o; const void* dout;
  bool f16;                  // inputs and gradients are fp16 (else bf16)
  const float* lse;
  void* dq; void* dk; void* dv;
  int64_t q_sb, q_ss, q_sh;
  int64_t k_sb, k_ss, k_sh;
  int64_t v_sb, v_ss, v_sh;
  int64_t o_sb, o_ss, o_sh;
  int64_t do_sb, do_ss, do_sh;
  int64_t dq_sb, dq_ss, dq_sh;
  int64_t dk_sb, dk_ss, dk_sh;
  int64_t dv_sb, dv_ss, dv_sh;
  int B, Sq, Sk, Hq, Hkv, D;
  float scale;
  const float* alibi;
  int64_t alibi_sb;
  float softcap;
  MaskArgs mask;
  BwdTiles tiles;            // block-sparse lists (kv_num_full == nullptr: dense)
  float* delta;              // workspace [B, Hq, Sq]
  float* lse2;               // workspace [B, Hq, Sq]: lse * log2(e), +inf for empty rows
  float* part_dk;            // workspace [B, Sk, Hq, D] (grouped heads only)
  float* part_dv;
  float* dq_acc;             // workspace [B, Sq, Hq, D]: non-deterministic dQ (nullptr: dQ kernel)
};
size_t bwd_workspace_bytes(int B, int Hq, int Hkv, int Sq, int Sk, int D);
// stage_mask bit k runs stage k (0 Delta, 1 dK/dV, 2 group sum, 3 dQ).
constexpr int kBwdAllStages = 0xF;
hipError_t launch_bwd_bf16(const BwdArgs& a, int stage_mask, hipStream_t s);

struct DecodeArgs {
  const void* q; const void* k; const void* v; void* o;
  bool f16;                  // q, caches, new rows and o are fp16 (else bf16)
  float* lse;
  const int32_t* seqlens;
  int64_t q_sb, q_ss, q_sh;
  int64_t k_sb, k_ss, k_sh;
  int64_t v_sb, v_ss, v_sh;
  int64_t o_sb, o_ss, o_sh;
  int B, Hq, Hkv, D, Smax;
  // Sq queries per sequence, the last Sq positions of it; a job's rows are
  // (query t, head) pairs, row = t * (Hq / Hkv) + head within the kv head.
  // causal: query t sees the first L - Sq + 1 + t keys (L keys in all).
  int Sq, causal;
  float scale;
  float softcap;
  int parts;                 // workgroups; the key work is cut into this many equal ranges
  int rows_job;              // rows per job: decode_job_rows()
  int nhg;                   // groups of up to rows_job rows per kv head
  uint16_t* part_o;          // workspace [parts + jobs][rows_job][D]: normalised partial O,
                             // rounded to the input type
  float* part_lse;           // workspace [parts + jobs][rows_job]
                             // (a job: sequence, kv head, up to rows_job rows)
  int32_t* job_seg;          // workspace [jobs][2]: first and last workgroup of each job
  // KV-cache addressing.  Contiguous: sequence b uses batch row batch_idx[b]
  // (b when null) of k/v.  Paged (block_table != null): row r of sequence b is
  // row r % page_size of page block_table[b * max_blocks + r / page_size],
  // k_pg / v_pg being the page strides.  Smax is the per-sequence capacity.
  const int32_t* batch_idx;
  int cache_batch;           // batch rows of a contiguous cache (batch_idx range)
  const int32_t* block_table;
  int max_blocks, page_size, num_pages;
  int64_t k_pg, v_pg;
  // In-place append of len_add new rows per sequence at [L_b, L_b + len_add).
  int len_add;
  const void* k_new; const void* v_new;
  int64_t kn_sb, kn_ss, kn_sh, vn_sb, vn_ss, vn_sh;
  uint32_t* status;          // sticky status word in the workspace (bits ORed in)
  int spin_limit;
};
// Bits of the decode status word.
constexpr uint32_t kDecodeStatusLength = 1;  // a cache length was outside [0, Smax - s_new]
constexpr uint32_t kDecodeStatusWait = 2;    // an in-kernel wait expired (rows poisoned with NaN)
constexpr int kDecodeRows = 128;      // rows (query, head) per decode job
constexpr int kDecodeRowsWide = 256;  // the same when a kv head has more than 128 rows
int decode_job_rows(int Hq, int Hkv, int Sq);
// Number of workgroups: num_splits when > 0, else the device's compute units.
int decode_parts(int num_splits);
int device_cu_count();  // compute units of the current device (cached per device)
int decode_head_groups(int Hq, int Hkv, int Sq);  // jobs per (sequence, kv head)
struct DecodeWorkspace {
  size_t status_off, o_off, lse_off, seg_off, bytes;
};
DecodeWorkspace decode_workspace(int B, int Hq, int Hkv, int Sq, int D, int parts);
hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t s);

struct BlockMaskArgs {
  int B, Sq, Sk, bm, bn, nQ, nK;
  MaskArgs mask;
  uint8_t* cls;
  int32_t* kv_num_partial; int32_t* kv_idx_partial;
  int32_t* kv_num_full; int32_t* kv_idx_full;
  int32_t* q_num_partial; int32_t* q_idx_partial;
  int32_t* q_num_full; int32_t* q_idx_full;
};
hipError_t launch_block_mask(const BlockMaskArgs& a, hipStream_t s);
int block_mask_max_block();  // largest block_m / block_n with a document mask

}  // namespace attn
