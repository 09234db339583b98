/*
 * attn.h - C ABI of the exact IO-aware attention library for AMD Instinct
 * MI355X (gfx950).
 *
 * Sources cited below (web pages):
 *   [TA]  "Accelerating AI: A Deep Dive into Flash Attention and Its Impacts"
 *         (Towards AI)
 *   [FA]  "FlashAttention: Fast and Memory-Efficient Exact Attention"
 *         (Dao-AILab/flash-attention repository overview)
 *   [HF]  "Improvements in attention_forward functions"
 *         (huggingface/transformers issue 36218)
 *   [GYM] "FlexAttention uses much more GPU memory than FlashAttention-2"
 *         (pytorch-labs/attention-gym issue 101)
 *   [FX4] "Lightning Talk: FlexAttention + FlashAttention-4: Fast and
 *         Flexible" (PyTorch Conference Europe 2026)
 *
 * What is computed.  For batch b, query head h, query row i and key j, with
 * g = h / (Hq / Hkv) the key/value head that h reads ([HF]: repeat_kv is a
 * repeat_interleave over heads, here done by indexing, never by copying) and
 * delta = Sk - Sq (last query aligned with the last key):
 *
 *   s   = scale * <q[b,i,h,:], k[b,j,g,:]>        scores, [TA] "Key-Value
 *                                                 Attention"; scale per [FA]
 *                                                 "Examples" (softmax_scale)
 *   t   = softcap > 0 ? softcap * tanh(s / softcap) : s
 *   u   = t - slope[b,h] * |i + delta - j|        if ALiBi slopes are given
 *   allowed(i,j) = causal:  j <= i + delta
 *                  window:  i + delta - left <= j <= i + delta + right
 *                           (a side of -1 is unbounded; [FA] "Examples")
 *                  block mask predicate (see attn_mask_desc) when given
 *   lse[b,h,i] = log sum_{allowed j} exp(u)       natural log; -inf if none
 *   o[b,i,h,:] = sum_{allowed j} exp(u - lse) * v[b,j,g,:]   (0 if none)
 *
 * computed tile by tile with an online softmax (running max and sum, [TA]
 * "Tiling the Computation" and "2. Online Softmax") so the Sq x Sk score
 * matrix never reaches device memory ([TA] "Enter Flash Attention").
 *
 * Conventions shared by every entry point.
 *  - All tensor and array arguments are DEVICE pointers unless stated.  The
 *    caller allocates and owns every buffer (inputs, outputs, LSE,
 *    workspace, block-mask arrays).  The library allocates nothing, frees
 *    nothing, never synchronises the device, and enqueues all work on the
 *    given stream (a hipStream_t passed as void*; NULL is the null stream).
 *    Work is asynchronous: outputs are valid once the stream reaches them.
 *  - Validation happens on the host before anything is enqueued.  On any
 *    failure the function returns a non-zero status, stores a message
 *    retrievable with attn_last_error() (thread-local), and enqueues
 *    nothing, so outputs are untouched.
 *  - attn_tensor strides are in ELEMENTS for the logical dims [B, S, H, D];
 *    the D stride must be 1 and the base pointer and the B/S/H strides must
 *    keep every row 16-byte aligned.  Any strides satisfying that are
 *    accepted, so [B, H, S, D] views ([GYM] transposes q/k/v to that layout
 *    for flex_attention) and packed-QKV slices ([FA] qkv of shape
 *    (batch, seqlen, 3, nheads, headdim)) are read in place.
 *    Gradients are written the same way, so dq/dk/dv may be slices of one
 *    packed dqkv tensor.
 *  - Supported head dims: 64 and 128.  Supported dtypes: ATTN_BF16 and
 *    ATTN_FP16 for all entry points ([TA] "FP16 vs. BF16 Representation": both
 *    16-bit types;
 *    fp32 accumulation, probabilities and dS rounded to the input type as
 *    matrix-core operands); ATTN_FP32 for attn_fwd (computed in fp32 on the
 *    vector ALU).  Every tensor of one call has the same dtype.
 */
#ifndef EXACT_ATTN_H
#define EXACT_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ATTN_OK = 0,
  ATTN_ERR_INVALID_ARG = 1,   /* a shape, stride, pointer or flag is wrong */
  ATTN_ERR_UNSUPPORTED = 2,   /* valid request this library does not cover */
  ATTN_ERR_WORKSPACE = 3,     /* workspace missing or smaller than required */
  ATTN_ERR_HIP = 4            /* the HIP runtime reported an error */
} attn_status;

typedef enum { ATTN_BF16 = 0, ATTN_FP32 = 1, ATTN_FP16 = 2 } attn_dtype;

typedef struct {
  void* data;          /* device pointer to element [0,0,0,0] */
  int32_t dtype;       /* attn_dtype */
  int64_t stride[4];   /* element strides of [B, S, H, D]; stride[3] == 1 */
} attn_tensor;

/* Mask predicate of a block-sparse mask ([GYM]: create_block_mask builds a
 * mask from a mask_mod such as q_idx >= kv_idx; [FX4]: mask patterns such as
 * causal and sliding window, evaluated inside the kernel).  The predicate is
 * the AND of the enabled terms:
 *   causal:   j <= i + (Sk - Sq)
 *   window:   as in attn_params (-1 = unbounded side)
 *   document: doc_q[b*Sq + i] == doc_k[b*Sk + j]  (device int32 arrays of
 *             shape [B, Sq] and [B, Sk]; both NULL to disable)
 * It does not depend on the head, so one mask serves every head. */
typedef struct {
  int32_t causal;
  int32_t window_left, window_right;
  const int32_t* doc_q;
  const int32_t* doc_k;
} attn_mask_desc;

/* Block mask: every (block_m x block_n) tile of every batch row classified
 * as 0 = EMPTY (no allowed pair; skipped), 1 = PARTIAL (predicate evaluated
 * per element), 2 = FULL (inside [0,Sq) x [0,Sk) and every pair allowed; no
 * predicate evaluated).  Lists are CSR-style per row of tiles, ascending,
 * with the unused tail zero-filled:
 *   cls            uint8 [B, nQ, nK]
 *   kv_num_partial int32 [B, nQ]      kv_idx_partial int32 [B, nQ, nK]
 *   kv_num_full    int32 [B, nQ]      kv_idx_full    int32 [B, nQ, nK]
 *   q_num_partial  int32 [B, nK]      q_idx_partial  int32 [B, nK, nQ]
 *   q_num_full     int32 [B, nK]      q_idx_full     int32 [B, nK, nQ]
 * The struct itself is host memory; the arrays are device memory carved by
 * block_mask_build() from one caller buffer. */
typedef struct {
  int32_t B, Sq, Sk, block_m, block_n, nQ, nK;
  attn_mask_desc desc;
  uint8_t* cls;
  int32_t* kv_num_partial;
  int32_t* kv_idx_partial;
  int32_t* kv_num_full;
  int32_t* kv_idx_full;
  int32_t* q_num_partial;
  int32_t* q_idx_partial;
  int32_t* q_num_full;
  int32_t* q_idx_full;
} attn_block_mask;

/* Problem description shared by attn_fwd / attn_bwd / attn_decode.
 * Arguments follow flash_attn_func ([FA] "Examples"): q [B, Sq, Hq, D],
 * k and v [B, Sk, Hkv, D] with Hq a multiple of Hkv (GQA/MQA). */
typedef struct {
  int32_t B, Sq, Sk, Hq, Hkv, D;
  float softmax_scale;          /* NaN means 1/sqrt(D) (the page's None) */
  int32_t causal;               /* bottom-right aligned when Sq != Sk */
  int32_t window_left;          /* -1 = unbounded; any side >= Sq + Sk
                                   excludes nothing and is taken as -1 */
  int32_t window_right;         /* -1 = unbounded (same rule) */
  const float* alibi_slopes;    /* device fp32, NULL = no ALiBi ([FA]:
                                   (nheads,) or (batch, nheads): element
                                   [b * alibi_batch_stride + h]) */
  int64_t alibi_batch_stride;   /* 0 for (Hq,), Hq for (B, Hq) */
  float softcap;                /* 0 = off; else softcap * tanh(s/softcap) */
  const attn_block_mask* block_mask;  /* NULL = dense; when given, causal
                                   must be 0 and the window (-1,-1): the
                                   mask's own predicate applies */
} attn_params;

/* Human-readable name of a status code (static storage). */
const char* attn_status_string(attn_status s);
/* Message describing the last failure on the calling thread ("" if none). */
const char* attn_last_error(void);

/* Testing hook: the bound, in sleep rounds, of every in-kernel wait of the
 * forward and decode kernels for launches enqueued after the call (a value
 * below 0 restores the default, about 4 million).  The bound is never reached
 * when the kernels' hand-over protocols work; a wait that reaches it stops
 * waiting, the kernel finishes normally, and the rows that may have read
 * unsynchronised data are written as NaN (o and lse); the decode path also
 * sets bit 2 of its status word (attn_decode).  With 0 the waits give up at
 * once, which lets a test see that path without a broken kernel.  Host only;
 * process-wide; never fails. */
void attn_debug_set_spin_limit(int32_t limit);

/* Schedule of the dK/dV pass for grouped-query heads (Hq > Hkv), for
 * launches enqueued after the call ([HF]: K and V are shared by the
 * G = Hq / Hkv query heads of a group and never repeated, so dK and dV are
 * sums over the group).
 *   0 (default) automatic: mode 2 when the (batch, kv head, 128-key block)
 *     grid has at least two workgroups per compute unit, else mode 1;
 *   1 one workgroup per query head and 128-key block, each writing fp32
 *     partial sums to the workspace, then a kernel that adds the G partials
 *     of each kv head in head order;
 *   2 one workgroup per kv head and 128-key block, looping over the G query
 *     heads into the same accumulators (no partials, no group sum).
 * Both are deterministic; they differ only in rounding order.  Any other
 * value selects 0.  Host only; process-wide; never fails. */
void attn_set_bwd_gqa_schedule(int32_t mode);

/* ---------------------------------------------------------------------
 * Forward ([TA] "Tiling the Computation", "2. Online Softmax",
 * "3. Weighted Sum of Values"; [FA] flash_attn_func; [FX4] score and mask
 * hooks, block-sparse iteration).
 *   q, k, v : inputs as above.  o : output [B, Sq, Hq, D], same dtype.
 *   lse     : output fp32 [B, Hq, Sq], contiguous, natural log.
 *   tile_trace : NULL, or uint8 [B, Hq, nQt, nKt] (contiguous) that the
 *             kernel fills with 1 / 2 for every tile it processed as
 *             partial / full and leaves untouched for tiles it skipped (the
 *             caller clears it).  nQt x nKt come from attn_fwd_tile_shape().
 *   workspace : unused by the forward (may be NULL / 0).
 * Errors: INVALID_ARG for inconsistent shapes, Hq % Hkv != 0, bad strides or
 * alignment, window < -1, softcap < 0 or non-finite, a block mask whose
 * B/Sq/Sk differ or combined with causal/window; UNSUPPORTED for D not in
 * {64, 128}, or a block mask tile other than block_m = 128 and block_n a
 * multiple of 64 (bf16) / 64 x 64 (fp32). */
attn_status attn_fwd(const attn_params* p, attn_tensor q, attn_tensor k,
                     attn_tensor v, attn_tensor o, float* lse,
                     uint8_t* tile_trace, void* workspace,
                     size_t workspace_bytes, void* stream);

/* Workspace bytes attn_fwd needs: 0 for every problem (the forward keeps
 * its running softmax state on chip and writes only o and lse).  Declared so
 * that callers size the workspaces of attn_fwd, attn_bwd and attn_decode the
 * same way.  Host only; never fails. */
size_t attn_fwd_workspace_size(const attn_params* p);

/* Query / key tile sizes the forward uses for this problem (host only).
 * The tile trace has ceil(Sq/block_m) x ceil(Sk/block_n) entries per head. */
attn_status attn_fwd_tile_shape(const attn_params* p, int32_t dtype,
                                int32_t* block_m, int32_t* block_n);

/* ---------------------------------------------------------------------
 * Backward from the saved LSE ([FX4]: the backward reuses the forward's
 * machinery; [FA]: deterministic backward flag).  Gradients of
 * sum(o * dout) with respect to q, k, v:
 *   dv[j,g] = sum_{h in g} sum_i P_ij dout_i
 *   dP_ij = <dout_i, v_j>;  Delta_i = <dout_i, o_i>
 *   dS_ij = P_ij (dP_ij - Delta_i) * (softcap ? 1 - tanh^2(s_ij/softcap) : 1)
 *   dq_i = scale sum_j dS_ij k_j;  dk[j,g] = scale sum_{h in g} sum_i dS_ij q_i
 * with P_ij = exp(u_ij - lse_i) recomputed tile by tile.  dk/dv of a kv head
 * sum the G query heads that read it.
 *   o, lse : the forward's outputs for the same inputs.
 *   dq, dk, dv : outputs, same shapes and dtype as q, k, v.
 *   deterministic : 1 = every output element is reduced in a fixed order
 *             without atomics (a separate dQ pass), so repeated calls are
 *             bitwise identical.  0 = dQ is accumulated by the dK/dV pass
 *             with fp32 atomic adds into the workspace and then scaled and
 *             rounded (FA's non-deterministic schedule).  dK and dV take no
 *             atomics in either schedule; at D = 128 their kernels differ,
 *             so dK of 0 and 1 agree to rounding, not bitwise.
 *             On gfx950 fp32 device atomics sustain only a few hundred G
 *             adds/s, so 0 is the slower schedule here (about 1.4x on
 *             B1 H32/8 S2048 D128 causal); 1 is the fast path.
 *             Other values: INVALID_ARG.
 *   workspace : at least attn_bwd_workspace_size(p) bytes, 256-byte aligned
 *             (enough for either value of deterministic: Delta and the LSE in
 *             exp2 units [B, Hq, Sq], fp32 per-head dK/dV partials
 *             [B, Sk, Hq, D] x 2 when Hq > Hkv, fp32 dQ [B, Sq, Hq, D]).
 *   p->block_mask : as in attn_fwd ([GYM] block mask, [FX4] block sparsity);
 *             the dK/dV pass walks each key block's query-block lists (FULL
 *             first, then PARTIAL), the dQ pass each query block's key-block
 *             lists; the predicate (causal / window / document) is evaluated
 *             on PARTIAL tiles only.  Needs block_m == 128, block_n a multiple
 *             of 128 and the query-block lists of block_mask_build().
 * Errors: as attn_fwd; UNSUPPORTED for fp32 inputs or a block mask whose
 * block_n is not a multiple of 128; WORKSPACE if too small. */
attn_status attn_bwd(const attn_params* p, attn_tensor q, attn_tensor k,
                     attn_tensor v, attn_tensor o, attn_tensor dout,
                     const float* lse, attn_tensor dq, attn_tensor dk,
                     attn_tensor dv, int32_t deterministic, void* workspace,
                     size_t workspace_bytes, void* stream);
size_t attn_bwd_workspace_size(const attn_params* p);

/* One stage of attn_bwd, same arguments and workspace, for callers that
 * time or interleave the stages.  Enqueuing stages 0, 1, 2, 3 in order on one
 * stream (with the same workspace) is exactly attn_bwd:
 *   0  deterministic == 1: the dQ kernel, which also writes
 *      Delta_i = <dout_i, o_i> and the LSE in exp2 units into the workspace;
 *      deterministic == 0: Delta and the LSE alone, and zeroes the dQ
 *      accumulator
 *   1  dK/dV kernel, reading Delta (fp32 per-head partials in the workspace
 *      when Hq > Hkv, else dk/dv directly; with deterministic == 0 also the
 *      atomic dQ accumulation)
 *   2  sum of the per-head partials of each kv head into dk/dv, in head order
 *      (nothing to do when Hq == Hkv)
 *   3  deterministic == 0: the scale-and-round of the dQ accumulator;
 *      nothing to do for deterministic == 1
 * Errors: as attn_bwd; INVALID_ARG for a stage outside 0..3. */
attn_status attn_bwd_stage(const attn_params* p, attn_tensor q, attn_tensor k,
                           attn_tensor v, attn_tensor o, attn_tensor dout,
                           const float* lse, attn_tensor dq, attn_tensor dk,
                           attn_tensor dv, int32_t deterministic,
                           void* workspace, size_t workspace_bytes,
                           int32_t stage, void* stream);

/* ---------------------------------------------------------------------
 * Decode over a KV cache ([FA] flash_attn_with_kvcache: q attends to the
 * first cache_seqlens[b] rows of its batch row of k_cache / v_cache; no
 * backward).  The Sq queries of a sequence are its last Sq positions (one
 * token, or a chunk of a prefill, or the draft tokens of speculative
 * decoding); with p->causal, bottom-right aligned as in attn_fwd, query t
 * attends to the first L - Sq + 1 + t of its L keys (none if that is <= 0:
 * o = 0, lse = -inf).  Split-K: the keys of every job (sequence, kv head,
 * group of up to 128 rows, a row being a (query t, query head) pair numbered
 * t * (Hq/Hkv) + head), in 32-key steps and job order, are cut into equal
 * contiguous ranges, one per workgroup; the pieces are attended
 * independently and merged with the LSE-weighted combine
 * lse = log sum_s exp(lse_s),  o = sum_s exp(lse_s - lse) o_s.  Each job
 * reads its sequence's keys once, so Sq * Hq/Hkv <= 128 reads them once.
 *   p : B, Sq (1 <= Sq <= Sk, else INVALID_ARG), Hq, Hkv, D as usual;
 *       Sk = cache capacity Smax; scale, softcap and causal apply; window,
 *       ALiBi and block masks are not supported by this entry point
 *       (UNSUPPORTED).
 *   q : [B, Sq, Hq, D];  k_cache, v_cache : [B, Smax, Hkv, D].
 *   cache_seqlens : device int32 [B], each in [0, Smax].  The lengths are read
 *       on the device only: a value outside that range is clamped to it and
 *       reported in the workspace status word (below).  A sequence of length
 *       0 gives o = 0 and lse = -inf.
 *   num_splits : number of ranges (workgroups) the total key work is cut
 *       into; 0 = one per compute unit of the current device.  At most
 *       65536.  Any value gives the same result up to rounding.
 *   o : [B, Sq, Hq, D];  lse : fp32 [B, Hq, Sq] contiguous.
 *   workspace : at least attn_decode_workspace_size(p, num_splits) bytes,
 *       256-byte aligned.  Its first 4 bytes are a sticky status word (uint32)
 *       that the kernels only OR bits into and never clear: bit 1 = some
 *       cache_seqlens[b] was outside [0, Smax - s_new] (s_new = 0 without an
 *       append) and was clamped; bit 2 = an in-kernel wait reached its bound
 *       (see attn_debug_set_spin_limit; the rows concerned are NaN).  The
 *       caller zeroes the word (e.g. when allocating the workspace) and reads
 *       it when it wants, after the stream has reached the call.  The rest of
 *       the workspace is scratch.
 */
attn_status attn_decode(const attn_params* p, attn_tensor q,
                        attn_tensor k_cache, attn_tensor v_cache,
                        const int32_t* cache_seqlens, int32_t num_splits,
                        attn_tensor o, float* lse, void* workspace,
                        size_t workspace_bytes, void* stream);
size_t attn_decode_workspace_size(const attn_params* p, int32_t num_splits);

/* ---------------------------------------------------------------------
 * attn_decode without a workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  Same computation, arguments, kernels and results as
 * attn_decode (bitwise, for the same num_splits), except:
 *   - the scratch is a device array inside the library, 64 MiB on each GPU
 *     it runs on (held until the process ends; attn_decode_noalloc_max_bytes()
 *     returns the size).  A problem whose attn_decode_workspace_size exceeds
 *     it is rejected with ATTN_ERR_UNSUPPORTED before anything is enqueued.
 *   - status : NULL, or a caller-owned device uint32 that receives the
 *     sticky status bits attn_decode writes into its workspace word (1 = a
 *     cache length was clamped, 2 = an in-kernel wait reached its bound);
 *     the library never clears it.
 *   - the scratch of the current device is shared by every call on that
 *     device: calls that may overlap on one GPU (different streams, or
 *     threads) race and must be serialised by the caller.  Nothing in the
 *     scratch needs clearing between calls (every value is written before it
 *     is read within a call).
 * The current device must be the device of the tensors and the stream.  The
 * call allocates and frees nothing (no hipMalloc / hipFree, no allocating
 * library routine); the first call on a device looks the scratch up with
 * hipGetSymbolAddress, which does not allocate. */
attn_status attn_decode_noalloc(const attn_params* p, attn_tensor q,
                                attn_tensor k_cache, attn_tensor v_cache,
                                const int32_t* cache_seqlens, int32_t num_splits,
                                attn_tensor o, float* lse, uint32_t* status,
                                void* stream);
size_t attn_decode_noalloc_max_bytes(void);

/* ---------------------------------------------------------------------
 * Decode over a paged and/or batch-indexed KV cache with in-place append
 * ([FA] flash_attn_with_kvcache: "k_cache, v_cache: cached keys/values,
 * updated inplace", arguments k, v, cache_batch_idx, block_table).
 *   block_table : device int32 [B, max_blocks] or NULL.  When set, k_cache and
 *       v_cache are [num_pages, page_size, Hkv, D] and row r of sequence b is
 *       row r % page_size of page block_table[b, r / page_size]; page_size
 *       is a positive multiple of 32 and p->Sk must equal
 *       max_blocks * page_size (the per-sequence capacity).  Entries outside
 *       [0, num_pages) are clamped to that range on the device.
 *   cache_batch_idx : device int32 [B] or NULL (contiguous caches only):
 *       sequence b uses batch row cache_batch_idx[b] of k_cache / v_cache,
 *       which then have cache_batch rows ([cache_batch, Sk, Hkv, D]); values
 *       are clamped to [0, cache_batch).
 *   k_new, v_new : [B, s_new, Hkv, D] of q's dtype (bf16 or fp16; data NULL =
 *       no append).  Before
 *       attending, rows [L_b, L_b + s_new) of each sequence's cache receive
 *       them (L_b = cache_seqlens[b], clamped to [0, Sk - s_new], a clamp
 *       reported by bit 1 of the workspace status word) and the
 *       queries then attend to L_b + s_new rows (with causal and
 *       Sq == s_new, query t sees the cache and the new rows up to t).  cache_seqlens is read, not
 *       advanced.  The caches are written in place (stream-ordered).
 * Other arguments, outputs, workspace and errors as attn_decode (which is
 * this call with a NULL kv).  Errors: INVALID_ARG for a page_size that is
 * not a positive multiple of 32, a capacity mismatch, k_new without v_new,
 * s_new outside [1, Sk]; UNSUPPORTED for block_table with cache_batch_idx. */
typedef struct {
  const int32_t* block_table;
  int32_t max_blocks;
  int32_t page_size;
  int32_t num_pages;
  const int32_t* cache_batch_idx;
  int32_t cache_batch;
  attn_tensor k_new, v_new;
  int32_t s_new;
} attn_kvcache;
attn_status attn_decode_kvcache(const attn_params* p, attn_tensor q, attn_tensor k_cache,
                                attn_tensor v_cache, const int32_t* cache_seqlens,
                                const attn_kvcache* kv, int32_t num_splits, attn_tensor o,
                                float* lse, void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------
 * Block-mask construction on the device ([GYM] create_block_mask with
 * BLOCK_SIZE; [FX4] block-sparse masks skip tiles with nothing to compute).
 * Classifies every tile exactly as if the predicate of `m` were evaluated on
 * every in-bounds pair of the tile (a tile crossing the end of the sequence
 * is never FULL): the causal / window part in closed form from the tile's
 * corner rows, document ids compared once per tile edge (a tile holding a
 * single document on each side) or, where a document boundary crosses the
 * tile, pair by pair; then writes the ascending CSR lists (forward and
 * transposed).  Any int32 document ids are accepted (they need not be
 * sorted or contiguous).
 *   buffer : device memory of at least attn_block_mask_bytes(...) bytes,
 *            256-byte aligned; `out` (host struct) receives the header and
 *            pointers into it.
 * Errors: INVALID_ARG for non-positive sizes, window < -1, only one of
 * doc_q / doc_k given; UNSUPPORTED for block_m or block_n above 1024 with
 * document ids; WORKSPACE if the buffer is too small. */
size_t attn_block_mask_bytes(int32_t B, int32_t Sq, int32_t Sk,
                             int32_t block_m, int32_t block_n);
attn_status block_mask_build(const attn_mask_desc* m, int32_t B, int32_t Sq,
                             int32_t Sk, int32_t block_m, int32_t block_n,
                             void* buffer, size_t buffer_bytes,
                             attn_block_mask* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* EXACT_ATTN_H */
