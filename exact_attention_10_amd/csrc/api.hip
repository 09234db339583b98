// C-ABI layer: argument validation, defaults and dispatch to the kernels.
// Declarations and the meaning of every argument are in include/attn.h.

#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "attn.h"
#include "internal.h"

namespace attn {
namespace {
std::atomic<int> g_spin_limit{kDefaultSpinLimit};
std::atomic<int> g_bwd_gqa_mode{0};
}
int spin_limit() { return g_spin_limit.load(std::memory_order_relaxed); }
bool bwd_group_loop_choice(long kv_grid, int cus) {
  switch (g_bwd_gqa_mode.load(std::memory_order_relaxed)) {
    case 1: return false;
    case 2: return true;
    default: return kv_grid >= 2L * cus;
  }
}
}  // namespace attn

namespace {

thread_local char g_err[512] = "";

attn_status fail(attn_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

attn_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ATTN_OK;
  return fail(ATTN_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

size_t dtype_size(int32_t dt) { return dt == ATTN_FP32 ? 4 : 2; }

// A tensor of logical shape [B, S, H, D]: D stride 1, 16-byte aligned rows.
attn_status check_tensor(const char* name, const attn_tensor& t, int32_t dtype,
                         int64_t B, int64_t S, int64_t H, bool need_data) {
  if (t.dtype != dtype)
    return fail(ATTN_ERR_INVALID_ARG, "%s: dtype %d differs from q's dtype %d", name, t.dtype, dtype);
  if (t.stride[3] != 1)
    return fail(ATTN_ERR_INVALID_ARG, "%s: the head-dim stride must be 1 (got %lld)", name,
                (long long)t.stride[3]);
  const size_t es = dtype_size(dtype);
  for (int i = 0; i < 3; ++i) {
    if (t.stride[i] < 0)
      return fail(ATTN_ERR_INVALID_ARG, "%s: negative stride", name);
    if ((t.stride[i] * es) % 16 != 0)
      return fail(ATTN_ERR_INVALID_ARG, "%s: stride[%d]=%lld elements is not a multiple of 16 bytes",
                  name, i, (long long)t.stride[i]);
  }
  if (need_data && B * S * H > 0) {
    if (t.data == nullptr) return fail(ATTN_ERR_INVALID_ARG, "%s: null data pointer", name);
    if (reinterpret_cast<uintptr_t>(t.data) % 16 != 0)
      return fail(ATTN_ERR_INVALID_ARG, "%s: data pointer is not 16-byte aligned", name);
  }
  return ATTN_OK;
}

struct Common {
  float scale;
};

attn_status check_params(const attn_params* p, Common* out) {
  if (p == nullptr) return fail(ATTN_ERR_INVALID_ARG, "params is NULL");
  if (p->B < 0 || p->Sq < 0 || p->Sk < 0)
    return fail(ATTN_ERR_INVALID_ARG, "negative B/Sq/Sk (%d, %d, %d)", p->B, p->Sq, p->Sk);
  if (p->Hq <= 0 || p->Hkv <= 0)
    return fail(ATTN_ERR_INVALID_ARG, "head counts must be positive (Hq=%d, Hkv=%d)", p->Hq, p->Hkv);
  if (p->Hq % p->Hkv != 0)
    return fail(ATTN_ERR_INVALID_ARG, "Hq=%d is not a multiple of Hkv=%d", p->Hq, p->Hkv);
  if (p->D != 64 && p->D != 128)
    return fail(ATTN_ERR_UNSUPPORTED, "head dim %d is not supported (64 or 128)", p->D);
  if (p->window_left < -1 || p->window_right < -1)
    return fail(ATTN_ERR_INVALID_ARG, "window sides must be >= -1 (got %d, %d)", p->window_left,
                p->window_right);
  if (!(p->softcap >= 0.0f) || !std::isfinite(p->softcap))
    return fail(ATTN_ERR_INVALID_ARG, "softcap must be finite and >= 0 (got %g)", (double)p->softcap);
  float scale = p->softmax_scale;
  if (std::isnan(scale)) scale = 1.0f / std::sqrt(static_cast<float>(p->D));
  if (!std::isfinite(scale)) return fail(ATTN_ERR_INVALID_ARG, "softmax_scale is not finite");
  if (p->alibi_slopes != nullptr && p->alibi_batch_stride != 0 && p->alibi_batch_stride != p->Hq)
    return fail(ATTN_ERR_INVALID_ARG, "alibi_batch_stride must be 0 or Hq (got %lld)",
                (long long)p->alibi_batch_stride);
  out->scale = scale;
  return ATTN_OK;
}

void strides3(const attn_tensor& t, int64_t* sb, int64_t* ss, int64_t* sh) {
  *sb = t.stride[0];
  *ss = t.stride[1];
  *sh = t.stride[2];
}

// A window side of Sq + Sk or more excludes no key (every |i + delta - j|
// is smaller), so it is the unbounded side; mapping it to -1 keeps the
// kernels' index arithmetic (sums of positions and window sides) inside int.
int32_t window_side(int32_t side, int32_t Sq, int32_t Sk) {
  return side >= 0 && (int64_t)side >= (int64_t)Sq + Sk ? -1 : side;
}

attn::MaskArgs mask_from(const attn_params* p) {
  attn::MaskArgs m{};
  if (p->block_mask != nullptr) {
    m.causal = p->block_mask->desc.causal;
    m.wl = p->block_mask->desc.window_left;
    m.wr = p->block_mask->desc.window_right;
    m.doc_q = p->block_mask->desc.doc_q;
    m.doc_k = p->block_mask->desc.doc_k;
  } else {
    m.causal = p->causal;
    m.wl = p->window_left;
    m.wr = p->window_right;
    m.doc_q = m.doc_k = nullptr;
  }
  m.wl = window_side(m.wl, p->Sq, p->Sk);
  m.wr = window_side(m.wr, p->Sq, p->Sk);
  return m;
}

attn_status check_block_mask(const attn_params* p, int32_t dtype) {
  const attn_block_mask* bm = p->block_mask;
  if (bm == nullptr) return ATTN_OK;
  if (p->causal || p->window_left != -1 || p->window_right != -1)
    return fail(ATTN_ERR_INVALID_ARG,
                "a block mask carries its own predicate: set causal=0 and window=(-1,-1)");
  if (bm->B != p->B || bm->Sq != p->Sq || bm->Sk != p->Sk)
    return fail(ATTN_ERR_INVALID_ARG, "block mask was built for B=%d Sq=%d Sk=%d, problem is B=%d Sq=%d Sk=%d",
                bm->B, bm->Sq, bm->Sk, p->B, p->Sq, p->Sk);
  if (bm->kv_num_full == nullptr || bm->kv_idx_full == nullptr || bm->kv_num_partial == nullptr ||
      bm->kv_idx_partial == nullptr)
    return fail(ATTN_ERR_INVALID_ARG, "block mask lists are NULL");
  if ((bm->desc.doc_q == nullptr) != (bm->desc.doc_k == nullptr))
    return fail(ATTN_ERR_INVALID_ARG, "block mask: give both doc_q and doc_k or neither");
  const int bn_kernel = dtype != ATTN_FP32 ? attn::kFwdBN : attn::kFwdF32BN;
  const int bm_kernel = dtype != ATTN_FP32 ? attn::kFwdBM : attn::kFwdF32BM;
  const bool m_ok = dtype != ATTN_FP32 ? bm->block_m == bm_kernel : bm->block_m % bm_kernel == 0;
  if (!m_ok || bm->block_n <= 0 || bm->block_n % bn_kernel != 0)
    return fail(ATTN_ERR_UNSUPPORTED,
                "block mask tile %dx%d is not supported (rows %s %d, columns a multiple of %d)",
                bm->block_m, bm->block_n, dtype != ATTN_FP32 ? "==" : "a multiple of", bm_kernel,
                bn_kernel);
  if (bm->nQ != (p->Sq + bm->block_m - 1) / bm->block_m || bm->nK != (p->Sk + bm->block_n - 1) / bm->block_n)
    return fail(ATTN_ERR_INVALID_ARG, "block mask tile grid does not match its sizes");
  return ATTN_OK;
}

}  // namespace

extern "C" {

const char* attn_status_string(attn_status s) {
  switch (s) {
    case ATTN_OK: return "ATTN_OK";
    case ATTN_ERR_INVALID_ARG: return "ATTN_ERR_INVALID_ARG";
    case ATTN_ERR_UNSUPPORTED: return "ATTN_ERR_UNSUPPORTED";
    case ATTN_ERR_WORKSPACE: return "ATTN_ERR_WORKSPACE";
    case ATTN_ERR_HIP: return "ATTN_ERR_HIP";
  }
  return "ATTN_ERR_UNKNOWN";
}

const char* attn_last_error(void) { return g_err; }

void attn_debug_set_spin_limit(int32_t limit) {
  attn::g_spin_limit.store(limit < 0 ? attn::kDefaultSpinLimit : limit, std::memory_order_relaxed);
}

void attn_set_bwd_gqa_schedule(int32_t mode) {
  attn::g_bwd_gqa_mode.store(mode == 1 || mode == 2 ? mode : 0, std::memory_order_relaxed);
}

attn_status attn_fwd_tile_shape(const attn_params* p, int32_t dtype, int32_t* block_m,
                                int32_t* block_n) {
  g_err[0] = 0;
  if (p == nullptr || block_m == nullptr || block_n == nullptr)
    return fail(ATTN_ERR_INVALID_ARG, "NULL argument");
  if (dtype != ATTN_BF16 && dtype != ATTN_FP16 && dtype != ATTN_FP32)
    return fail(ATTN_ERR_UNSUPPORTED, "dtype %d", dtype);
  if (p->block_mask != nullptr) {
    *block_m = p->block_mask->block_m;
    *block_n = p->block_mask->block_n;
  } else if (dtype != ATTN_FP32) {
    *block_m = attn::fwd_bf16_rows_per_block(p->B, p->Sq, p->Hq, p->causal, false);
    *block_n = attn::kFwdBN;
  } else {
    *block_m = attn::kFwdF32BM;
    *block_n = attn::kFwdF32BN;
  }
  return ATTN_OK;
}

attn_status attn_fwd(const attn_params* p, attn_tensor q, attn_tensor k, attn_tensor v,
                     attn_tensor o, float* lse, uint8_t* tile_trace, void* workspace,
                     size_t workspace_bytes, void* stream) {
  (void)workspace;
  (void)workspace_bytes;
  g_err[0] = 0;
  Common cm;
  attn_status st = check_params(p, &cm);
  if (st != ATTN_OK) return st;
  const int32_t dt = q.dtype;
  if (dt != ATTN_BF16 && dt != ATTN_FP16 && dt != ATTN_FP32) return fail(ATTN_ERR_UNSUPPORTED, "q: dtype %d", dt);
  if ((st = check_tensor("q", q, dt, p->B, p->Sq, p->Hq, true)) != ATTN_OK) return st;
  if ((st = check_tensor("k", k, dt, p->B, p->Sk, p->Hkv, true)) != ATTN_OK) return st;
  if ((st = check_tensor("v", v, dt, p->B, p->Sk, p->Hkv, true)) != ATTN_OK) return st;
  if ((st = check_tensor("o", o, dt, p->B, p->Sq, p->Hq, true)) != ATTN_OK) return st;
  if (lse == nullptr && p->B * p->Sq > 0) return fail(ATTN_ERR_INVALID_ARG, "lse is NULL");
  if ((st = check_block_mask(p, dt)) != ATTN_OK) return st;

  attn::FwdArgs a{};
  a.q = q.data; a.k = k.data; a.v = v.data; a.o = o.data;
  a.f16 = dt == ATTN_FP16;
  a.lse = lse;
  a.trace = tile_trace;
  strides3(q, &a.q_sb, &a.q_ss, &a.q_sh);
  strides3(k, &a.k_sb, &a.k_ss, &a.k_sh);
  strides3(v, &a.v_sb, &a.v_ss, &a.v_sh);
  strides3(o, &a.o_sb, &a.o_ss, &a.o_sh);
  a.B = p->B; a.Sq = p->Sq; a.Sk = p->Sk; a.Hq = p->Hq; a.Hkv = p->Hkv; a.D = p->D;
  a.scale = cm.scale;
  a.alibi = p->alibi_slopes;
  a.alibi_sb = p->alibi_batch_stride;
  a.softcap = p->softcap;
  a.mask = mask_from(p);
  a.spin_limit = attn::spin_limit();
  if (p->block_mask != nullptr) {
    const attn_block_mask* bm = p->block_mask;
    a.tiles.kv_num_full = bm->kv_num_full;
    a.tiles.kv_idx_full = bm->kv_idx_full;
    a.tiles.kv_num_partial = bm->kv_num_partial;
    a.tiles.kv_idx_partial = bm->kv_idx_partial;
    a.tiles.nQ = bm->nQ;
    a.tiles.nK = bm->nK;
    a.tiles.block_m = bm->block_m;
    a.tiles.sub = bm->block_n / (dt != ATTN_FP32 ? attn::kFwdBN : attn::kFwdF32BN);
    a.nQt = bm->nQ;
    a.nKt = bm->nK;
  } else {
    const int bmr = dt != ATTN_FP32 ? attn::fwd_bf16_rows_per_block(p->B, p->Sq, p->Hq, p->causal, false)
                                    : attn::kFwdF32BM;
    const int bnr = dt != ATTN_FP32 ? attn::kFwdBN : attn::kFwdF32BN;
    a.nQt = (p->Sq + bmr - 1) / bmr;
    a.nKt = (p->Sk + bnr - 1) / bnr;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = dt != ATTN_FP32 ? attn::launch_fwd_bf16(a, s) : attn::launch_fwd_f32(a, s);
  return hip_status(e, "attn_fwd launch");
}

static attn_status bwd_impl(const attn_params* p, attn_tensor q, attn_tensor k, attn_tensor v,
                            attn_tensor o, attn_tensor dout, const float* lse, attn_tensor dq,
                            attn_tensor dk, attn_tensor dv, int32_t deterministic, void* workspace,
                            size_t workspace_bytes, int stage_mask, void* stream) {
  g_err[0] = 0;
  Common cm;
  attn_status st = check_params(p, &cm);
  if (st != ATTN_OK) return st;
  const int32_t dt = q.dtype;
  if (dt != ATTN_BF16 && dt != ATTN_FP16)
    return fail(ATTN_ERR_UNSUPPORTED, "attn_bwd supports bf16 and fp16 (dtype %d)", dt);
  if ((st = check_tensor("q", q, dt, p->B, p->Sq, p->Hq, true)) != ATTN_OK) return st;
  if ((st = check_tensor("k", k, dt, p->B, p->Sk, p->Hkv, true)) != ATTN_OK) return st;
  if ((st = check_tensor("v", v, dt, p->B, p->Sk, p->Hkv, true)) != ATTN_OK) return st;
  if ((st = check_tensor("o", o, dt, p->B, p->Sq, p->Hq, true)) != ATTN_OK) return st;
  if ((st = check_tensor("dout", dout, dt, p->B, p->Sq, p->Hq, true)) != ATTN_OK) return st;
  if ((st = check_tensor("dq", dq, dt, p->B, p->Sq, p->Hq, true)) != ATTN_OK) return st;
  if ((st = check_tensor("dk", dk, dt, p->B, p->Sk, p->Hkv, true)) != ATTN_OK) return st;
  if ((st = check_tensor("dv", dv, dt, p->B, p->Sk, p->Hkv, true)) != ATTN_OK) return st;
  if (lse == nullptr && p->B * p->Sq > 0) return fail(ATTN_ERR_INVALID_ARG, "lse is NULL");
  if ((st = check_block_mask(p, dt)) != ATTN_OK) return st;
  if (p->block_mask != nullptr) {
    const attn_block_mask* bm = p->block_mask;
    if (bm->block_n % 128 != 0)
      return fail(ATTN_ERR_UNSUPPORTED, "attn_bwd takes block masks with block_n a multiple of 128 (got %d)",
                  bm->block_n);
    if (bm->q_num_full == nullptr || bm->q_idx_full == nullptr || bm->q_num_partial == nullptr ||
        bm->q_idx_partial == nullptr)
      return fail(ATTN_ERR_INVALID_ARG, "block mask query lists are NULL (attn_bwd needs them)");
  }
  if (deterministic != 0 && deterministic != 1)
    return fail(ATTN_ERR_INVALID_ARG, "deterministic must be 0 or 1 (got %d)", deterministic);
  const size_t need = attn_bwd_workspace_size(p);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need))
    return fail(ATTN_ERR_WORKSPACE, "attn_bwd needs %zu workspace bytes, got %zu", need, workspace_bytes);
  if (need > 0 && reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
    return fail(ATTN_ERR_WORKSPACE, "workspace must be 256-byte aligned");

  attn::BwdArgs a{};
  a.f16 = dt == ATTN_FP16;
  a.q = q.data; a.k = k.data; a.v = v.data; a.o = o.data; a.dout = dout.data;
  a.lse = lse;
  a.dq = dq.data; a.dk = dk.data; a.dv = dv.data;
  strides3(q, &a.q_sb, &a.q_ss, &a.q_sh);
  strides3(k, &a.k_sb, &a.k_ss, &a.k_sh);
  strides3(v, &a.v_sb, &a.v_ss, &a.v_sh);
  strides3(o, &a.o_sb, &a.o_ss, &a.o_sh);
  strides3(dout, &a.do_sb, &a.do_ss, &a.do_sh);
  strides3(dq, &a.dq_sb, &a.dq_ss, &a.dq_sh);
  strides3(dk, &a.dk_sb, &a.dk_ss, &a.dk_sh);
  strides3(dv, &a.dv_sb, &a.dv_ss, &a.dv_sh);
  a.B = p->B; a.Sq = p->Sq; a.Sk = p->Sk; a.Hq = p->Hq; a.Hkv = p->Hkv; a.D = p->D;
  a.scale = cm.scale;
  a.alibi = p->alibi_slopes;
  a.alibi_sb = p->alibi_batch_stride;
  a.softcap = p->softcap;
  a.mask = mask_from(p);
  if (p->block_mask != nullptr) {
    const attn_block_mask* bm = p->block_mask;
    a.tiles.kv_num_full = bm->kv_num_full;
    a.tiles.kv_idx_full = bm->kv_idx_full;
    a.tiles.kv_num_partial = bm->kv_num_partial;
    a.tiles.kv_idx_partial = bm->kv_idx_partial;
    a.tiles.q_num_full = bm->q_num_full;
    a.tiles.q_idx_full = bm->q_idx_full;
    a.tiles.q_num_partial = bm->q_num_partial;
    a.tiles.q_idx_partial = bm->q_idx_partial;
    a.tiles.nQ = bm->nQ;
    a.tiles.nK = bm->nK;
    a.tiles.block_n = bm->block_n;
  }
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  a.delta = static_cast<float*>(workspace);
  const size_t rows_bytes = up((size_t)p->B * p->Hq * p->Sq * sizeof(float));
  a.lse2 = reinterpret_cast<float*>(static_cast<char*>(workspace) + rows_bytes);
  char* rest = static_cast<char*>(workspace) + 2 * rows_bytes;
  const size_t part = up((size_t)p->B * p->Sk * p->Hq * p->D * sizeof(float));
  a.part_dk = p->Hq / p->Hkv > 1 ? reinterpret_cast<float*>(rest) : nullptr;
  a.part_dv = p->Hq / p->Hkv > 1 ? reinterpret_cast<float*>(rest + part) : nullptr;
  if (p->Hq / p->Hkv > 1) rest += 2 * part;
  a.dq_acc = deterministic ? nullptr : reinterpret_cast<float*>(rest);
  return hip_status(attn::launch_bwd_bf16(a, stage_mask, static_cast<hipStream_t>(stream)), "attn_bwd launch");
}

attn_status attn_bwd(const attn_params* p, attn_tensor q, attn_tensor k, attn_tensor v,
                     attn_tensor o, attn_tensor dout, const float* lse, attn_tensor dq,
                     attn_tensor dk, attn_tensor dv, int32_t deterministic, void* workspace,
                     size_t workspace_bytes, void* stream) {
  return bwd_impl(p, q, k, v, o, dout, lse, dq, dk, dv, deterministic, workspace, workspace_bytes,
                  attn::kBwdAllStages, stream);
}

attn_status attn_bwd_stage(const attn_params* p, attn_tensor q, attn_tensor k, attn_tensor v,
                           attn_tensor o, attn_tensor dout, const float* lse, attn_tensor dq,
                           attn_tensor dk, attn_tensor dv, int32_t deterministic,
                           void* workspace, size_t workspace_bytes, int32_t stage,
                           void* stream) {
  g_err[0] = 0;
  if (stage < 0 || stage > 3) return fail(ATTN_ERR_INVALID_ARG, "stage %d is not in 0..3", stage);
  return bwd_impl(p, q, k, v, o, dout, lse, dq, dk, dv, deterministic, workspace, workspace_bytes,
                  1 << stage, stream);
}

size_t attn_fwd_workspace_size(const attn_params* p) {
  (void)p;
  return 0;
}

size_t attn_bwd_workspace_size(const attn_params* p) {
  if (p == nullptr || p->B < 0 || p->Hq <= 0 || p->Hkv <= 0 || p->Sq < 0 || p->Sk < 0 || p->D <= 0)
    return 0;
  return attn::bwd_workspace_bytes(p->B, p->Hq, p->Hkv, p->Sq, p->Sk, p->D);
}

size_t attn_decode_workspace_size(const attn_params* p, int32_t num_splits) {
  if (p == nullptr || p->B <= 0 || p->Hq <= 0 || p->Hkv <= 0 || p->D <= 0 || p->Sk <= 0 ||
      num_splits < 0 || num_splits > 65536)
    return 0;
  return attn::decode_workspace(p->B, p->Hq, p->Hkv, p->Sq, p->D, attn::decode_parts(num_splits)).bytes;
}

static attn_status decode_impl(const attn_params* p, attn_tensor q, attn_tensor k_cache,
                               attn_tensor v_cache, const int32_t* cache_seqlens,
                               const attn_kvcache* kv, int32_t num_splits, attn_tensor o, float* lse,
                               void* workspace, size_t workspace_bytes, void* stream,
                               uint32_t* status = nullptr, const char* scratch_name = nullptr) {
  g_err[0] = 0;
  Common cm;
  attn_status st = check_params(p, &cm);
  if (st != ATTN_OK) return st;
  if (p->Sq < 1 || p->Sq > p->Sk)
    return fail(ATTN_ERR_INVALID_ARG, "attn_decode takes 1 <= Sq <= Sk queries per sequence (Sq=%d, Sk=%d)",
                p->Sq, p->Sk);
  if (p->window_left != -1 || p->window_right != -1 || p->alibi_slopes != nullptr || p->block_mask != nullptr)
    return fail(ATTN_ERR_UNSUPPORTED, "attn_decode supports scale, softcap and causal only");
  const int32_t dt = q.dtype;
  if (dt != ATTN_BF16 && dt != ATTN_FP16)
    return fail(ATTN_ERR_UNSUPPORTED, "attn_decode supports bf16 and fp16 (dtype %d)", dt);
  const bool paged = kv != nullptr && kv->block_table != nullptr;
  const bool remap = kv != nullptr && kv->cache_batch_idx != nullptr;
  const bool append = kv != nullptr && kv->k_new.data != nullptr;
  if (kv != nullptr && (kv->k_new.data == nullptr) != (kv->v_new.data == nullptr))
    return fail(ATTN_ERR_INVALID_ARG, "k_new and v_new must be given together");
  if (paged && remap)
    return fail(ATTN_ERR_UNSUPPORTED, "cache_batch_idx is for contiguous caches (not with block_table)");
  if (paged) {
    if (kv->page_size <= 0 || kv->page_size % 32 != 0)
      return fail(ATTN_ERR_INVALID_ARG, "page_size must be a positive multiple of 32 (got %d)", kv->page_size);
    if (kv->max_blocks <= 0 || kv->num_pages <= 0)
      return fail(ATTN_ERR_INVALID_ARG, "max_blocks and num_pages must be positive");
    if ((int64_t)kv->max_blocks * kv->page_size != p->Sk)
      return fail(ATTN_ERR_INVALID_ARG, "paged cache: Sk (%d) must equal max_blocks * page_size (%lld)",
                  p->Sk, (long long)kv->max_blocks * kv->page_size);
  }
  if (remap && kv->cache_batch <= 0)
    return fail(ATTN_ERR_INVALID_ARG, "cache_batch must be positive with cache_batch_idx");
  if (append && (kv->s_new <= 0 || kv->s_new > p->Sk))
    return fail(ATTN_ERR_INVALID_ARG, "s_new must be in [1, Sk] (got %d)", kv->s_new);
  if ((st = check_tensor("q", q, dt, p->B, p->Sq, p->Hq, true)) != ATTN_OK) return st;
  const int64_t cache_rows0 = paged ? kv->num_pages : (remap ? kv->cache_batch : p->B);
  const int64_t cache_rows1 = paged ? kv->page_size : p->Sk;
  if ((st = check_tensor("k_cache", k_cache, dt, cache_rows0, cache_rows1, p->Hkv, true)) != ATTN_OK) return st;
  if ((st = check_tensor("v_cache", v_cache, dt, cache_rows0, cache_rows1, p->Hkv, true)) != ATTN_OK) return st;
  if (append) {
    if ((st = check_tensor("k_new", kv->k_new, dt, p->B, kv->s_new, p->Hkv, true)) != ATTN_OK) return st;
    if ((st = check_tensor("v_new", kv->v_new, dt, p->B, kv->s_new, p->Hkv, true)) != ATTN_OK) return st;
  }
  if ((st = check_tensor("o", o, dt, p->B, p->Sq, p->Hq, true)) != ATTN_OK) return st;
  if (p->B > 0 && (cache_seqlens == nullptr || lse == nullptr))
    return fail(ATTN_ERR_INVALID_ARG, "cache_seqlens and lse must not be NULL");
  if (num_splits < 0 || num_splits > 65536)
    return fail(ATTN_ERR_INVALID_ARG, "num_splits must be in [0, 65536] (got %d)", num_splits);
  if (p->B == 0) return ATTN_OK;
  const size_t need = attn_decode_workspace_size(p, num_splits);
  if (scratch_name != nullptr && need > workspace_bytes)
    return fail(ATTN_ERR_UNSUPPORTED,
                "this decode needs %zu bytes of scratch; %s holds at most %zu (use attn_decode "
                "with a caller workspace, or fewer splits / sequences)",
                need, scratch_name, workspace_bytes);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need))
    return fail(ATTN_ERR_WORKSPACE, "attn_decode needs %zu workspace bytes, got %zu", need, workspace_bytes);
  if (need > 0 && reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
    return fail(ATTN_ERR_WORKSPACE, "workspace must be 256-byte aligned");

  attn::DecodeArgs a{};
  a.f16 = dt == ATTN_FP16;
  a.q = q.data; a.k = k_cache.data; a.v = v_cache.data; a.o = o.data;
  a.lse = lse;
  a.seqlens = cache_seqlens;
  a.q_sb = q.stride[0]; a.q_ss = q.stride[1]; a.q_sh = q.stride[2];
  strides3(k_cache, &a.k_sb, &a.k_ss, &a.k_sh);
  strides3(v_cache, &a.v_sb, &a.v_ss, &a.v_sh);
  a.o_sb = o.stride[0]; a.o_ss = o.stride[1]; a.o_sh = o.stride[2];
  a.B = p->B; a.Hq = p->Hq; a.Hkv = p->Hkv; a.D = p->D; a.Smax = p->Sk;
  a.Sq = p->Sq;
  a.causal = p->causal ? 1 : 0;
  a.scale = cm.scale;
  a.softcap = p->softcap;
  if (paged) {
    a.block_table = kv->block_table;
    a.max_blocks = kv->max_blocks;
    a.page_size = kv->page_size;
    a.num_pages = kv->num_pages;
    a.k_pg = k_cache.stride[0];
    a.v_pg = v_cache.stride[0];
  }
  if (remap) {
    a.batch_idx = kv->cache_batch_idx;
    a.cache_batch = kv->cache_batch;
  }
  if (append) {
    a.len_add = kv->s_new;
    a.k_new = kv->k_new.data;
    a.v_new = kv->v_new.data;
    strides3(kv->k_new, &a.kn_sb, &a.kn_ss, &a.kn_sh);
    strides3(kv->v_new, &a.vn_sb, &a.vn_ss, &a.vn_sh);
  }
  a.parts = attn::decode_parts(num_splits);
  a.rows_job = attn::decode_job_rows(p->Hq, p->Hkv, p->Sq);
  a.nhg = attn::decode_head_groups(p->Hq, p->Hkv, p->Sq);
  const attn::DecodeWorkspace wl = attn::decode_workspace(p->B, p->Hq, p->Hkv, p->Sq, p->D, a.parts);
  char* wsb = static_cast<char*>(workspace);
  a.status = status != nullptr ? status : reinterpret_cast<uint32_t*>(wsb + wl.status_off);
  a.spin_limit = attn::spin_limit();
  a.part_o = reinterpret_cast<uint16_t*>(wsb + wl.o_off);
  a.part_lse = reinterpret_cast<float*>(wsb + wl.lse_off);
  a.job_seg = reinterpret_cast<int32_t*>(wsb + wl.seg_off);
  return hip_status(attn::launch_decode_bf16(a, static_cast<hipStream_t>(stream)), "attn_decode launch");
}

attn_status attn_decode(const attn_params* p, attn_tensor q, attn_tensor k_cache,
                        attn_tensor v_cache, const int32_t* cache_seqlens, int32_t num_splits,
                        attn_tensor o, float* lse, void* workspace, size_t workspace_bytes,
                        void* stream) {
  return decode_impl(p, q, k_cache, v_cache, cache_seqlens, nullptr, num_splits, o, lse, workspace,
                     workspace_bytes, stream);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Decode without allocation or caller workspace (attn_decode_noalloc).  Its
// scratch is this file-scope device array: each GPU the library runs on
// holds one copy for the life of the process.  In host code `scratch` names
// a host-side stand-in, not the device copy, so its device address is looked
// up once per device with hipGetSymbolAddress and only that address is
// handed to kernels.
namespace {

constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;  // 64 MiB per GPU
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// The calling thread's current device's copy of `scratch` (looked up on
// the first call on that device).
attn_status scratch_for_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(ATTN_ERR_UNSUPPORTED, "device %d: at most %d devices are supported", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(scratch)");
    if (ptr == nullptr) return fail(ATTN_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return ATTN_OK;
}

}  // namespace

extern "C" {

size_t attn_decode_noalloc_max_bytes(void) { return kNoAllocScratchBytes; }

attn_status attn_decode_noalloc(const attn_params* p, attn_tensor q, attn_tensor k_cache,
                                attn_tensor v_cache, const int32_t* cache_seqlens,
                                int32_t num_splits, attn_tensor o, float* lse, uint32_t* status,
                                void* stream) {
  g_err[0] = 0;
  void* ws = nullptr;
  attn_status st = scratch_for_current_device(&ws);
  if (st != ATTN_OK) return st;
  return decode_impl(p, q, k_cache, v_cache, cache_seqlens, nullptr, num_splits, o, lse, ws,
                     kNoAllocScratchBytes, stream, status, "attn_decode_noalloc's device scratch");
}

attn_status attn_decode_kvcache(const attn_params* p, attn_tensor q, attn_tensor k_cache,
                                attn_tensor v_cache, const int32_t* cache_seqlens,
                                const attn_kvcache* kv, int32_t num_splits, attn_tensor o,
                                float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  return decode_impl(p, q, k_cache, v_cache, cache_seqlens, kv, num_splits, o, lse, workspace,
                     workspace_bytes, stream);
}

size_t attn_block_mask_bytes(int32_t B, int32_t Sq, int32_t Sk, int32_t block_m, int32_t block_n) {
  if (B <= 0 || Sq <= 0 || Sk <= 0 || block_m <= 0 || block_n <= 0) return 0;
  const size_t nQ = (Sq + block_m - 1) / block_m, nK = (Sk + block_n - 1) / block_n;
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  size_t total = up(B * nQ * nK);               // cls
  total += 2 * (up(B * nQ * 4) + up(B * nQ * nK * 4));  // kv lists
  total += 2 * (up(B * nK * 4) + up(B * nK * nQ * 4));  // q lists
  return total;
}

attn_status block_mask_build(const attn_mask_desc* m, int32_t B, int32_t Sq, int32_t Sk,
                             int32_t block_m, int32_t block_n, void* buffer, size_t buffer_bytes,
                             attn_block_mask* out, void* stream) {
  g_err[0] = 0;
  if (m == nullptr || out == nullptr) return fail(ATTN_ERR_INVALID_ARG, "NULL mask descriptor or output");
  if (B <= 0 || Sq <= 0 || Sk <= 0 || block_m <= 0 || block_n <= 0)
    return fail(ATTN_ERR_INVALID_ARG, "sizes must be positive (B=%d Sq=%d Sk=%d block %dx%d)", B, Sq,
                Sk, block_m, block_n);
  if (m->window_left < -1 || m->window_right < -1)
    return fail(ATTN_ERR_INVALID_ARG, "window sides must be >= -1");
  if ((m->doc_q == nullptr) != (m->doc_k == nullptr))
    return fail(ATTN_ERR_INVALID_ARG, "give both doc_q and doc_k or neither");
  if (m->doc_q != nullptr && (block_m > attn::block_mask_max_block() || block_n > attn::block_mask_max_block()))
    return fail(ATTN_ERR_UNSUPPORTED, "with document ids the block size is at most %d (got %dx%d)",
                attn::block_mask_max_block(), block_m, block_n);
  const size_t need = attn_block_mask_bytes(B, Sq, Sk, block_m, block_n);
  if (buffer == nullptr || buffer_bytes < need)
    return fail(ATTN_ERR_WORKSPACE, "block mask needs %zu bytes, got %zu", need, buffer_bytes);
  if (reinterpret_cast<uintptr_t>(buffer) % 256 != 0)
    return fail(ATTN_ERR_WORKSPACE, "block mask buffer must be 256-byte aligned");
  const int nQ = (Sq + block_m - 1) / block_m, nK = (Sk + block_n - 1) / block_n;
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  char* p = static_cast<char*>(buffer);
  auto take = [&](size_t bytes) { char* r = p; p += up(bytes); return r; };
  attn_block_mask r{};
  r.B = B; r.Sq = Sq; r.Sk = Sk; r.block_m = block_m; r.block_n = block_n; r.nQ = nQ; r.nK = nK;
  r.desc = *m;
  r.cls = reinterpret_cast<uint8_t*>(take((size_t)B * nQ * nK));
  r.kv_num_partial = reinterpret_cast<int32_t*>(take((size_t)B * nQ * 4));
  r.kv_idx_partial = reinterpret_cast<int32_t*>(take((size_t)B * nQ * nK * 4));
  r.kv_num_full = reinterpret_cast<int32_t*>(take((size_t)B * nQ * 4));
  r.kv_idx_full = reinterpret_cast<int32_t*>(take((size_t)B * nQ * nK * 4));
  r.q_num_partial = reinterpret_cast<int32_t*>(take((size_t)B * nK * 4));
  r.q_idx_partial = reinterpret_cast<int32_t*>(take((size_t)B * nK * nQ * 4));
  r.q_num_full = reinterpret_cast<int32_t*>(take((size_t)B * nK * 4));
  r.q_idx_full = reinterpret_cast<int32_t*>(take((size_t)B * nK * nQ * 4));

  attn::BlockMaskArgs a{};
  a.B = B; a.Sq = Sq; a.Sk = Sk; a.bm = block_m; a.bn = block_n; a.nQ = nQ; a.nK = nK;
  a.mask.causal = m->causal;
  a.mask.wl = window_side(m->window_left, Sq, Sk);
  a.mask.wr = window_side(m->window_right, Sq, Sk);
  a.mask.doc_q = m->doc_q;
  a.mask.doc_k = m->doc_k;
  a.cls = r.cls;
  a.kv_num_partial = r.kv_num_partial; a.kv_idx_partial = r.kv_idx_partial;
  a.kv_num_full = r.kv_num_full; a.kv_idx_full = r.kv_idx_full;
  a.q_num_partial = r.q_num_partial; a.q_idx_partial = r.q_idx_partial;
  a.q_num_full = r.q_num_full; a.q_idx_full = r.q_idx_full;
  attn_status st = hip_status(attn::launch_block_mask(a, static_cast<hipStream_t>(stream)),
                              "block_mask_build launch");
  if (st == ATTN_OK) *out = r;
  return st;
}

}  // extern "C"
