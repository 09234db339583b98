// Split-K decode over a KV cache, bf16 (gfx950).
//
// flash_attn_with_kvcache ("FlashAttention: Fast and Memory-Efficient Exact
// Attention", "Examples") attends one new query per sequence to the first
// cache_seqlens[b] rows of that sequence's cache.  Here each sequence's
// valid prefix is cut into chunks of `chunk` keys; one workgroup attends all
// query heads of one kv head to one chunk and writes a partial result
// (normalised O_s in fp32 and its log-sum-exp), and a second kernel merges
// the chunks of each sequence with the LSE-weighted combine
//   lse = log sum_s exp(lse_s),   O = sum_s exp(lse_s - lse) O_s
// (the chunk-level form of the online softmax of "Accelerating AI: A Deep
// Dive into Flash Attention", "2. Online Softmax").
//
// With multi-query heads (128 query heads reading one kv head) the query
// heads play the role of query rows: the matrix-core tiles are the same as in
// the forward kernel, S^T = K Q^T with 32 heads per wave, so each K/V byte
// read from HBM feeds 128 heads.

#include "common.h"
#include "internal.h"

namespace attn {
namespace {

constexpr float kNegInf = -__builtin_huge_valf();

template <int D>
struct DecCfg {
  static constexpr int ROWS = 128;         // query heads per workgroup
  static constexpr int BN = 64;            // keys per tile
  static constexpr int NT = 256;
  static constexpr int KS = D + 8;
  static constexpr int VS = D + 32;
  static constexpr int KT = BN * KS;
  static constexpr int VT = BN * VS;
  static constexpr int CPT = BN * D / 8 / NT;
  static constexpr int DSTEPS = D / 16;
  static constexpr int DBLK = D / 32;
};

template <int D, bool kSoftcap>
__global__ __launch_bounds__(256, 2) void decode_split_kernel(DecodeArgs a) {
  using C = DecCfg<D>;
  __shared__ __attribute__((aligned(16))) bf16_t lds_k[2 * C::KT];
  __shared__ __attribute__((aligned(16))) bf16_t lds_v[2 * C::VT];

  const int split = blockIdx.x;
  const int b = blockIdx.z;
  int L = a.seqlens[b];
  L = L < 0 ? 0 : (L > a.Smax ? a.Smax : L);
  const int k_begin = split * a.chunk;
  if (k_begin >= L) return;  // the combine only reads the first ceil(L / chunk) splits
  const int k_end = min(L, k_begin + a.chunk);

  const int G = a.Hq / a.Hkv;
  const int nhb = (G + C::ROWS - 1) / C::ROWS;
  const int g_kv = blockIdx.y / nhb;
  const int hb = blockIdx.y % nhb;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, c = lane & 31;
  const int row = hb * C::ROWS + wave * 32 + c;
  const bool row_ok = row < G;
  const int h = g_kv * G + row;

  const bf16_t* qp = static_cast<const bf16_t*>(a.q) + b * a.q_sb + (int64_t)h * a.q_sh;
  const bf16_t* kp = static_cast<const bf16_t*>(a.k) + b * a.k_sb + g_kv * a.k_sh;
  const bf16_t* vp = static_cast<const bf16_t*>(a.v) + b * a.v_sb + g_kv * a.v_sh;

  const float scale_abs = fabsf(a.scale);
  const uint32_t sign_flip = a.scale < 0.0f ? 0x80008000u : 0u;
  bf16x8 qf[C::DSTEPS];
#pragma unroll
  for (int ds = 0; ds < C::DSTEPS; ++ds) {
    if (row_ok) {
      uint4 raw = *reinterpret_cast<const uint4*>(qp + 16 * ds + 8 * g);
      raw.x ^= sign_flip; raw.y ^= sign_flip; raw.z ^= sign_flip; raw.w ^= sign_flip;
      qf[ds] = __builtin_bit_cast(bf16x8, raw);
    } else {
      uint4 z = make_uint4(0, 0, 0, 0);
      qf[ds] = __builtin_bit_cast(bf16x8, z);
    }
  }
  const float scale_log2 = scale_abs * kLog2e;
  const float cap_k2 = kSoftcap ? 2.0f * kLog2e * scale_abs / a.softcap : 0.0f;
  const float cap_log2 = a.softcap * kLog2e;

  const int t_begin = k_begin / C::BN;
  const int ntiles = (k_end - k_begin + C::BN - 1) / C::BN;

  uint4 kr[C::CPT], vr[C::CPT];
  auto load_regs = [&](int kt) {
#pragma unroll
    for (int u = 0; u < C::CPT; ++u) {
      const int chunk = tid + u * C::NT;
      const int r = chunk / (D / 8);
      const int col = (chunk % (D / 8)) * 8;
      const int key = kt * C::BN + r;
      if (key < k_end) {
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
      const int r = chunk / (D / 8);
      const int col = (chunk % (D / 8)) * 8;
      *reinterpret_cast<uint4*>(lds_k + buf * C::KT + r * C::KS + col) = kr[u];
      *reinterpret_cast<uint4*>(lds_v + buf * C::VT + r * C::VS + col) = vr[u];
    }
  };

  float m_run = kNegInf, l_run = 0.0f;
  f32x16 oacc[C::DBLK];
#pragma unroll
  for (int db = 0; db < C::DBLK; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.0f;

  load_regs(t_begin);
  store_regs(0);
  __syncthreads();

  const int beta = lane >> 4, s16 = lane & 15;
  const int tr_row = 4 * (beta >> 1) + (s16 >> 2);
  const int tr_col = 16 * (beta & 1) + 4 * (s16 & 3);

  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    const int kt = t_begin + t;
    const bool has_next = t + 1 < ntiles;
    if (has_next) load_regs(kt + 1);

    const bf16_t* kb_base = lds_k + buf * C::KT;
    f32x16 sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.0f;
#pragma unroll
    for (int ds = 0; ds < C::DSTEPS; ++ds) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8 ka = *reinterpret_cast<const bf16x8*>(kb_base + (32 * kb + c) * C::KS + 16 * ds + 8 * g);
        sacc[kb] = mfma32(ka, qf[ds], sacc[kb]);
      }
    }
    if (kSoftcap) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float e = fast_exp2(sacc[kb][r] * cap_k2);
          sacc[kb][r] = cap_log2 * (1.0f - 2.0f * fast_rcp(e + 1.0f));
        }
    }
    const int key0 = kt * C::BN + 4 * g;
    if (kt * C::BN + C::BN > k_end) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (key0 + 32 * kb + 8 * (r >> 2) + (r & 3) >= k_end) sacc[kb][r] = kNegInf;
    }

    float mx = kNegInf;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
    mx = fmaxf(mx, wave_xor32(mx));
    const float mx2 = kSoftcap ? mx : mx * scale_log2;
    if (__any(mx2 > m_run + 8.0f)) {
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
    bf16x8 pf[2][2];
    float ls = 0.0f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = kSoftcap ? fast_exp2(sacc[kb][r] - msub)
                                 : fast_exp2(__builtin_fmaf(sacc[kb][r], scale_log2, -msub));
        ls += p;
        pf[kb][r >> 3][r & 7] = static_cast<__bf16>(p);
      }
    l_run += ls;

    const bf16_t* vb_base = lds_v + buf * C::VT;
#pragma unroll
    for (int db = 0; db < C::DBLK; ++db)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const bf16_t* p0 = vb_base + (32 * kb + 16 * ks + tr_row) * C::VS + 32 * db + tr_col;
          const i16x4 lo = lds_read_tr16(p0);
          const i16x4 hi = lds_read_tr16(p0 + 8 * C::VS);
          const bf16x8 va = cat_frag(lo, hi);
          oacc[db] = mfma32(va, pf[kb][ks], oacc[db]);
        }

    if (has_next) store_regs(buf ^ 1);
    __syncthreads();
  }

  const float l_tot = l_run + wave_xor32(l_run);
  if (row_ok) {
    const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
    float* op = a.part_o + (((int64_t)b * a.max_splits + split) * a.Hq + h) * D;
#pragma unroll
    for (int db = 0; db < C::DBLK; ++db)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        float4 v4 = make_float4(oacc[db][4 * rr] * inv, oacc[db][4 * rr + 1] * inv,
                                oacc[db][4 * rr + 2] * inv, oacc[db][4 * rr + 3] * inv);
        *reinterpret_cast<float4*>(op + 32 * db + 8 * rr + 4 * g) = v4;
      }
    if (g == 0)
      a.part_lse[((int64_t)b * a.max_splits + split) * a.Hq + h] =
          l_tot > 0.0f ? (m_run + fast_log2(l_tot)) * kLn2 : kNegInf;
  }
}

// One thread per (head, d): merge the splits of one sequence.
template <int D>
__global__ __launch_bounds__(256) void decode_combine_kernel(DecodeArgs a) {
  constexpr int HPB = 256 / D;  // heads per block
  const int b = blockIdx.y;
  const int h = blockIdx.x * HPB + threadIdx.x / D;
  const int d = threadIdx.x % D;
  if (h >= a.Hq) return;
  int L = a.seqlens[b];
  L = L < 0 ? 0 : (L > a.Smax ? a.Smax : L);
  const int n = (L + a.chunk - 1) / a.chunk;
  const float* pl = a.part_lse + (int64_t)b * a.max_splits * a.Hq + h;
  const float* po = a.part_o + ((int64_t)b * a.max_splits * a.Hq + h) * D + d;
  float m = kNegInf;
  for (int s = 0; s < n; ++s) m = fmaxf(m, pl[(int64_t)s * a.Hq]);
  float tot = 0.0f, acc = 0.0f;
  if (m != kNegInf) {
    for (int s = 0; s < n; ++s) {
      const float ls = pl[(int64_t)s * a.Hq];
      const float w = ls == kNegInf ? 0.0f : fast_exp2((ls - m) * kLog2e);
      tot += w;
      acc = __builtin_fmaf(w, po[(int64_t)s * a.Hq * D], acc);
    }
  }
  bf16_t* op = static_cast<bf16_t*>(a.o) + b * a.o_sb + (int64_t)h * a.o_sh;
  op[d] = f32_to_bf16(tot > 0.0f ? acc / tot : 0.0f);
  if (d == 0) a.lse[(int64_t)b * a.Hq + h] = tot > 0.0f ? m + fast_log2(tot) * kLn2 : kNegInf;
}

template <int D>
hipError_t launch_d(const DecodeArgs& a, hipStream_t s) {
  const int G = a.Hq / a.Hkv;
  const int nhb = (G + DecCfg<D>::ROWS - 1) / DecCfg<D>::ROWS;
  const dim3 grid(a.max_splits, a.Hkv * nhb, a.B);
  if (a.softcap > 0.0f) hipLaunchKernelGGL((decode_split_kernel<D, true>), grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL((decode_split_kernel<D, false>), grid, dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  constexpr int HPB = 256 / D;
  hipLaunchKernelGGL(decode_combine_kernel<D>, dim3((a.Hq + HPB - 1) / HPB, a.B), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

size_t decode_workspace_bytes(int B, int Hq, int D, int max_splits) {
  const size_t o = ((size_t)B * max_splits * Hq * D * sizeof(float) + 255) / 256 * 256;
  const size_t l = ((size_t)B * max_splits * Hq * sizeof(float) + 255) / 256 * 256;
  return o + l;
}

hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t s) {
  if (a.B == 0 || a.max_splits == 0) return hipSuccess;
  if (a.D == 64) return launch_d<64>(a, s);
  return launch_d<128>(a, s);
}

}  // namespace attn
