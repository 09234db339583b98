"""Thin ctypes binding of the C-ABI attention library (libattn.so).

Argument marshalling only: torch tensors provide device memory and the
current stream; every step of the computation runs in the library's HIP
kernels.  Importing this module loads the library and raises ImportError
when it has not been built (there is no fallback path).

Function names mirror include/attn.h: attn_fwd, attn_bwd, attn_decode,
block_mask_build.  Tensors use the logical layout [B, S, H, D] of
flash_attn_func (q [B, Sq, Hq, D], k / v [B, Sk, Hkv, D]); any strides
with a unit head-dim stride and 16-byte aligned rows are passed through
without copies.
"""

import ctypes
import math
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libattn.so")
if not os.path.exists(_LIB_PATH):
    raise ImportError(
        "libattn.so is not built; run `python -m exact_attention_10_amd.build` "
        "(or __graft_entry__.build()) first")
_lib = ctypes.CDLL(_LIB_PATH)

ATTN_OK = 0
ATTN_BF16 = 0
ATTN_FP32 = 1
ATTN_FP16 = 2
STATUS = {0: "ATTN_OK", 1: "ATTN_ERR_INVALID_ARG", 2: "ATTN_ERR_UNSUPPORTED",
          3: "ATTN_ERR_WORKSPACE", 4: "ATTN_ERR_HIP"}


class AttnError(RuntimeError):
    def __init__(self, status, message):
        super().__init__("%s: %s" % (STATUS.get(status, status), message))
        self.status = status


class attn_tensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32),
                ("stride", ctypes.c_int64 * 4)]


class attn_mask_desc(ctypes.Structure):
    _fields_ = [("causal", ctypes.c_int32), ("window_left", ctypes.c_int32),
                ("window_right", ctypes.c_int32), ("doc_q", ctypes.c_void_p),
                ("doc_k", ctypes.c_void_p)]


class attn_block_mask(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("Sq", ctypes.c_int32), ("Sk", ctypes.c_int32),
                ("block_m", ctypes.c_int32), ("block_n", ctypes.c_int32),
                ("nQ", ctypes.c_int32), ("nK", ctypes.c_int32),
                ("desc", attn_mask_desc),
                ("cls", ctypes.c_void_p),
                ("kv_num_partial", ctypes.c_void_p), ("kv_idx_partial", ctypes.c_void_p),
                ("kv_num_full", ctypes.c_void_p), ("kv_idx_full", ctypes.c_void_p),
                ("q_num_partial", ctypes.c_void_p), ("q_idx_partial", ctypes.c_void_p),
                ("q_num_full", ctypes.c_void_p), ("q_idx_full", ctypes.c_void_p)]


class attn_params(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("Sq", ctypes.c_int32), ("Sk", ctypes.c_int32),
                ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32), ("D", ctypes.c_int32),
                ("softmax_scale", ctypes.c_float), ("causal", ctypes.c_int32),
                ("window_left", ctypes.c_int32), ("window_right", ctypes.c_int32),
                ("alibi_slopes", ctypes.c_void_p), ("alibi_batch_stride", ctypes.c_int64),
                ("softcap", ctypes.c_float),
                ("block_mask", ctypes.POINTER(attn_block_mask))]


_P = ctypes.POINTER
_lib.attn_status_string.restype = ctypes.c_char_p
_lib.attn_status_string.argtypes = [ctypes.c_int]
_lib.attn_last_error.restype = ctypes.c_char_p
_lib.attn_last_error.argtypes = []
_lib.attn_fwd.restype = ctypes.c_int
_lib.attn_fwd.argtypes = [_P(attn_params), attn_tensor, attn_tensor, attn_tensor, attn_tensor,
                          ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                          ctypes.c_void_p]
_lib.attn_fwd_tile_shape.restype = ctypes.c_int
_lib.attn_fwd_tile_shape.argtypes = [_P(attn_params), ctypes.c_int32, _P(ctypes.c_int32),
                                     _P(ctypes.c_int32)]
_lib.attn_bwd.restype = ctypes.c_int
_lib.attn_bwd.argtypes = [_P(attn_params), attn_tensor, attn_tensor, attn_tensor, attn_tensor,
                          attn_tensor, ctypes.c_void_p, attn_tensor, attn_tensor, attn_tensor,
                          ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
_lib.attn_bwd_stage.restype = ctypes.c_int
_lib.attn_bwd_stage.argtypes = [_P(attn_params), attn_tensor, attn_tensor, attn_tensor,
                                attn_tensor, attn_tensor, ctypes.c_void_p, attn_tensor,
                                attn_tensor, attn_tensor, ctypes.c_int32, ctypes.c_void_p,
                                ctypes.c_size_t, ctypes.c_int32, ctypes.c_void_p]
_lib.attn_fwd_workspace_size.restype = ctypes.c_size_t
_lib.attn_fwd_workspace_size.argtypes = [_P(attn_params)]
_lib.attn_bwd_workspace_size.restype = ctypes.c_size_t
_lib.attn_bwd_workspace_size.argtypes = [_P(attn_params)]
_lib.attn_decode.restype = ctypes.c_int
_lib.attn_decode.argtypes = [_P(attn_params), attn_tensor, attn_tensor, attn_tensor,
                             ctypes.c_void_p, ctypes.c_int32, attn_tensor, ctypes.c_void_p,
                             ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]


class attn_kvcache(ctypes.Structure):
    _fields_ = [("block_table", ctypes.c_void_p), ("max_blocks", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("num_pages", ctypes.c_int32),
                ("cache_batch_idx", ctypes.c_void_p), ("cache_batch", ctypes.c_int32),
                ("k_new", attn_tensor), ("v_new", attn_tensor), ("s_new", ctypes.c_int32)]


_lib.attn_decode_kvcache.restype = ctypes.c_int
_lib.attn_decode_kvcache.argtypes = [_P(attn_params), attn_tensor, attn_tensor, attn_tensor,
                                     ctypes.c_void_p, _P(attn_kvcache), ctypes.c_int32,
                                     attn_tensor, ctypes.c_void_p, ctypes.c_void_p,
                                     ctypes.c_size_t, ctypes.c_void_p]
_lib.attn_decode_workspace_size.restype = ctypes.c_size_t
_lib.attn_decode_workspace_size.argtypes = [_P(attn_params), ctypes.c_int32]
_lib.attn_block_mask_bytes.restype = ctypes.c_size_t
_lib.attn_block_mask_bytes.argtypes = [ctypes.c_int32] * 5
_lib.block_mask_build.restype = ctypes.c_int
_lib.block_mask_build.argtypes = [_P(attn_mask_desc), ctypes.c_int32, ctypes.c_int32,
                                  ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                  ctypes.c_void_p, ctypes.c_size_t, _P(attn_block_mask),
                                  ctypes.c_void_p]

_lib.attn_decode_noalloc.restype = ctypes.c_int
_lib.attn_decode_noalloc.argtypes = [_P(attn_params), attn_tensor, attn_tensor, attn_tensor,
                                     ctypes.c_void_p, ctypes.c_int32, attn_tensor,
                                     ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
_lib.attn_decode_noalloc_max_bytes.restype = ctypes.c_size_t
_lib.attn_decode_noalloc_max_bytes.argtypes = []
_lib.attn_debug_set_spin_limit.restype = None
_lib.attn_debug_set_spin_limit.argtypes = [ctypes.c_int32]
_lib.attn_set_bwd_gqa_schedule.restype = None
_lib.attn_set_bwd_gqa_schedule.argtypes = [ctypes.c_int32]

EXPORTED = ["attn_status_string", "attn_last_error", "attn_debug_set_spin_limit",
            "attn_set_bwd_gqa_schedule",
            "attn_fwd", "attn_fwd_tile_shape",
            "attn_fwd_workspace_size",
            "attn_bwd", "attn_bwd_stage", "attn_bwd_workspace_size", "attn_decode",
            "attn_decode_kvcache", "attn_decode_workspace_size", "attn_decode_noalloc",
            "attn_decode_noalloc_max_bytes", "attn_block_mask_bytes",
            "block_mask_build"]


def library():
    return _lib


def _check(status):
    if status != ATTN_OK:
        raise AttnError(status, _lib.attn_last_error().decode())


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return ATTN_BF16
    if t.dtype == torch.float16:
        return ATTN_FP16
    if t.dtype == torch.float32:
        return ATTN_FP32
    raise TypeError("unsupported dtype %s (bfloat16, float16 or float32)" % t.dtype)


def _tensor(t):
    if t.dim() != 4:
        raise ValueError("expected a 4-d [B, S, H, D] tensor, got shape %s" % (tuple(t.shape),))
    s = attn_tensor()
    s.data = t.data_ptr()
    s.dtype = _dtype_code(t)
    for i in range(4):
        s.stride[i] = t.stride(i)
    return s


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


class BlockMask:
    """Device block mask built by block_mask_build (keeps its buffer alive)."""

    def __init__(self, struct, buffer, doc_q, doc_k):
        self.struct = struct
        self.buffer = buffer
        self._docs = (doc_q, doc_k)

    def _view(self, field, dtype, shape):
        ptr = getattr(self.struct, field)
        off = ptr - self.buffer.data_ptr()
        n = 1
        for x in shape:
            n *= x
        size = torch.empty((), dtype=dtype).element_size()
        return self.buffer[off:off + n * size].view(dtype).view(*shape)

    def arrays(self):
        s = self.struct
        B, nQ, nK = s.B, s.nQ, s.nK
        return {
            "cls": self._view("cls", torch.uint8, (B, nQ, nK)),
            "kv_num_partial": self._view("kv_num_partial", torch.int32, (B, nQ)),
            "kv_idx_partial": self._view("kv_idx_partial", torch.int32, (B, nQ, nK)),
            "kv_num_full": self._view("kv_num_full", torch.int32, (B, nQ)),
            "kv_idx_full": self._view("kv_idx_full", torch.int32, (B, nQ, nK)),
            "q_num_partial": self._view("q_num_partial", torch.int32, (B, nK)),
            "q_idx_partial": self._view("q_idx_partial", torch.int32, (B, nK, nQ)),
            "q_num_full": self._view("q_num_full", torch.int32, (B, nK)),
            "q_idx_full": self._view("q_idx_full", torch.int32, (B, nK, nQ)),
        }


def block_mask_build(B, Sq, Sk, block_m=128, block_n=128, causal=False, window=(-1, -1),
                     doc_q=None, doc_k=None, device="cuda"):
    """Build a block mask on the device (doc_q / doc_k: int32 [B, S] device tensors)."""
    if (doc_q is None) != (doc_k is None):
        raise ValueError("give both doc_q and doc_k or neither")
    if doc_q is not None:
        _need_shape("doc_q", doc_q, (B, Sq))
        _need_shape("doc_k", doc_k, (B, Sk))
        _need_dtype("doc_q", doc_q, torch.int32)
        _need_dtype("doc_k", doc_k, torch.int32)
        if doc_q.device.type != "cuda" or doc_k.device != doc_q.device:
            raise ValueError("doc_q and doc_k must be on one GPU")
        if torch.device(device) != doc_q.device and torch.device(device).index is not None:
            raise ValueError("doc_q is on %s, the mask is built on %s" % (doc_q.device, device))
        device = doc_q.device
    desc = attn_mask_desc()
    desc.causal = int(bool(causal))
    desc.window_left, desc.window_right = int(window[0]), int(window[1])
    if doc_q is not None:
        doc_q = doc_q.contiguous()
        doc_k = doc_k.contiguous()
    desc.doc_q = None if doc_q is None else doc_q.data_ptr()
    desc.doc_k = None if doc_k is None else doc_k.data_ptr()
    nbytes = _lib.attn_block_mask_bytes(B, Sq, Sk, block_m, block_n)
    buf = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
    out = attn_block_mask()
    _check(_lib.block_mask_build(ctypes.byref(desc), B, Sq, Sk, block_m, block_n,
                                 ctypes.c_void_p(buf.data_ptr()), nbytes, ctypes.byref(out),
                                 _stream()))
    return BlockMask(out, buf, doc_q, doc_k)


def _shape_of(t):
    return tuple(int(x) for x in t.shape)


def _need_shape(name, t, shape):
    if _shape_of(t) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), _shape_of(t)))


def _need_dtype(name, t, dtype):
    if t.dtype != dtype:
        raise ValueError("%s must be %s, got %s" % (name, dtype, t.dtype))


def _need_contig(name, t):
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _need_device(q, **tensors):
    """Every tensor the library reads or writes lives on q's GPU: the C ABI
    takes raw device pointers, so a host tensor or one on another device
    would reach a kernel as an invalid address."""
    if q.device.type != "cuda":
        raise ValueError("q must be a GPU tensor (got device %s)" % q.device)
    for name, t in tensors.items():
        if t is not None and t.device != q.device:
            raise ValueError("%s is on %s, q on %s: every tensor must be on q's device"
                             % (name, t.device, q.device))


def _check_qkv(q, k, v):
    """q [B, Sq, Hq, D], k and v [B, Sk, Hkv, D] of one dtype."""
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.dim() != 4:
            raise ValueError("%s must be a 4-d [B, S, H, D] tensor, got shape %s"
                             % (name, _shape_of(t)))
    B, _, _, D = q.shape
    if k.shape[0] != B or k.shape[3] != D:
        raise ValueError("k must be [B=%d, Sk, Hkv, D=%d], got %s" % (B, D, _shape_of(k)))
    _need_shape("v", v, k.shape)
    _need_dtype("k", k, q.dtype)
    _need_dtype("v", v, q.dtype)


def _check_like(name, t, ref):
    if t is not None:
        _need_shape(name, t, ref.shape)
        _need_dtype(name, t, ref.dtype)


def _check_lse(lse, B, Hq, Sq):
    if lse is not None:
        _need_shape("lse", lse, (B, Hq, Sq))
        _need_dtype("lse", lse, torch.float32)
        _need_contig("lse", lse)


def _check_alibi(alibi_slopes, B, Hq):
    if alibi_slopes is None:
        return
    _need_dtype("alibi_slopes", alibi_slopes, torch.float32)
    _need_contig("alibi_slopes", alibi_slopes)
    if _shape_of(alibi_slopes) not in ((Hq,), (B, Hq)):
        raise ValueError("alibi_slopes must be (Hq,) = (%d,) or (B, Hq) = (%d, %d), got %s"
                         % (Hq, B, Hq, _shape_of(alibi_slopes)))


def _params(q, k, D, softmax_scale, causal, window, alibi_slopes, softcap, block_mask):
    p = attn_params()
    p.B, p.Sq, p.Hq = q.shape[0], q.shape[1], q.shape[2]
    p.Sk, p.Hkv = k.shape[1], k.shape[2]
    p.D = D
    p.softmax_scale = math.nan if softmax_scale is None else float(softmax_scale)
    p.causal = int(bool(causal))
    p.window_left, p.window_right = int(window[0]), int(window[1])
    if alibi_slopes is not None:
        _check_alibi(alibi_slopes, p.B, p.Hq)
        p.alibi_slopes = alibi_slopes.data_ptr()
        p.alibi_batch_stride = 0 if alibi_slopes.dim() == 1 else alibi_slopes.shape[-1]
    else:
        p.alibi_slopes = None
        p.alibi_batch_stride = 0
    p.softcap = float(softcap)
    p.block_mask = ctypes.pointer(block_mask.struct) if block_mask is not None else None
    return p


def tile_shape(q, k, block_mask=None, causal=False):
    """(rows, keys) of the forward's tiles for this problem: the tile trace
    has ceil(Sq / rows) x ceil(Sk / keys) entries per (batch, head)."""
    p = _params(q, k, q.shape[3], None, causal, (-1, -1), None, 0.0, block_mask)
    bm, bn = ctypes.c_int32(), ctypes.c_int32()
    _check(_lib.attn_fwd_tile_shape(ctypes.byref(p), _dtype_code(q), ctypes.byref(bm),
                                    ctypes.byref(bn)))
    return bm.value, bn.value


def attn_fwd(q, k, v, softmax_scale=None, causal=False, window=(-1, -1), alibi_slopes=None,
             softcap=0.0, block_mask=None, out=None, lse=None, tile_trace=None):
    """Forward attention.  Returns (out [B, Sq, Hq, D], lse fp32 [B, Hq, Sq])."""
    _check_qkv(q, k, v)
    B, Sq, Hq, D = q.shape
    _check_like("out", out, q)
    _check_lse(lse, B, Hq, Sq)
    _check_alibi(alibi_slopes, B, Hq)
    if tile_trace is not None:
        _need_dtype("tile_trace", tile_trace, torch.uint8)
        _need_contig("tile_trace", tile_trace)
        bm, bn = tile_shape(q, k, block_mask, causal)
        n = B * Hq * (-(-Sq // bm)) * (-(-k.shape[1] // bn))
        if tile_trace.numel() != n:
            raise ValueError("tile_trace must hold B*Hq*nQt*nKt = %d entries, got %d"
                             % (n, tile_trace.numel()))
    _need_device(q, k=k, v=v, out=out, lse=lse, tile_trace=tile_trace,
                 alibi_slopes=alibi_slopes,
                 block_mask=None if block_mask is None else block_mask.buffer)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device)
    p = _params(q, k, D, softmax_scale, causal, window, alibi_slopes, softcap, block_mask)
    _check(_lib.attn_fwd(ctypes.byref(p), _tensor(q), _tensor(k), _tensor(v), _tensor(out),
                         _ptr(lse), _ptr(tile_trace), None, 0, _stream()))
    return out, lse


def attn_bwd(q, k, v, out, dout, lse, softmax_scale=None, causal=False, window=(-1, -1),
             alibi_slopes=None, softcap=0.0, deterministic=True, dq=None, dk=None, dv=None,
             workspace=None, block_mask=None):
    """Backward attention from the saved LSE.  Returns (dq, dk, dv)."""
    _check_qkv(q, k, v)
    B, Sq, Hq, D = q.shape
    _check_like("out", out, q)
    _check_like("dout", dout, q)
    if lse is None:
        raise ValueError("lse (the forward's log-sum-exp) is required")
    _check_lse(lse, B, Hq, Sq)
    _check_alibi(alibi_slopes, B, Hq)
    _check_like("dq", dq, q)
    _check_like("dk", dk, k)
    _check_like("dv", dv, v)
    if workspace is not None:
        _need_dtype("workspace", workspace, torch.uint8)
    _need_device(q, k=k, v=v, out=out, dout=dout, lse=lse, dq=dq, dk=dk, dv=dv,
                 workspace=workspace, alibi_slopes=alibi_slopes,
                 block_mask=None if block_mask is None else block_mask.buffer)
    p = _params(q, k, D, softmax_scale, causal, window, alibi_slopes, softcap, block_mask)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    need = _lib.attn_bwd_workspace_size(ctypes.byref(p))
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    _check(_lib.attn_bwd(ctypes.byref(p), _tensor(q), _tensor(k), _tensor(v), _tensor(out),
                         _tensor(dout), _ptr(lse), _tensor(dq), _tensor(dk), _tensor(dv),
                         1 if deterministic else 0, _ptr(workspace), workspace.numel(),
                         _stream()))
    return dq, dk, dv


def _unpack(x, n, name):
    if x.dim() != 5 or x.shape[2] != n:
        raise ValueError("%s must be [B, S, %d, H, D], got shape %s" % (name, n, tuple(x.shape)))
    return [x[:, :, i] for i in range(n)]


def attn_fwd_qkvpacked(qkv, softmax_scale=None, causal=False, window=(-1, -1), alibi_slopes=None,
                       softcap=0.0, out=None, lse=None):
    """Forward on a packed qkv [B, S, 3, H, D] ([FA] flash_attn_qkvpacked_func):
    q, k, v are strided views of it, no copy.  Returns (out, lse)."""
    q, k, v = _unpack(qkv, 3, "qkv")
    return attn_fwd(q, k, v, softmax_scale, causal, window, alibi_slopes, softcap, out=out, lse=lse)


def attn_bwd_qkvpacked(qkv, out, dout, lse, softmax_scale=None, causal=False, window=(-1, -1),
                       alibi_slopes=None, softcap=0.0, deterministic=True, dqkv=None, workspace=None):
    """Backward of attn_fwd_qkvpacked with the gradient in the packed layout:
    dq, dk, dv are written straight into views of one dqkv [B, S, 3, H, D]."""
    q, k, v = _unpack(qkv, 3, "qkv")
    dqkv = torch.empty_like(qkv) if dqkv is None else dqkv
    dq, dk, dv = _unpack(dqkv, 3, "dqkv")
    attn_bwd(q, k, v, out, dout, lse, softmax_scale, causal, window, alibi_slopes, softcap,
             deterministic, dq=dq, dk=dk, dv=dv, workspace=workspace)
    return dqkv


def attn_fwd_kvpacked(q, kv, softmax_scale=None, causal=False, window=(-1, -1), alibi_slopes=None,
                      softcap=0.0, out=None, lse=None):
    """Forward with a packed kv [B, Sk, 2, Hkv, D] ([FA] flash_attn_kvpacked_func)."""
    k, v = _unpack(kv, 2, "kv")
    return attn_fwd(q, k, v, softmax_scale, causal, window, alibi_slopes, softcap, out=out, lse=lse)


def attn_bwd_kvpacked(q, kv, out, dout, lse, softmax_scale=None, causal=False, window=(-1, -1),
                      alibi_slopes=None, softcap=0.0, deterministic=True, dq=None, dkv=None,
                      workspace=None):
    """Backward of attn_fwd_kvpacked; returns (dq, dkv) with dkv [B, Sk, 2, Hkv, D]."""
    k, v = _unpack(kv, 2, "kv")
    dkv = torch.empty_like(kv) if dkv is None else dkv
    dk, dv = _unpack(dkv, 2, "dkv")
    dq = torch.empty_like(q) if dq is None else dq
    attn_bwd(q, k, v, out, dout, lse, softmax_scale, causal, window, alibi_slopes, softcap,
             deterministic, dq=dq, dk=dk, dv=dv, workspace=workspace)
    return dq, dkv


def attn_bwd_stage(stage, q, k, v, out, dout, lse, dq, dk, dv, workspace, softmax_scale=None,
                   causal=False, window=(-1, -1), alibi_slopes=None, softcap=0.0, block_mask=None,
                   deterministic=True):
    """Enqueue one stage of attn_bwd (deterministic: 0 dQ with Delta, 1 dK/dV,
    2 group sum, 3 nothing; see attn.h); stages 0..3 in order with one
    workspace equal attn_bwd."""
    _check_qkv(q, k, v)
    B, Sq, Hq, D = q.shape
    for name, t, ref in (("out", out, q), ("dout", dout, q), ("dq", dq, q), ("dk", dk, k),
                         ("dv", dv, v)):
        _check_like(name, t, ref)
    _check_lse(lse, B, Hq, Sq)
    _need_dtype("workspace", workspace, torch.uint8)
    _need_device(q, k=k, v=v, out=out, dout=dout, lse=lse, dq=dq, dk=dk, dv=dv,
                 workspace=workspace, alibi_slopes=alibi_slopes,
                 block_mask=None if block_mask is None else block_mask.buffer)
    p = _params(q, k, D, softmax_scale, causal, window, alibi_slopes, softcap, block_mask)
    _check(_lib.attn_bwd_stage(ctypes.byref(p), _tensor(q), _tensor(k), _tensor(v), _tensor(out),
                               _tensor(dout), _ptr(lse), _tensor(dq), _tensor(dk), _tensor(dv),
                               1 if deterministic else 0, _ptr(workspace), workspace.numel(),
                               int(stage), _stream()))


def attn_decode(q, k_cache, v_cache, cache_seqlens, softmax_scale=None, softcap=0.0,
                num_splits=0, out=None, lse=None, workspace=None, block_table=None,
                cache_batch_idx=None, k_new=None, v_new=None, causal=False):
    """Decode over a KV cache.  q [B, Sq, Hq, D] (the last Sq positions of
    each sequence; causal: bottom-right aligned); caches [B, Smax, Hkv, D]
    (paged: [num_pages, page_size, Hkv, D] with block_table int32
    [B, max_blocks]); cache_seqlens int32 [B] on the device; optional
    cache_batch_idx int32 [B] (contiguous caches) and k_new / v_new
    [B, s_new, Hkv, D] appended in place at rows [L_b, L_b + s_new).
    Returns (out, lse [B, Hq, Sq])."""
    if q.dim() != 4 or k_cache.dim() != 4:
        raise ValueError("q and the caches must be 4-d tensors")
    B, Sq, Hq, D = q.shape
    if k_cache.shape[3] != D:
        raise ValueError("k_cache head dim %d differs from q's %d" % (k_cache.shape[3], D))
    _check_like("v_cache", v_cache, k_cache)
    _need_dtype("k_cache", k_cache, q.dtype)
    Hkv = k_cache.shape[2]
    if block_table is not None:
        if block_table.dtype != torch.int32 or block_table.dim() != 2:
            raise ValueError("block_table must be a 2-d int32 tensor")
        if block_table.shape[0] != B:
            raise ValueError("block_table must have B = %d rows, got %d" % (B, block_table.shape[0]))
        _need_contig("block_table", block_table)
    elif cache_batch_idx is None and k_cache.shape[0] != B:
        raise ValueError("k_cache must have B = %d batch rows, got %d" % (B, k_cache.shape[0]))
    if cache_batch_idx is not None:
        _need_shape("cache_batch_idx", cache_batch_idx, (B,))
        _need_dtype("cache_batch_idx", cache_batch_idx, torch.int32)
        _need_contig("cache_batch_idx", cache_batch_idx)
    _need_shape("cache_seqlens", cache_seqlens, (B,))
    _need_dtype("cache_seqlens", cache_seqlens, torch.int32)
    _need_contig("cache_seqlens", cache_seqlens)
    if (k_new is None) != (v_new is None):
        raise ValueError("k_new and v_new must be given together")
    if k_new is not None:
        if k_new.dim() != 4 or k_new.shape[0] != B or tuple(k_new.shape[2:]) != (Hkv, D):
            raise ValueError("k_new must be [B=%d, s_new, Hkv=%d, D=%d], got %s"
                             % (B, Hkv, D, _shape_of(k_new)))
        _check_like("v_new", v_new, k_new)
        _need_dtype("k_new", k_new, q.dtype)
    _check_like("out", out, q)
    _check_lse(lse, B, Hq, Sq)
    if workspace is not None:
        _need_dtype("workspace", workspace, torch.uint8)
    _need_device(q, k_cache=k_cache, v_cache=v_cache, cache_seqlens=cache_seqlens,
                 block_table=block_table, cache_batch_idx=cache_batch_idx, k_new=k_new,
                 v_new=v_new, out=out, lse=lse, workspace=workspace)
    p = _params(q, k_cache, D, softmax_scale, causal, (-1, -1), None, softcap, None)
    kv = None
    if block_table is not None or cache_batch_idx is not None or k_new is not None:
        kv = attn_kvcache()
        if block_table is not None:
            kv.block_table = block_table.data_ptr()
            kv.max_blocks = block_table.shape[1]
            kv.page_size = k_cache.shape[1]
            kv.num_pages = k_cache.shape[0]
            p.Sk = block_table.shape[1] * k_cache.shape[1]
        if cache_batch_idx is not None:
            kv.cache_batch_idx = cache_batch_idx.data_ptr()
            kv.cache_batch = k_cache.shape[0]
        if k_new is not None:
            kv.k_new, kv.v_new = _tensor(k_new), _tensor(v_new)
            kv.s_new = k_new.shape[1]
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device)
    need = _lib.attn_decode_workspace_size(ctypes.byref(p), int(num_splits))
    if workspace is None or workspace.numel() < need:
        # zeroed: its first word is the sticky status word (decode_status)
        workspace = torch.zeros(max(need, 256), dtype=torch.uint8, device=q.device)
    if kv is None:
        _check(_lib.attn_decode(ctypes.byref(p), _tensor(q), _tensor(k_cache), _tensor(v_cache),
                                _ptr(cache_seqlens), int(num_splits), _tensor(out), _ptr(lse),
                                _ptr(workspace), workspace.numel(), _stream()))
    else:
        _check(_lib.attn_decode_kvcache(ctypes.byref(p), _tensor(q), _tensor(k_cache),
                                        _tensor(v_cache), _ptr(cache_seqlens), ctypes.byref(kv),
                                        int(num_splits), _tensor(out), _ptr(lse), _ptr(workspace),
                                        workspace.numel(), _stream()))
    return out, lse


def attn_decode_noalloc(q, k_cache, v_cache, cache_seqlens, out, lse, softmax_scale=None,
                        softcap=0.0, num_splits=0, causal=False, status=None):
    """attn_decode without a workspace (the library's per-device scratch):
    out and lse are caller-provided, nothing is allocated.  status: None or
    a device int32 tensor of one element receiving the sticky status bits."""
    if q.dim() != 4 or k_cache.dim() != 4:
        raise ValueError("q and the caches must be 4-d tensors")
    B, Sq, Hq, D = q.shape
    if k_cache.shape[0] != B or k_cache.shape[3] != D:
        raise ValueError("k_cache must be [B=%d, Smax, Hkv, D=%d], got %s" % (B, D, _shape_of(k_cache)))
    _check_like("v_cache", v_cache, k_cache)
    _need_dtype("k_cache", k_cache, q.dtype)
    _need_shape("cache_seqlens", cache_seqlens, (B,))
    _need_dtype("cache_seqlens", cache_seqlens, torch.int32)
    _need_contig("cache_seqlens", cache_seqlens)
    if out is None or lse is None:
        raise ValueError("attn_decode_noalloc writes into caller-provided out and lse")
    _check_like("out", out, q)
    _check_lse(lse, B, Hq, Sq)
    if status is not None:
        if status.numel() != 1 or status.dtype != torch.int32:
            raise ValueError("status must be a one-element int32 tensor")
    _need_device(q, k_cache=k_cache, v_cache=v_cache, cache_seqlens=cache_seqlens, out=out,
                 lse=lse, status=status)
    p = _params(q, k_cache, D, softmax_scale, causal, (-1, -1), None, softcap, None)
    _check(_lib.attn_decode_noalloc(ctypes.byref(p), _tensor(q), _tensor(k_cache), _tensor(v_cache),
                                    _ptr(cache_seqlens), int(num_splits), _tensor(out), _ptr(lse),
                                    _ptr(status), _stream()))
    return out, lse


def decode_noalloc_max_bytes():
    return _lib.attn_decode_noalloc_max_bytes()


def decode_status(workspace):
    """The sticky status word at the start of a decode workspace (reads the
    device; call after the decode): bit 1 = a cache length was out of range
    and clamped, bit 2 = an in-kernel wait reached its bound."""
    return int(workspace[:4].view(torch.int32).item()) & 0xFFFFFFFF


def set_spin_limit(limit):
    """Testing hook (attn_debug_set_spin_limit): bound of the in-kernel
    waits for later launches; a negative value restores the default."""
    _lib.attn_debug_set_spin_limit(int(limit))


def set_bwd_gqa_schedule(mode):
    """attn_set_bwd_gqa_schedule: schedule of the dK/dV pass for grouped-query
    heads in later launches (0 automatic, 1 per-head partials and a group
    sum, 2 the group's heads looped inside each workgroup)."""
    _lib.attn_set_bwd_gqa_schedule(int(mode))


def decode_workspace_size(q, k_cache, num_splits=0, softcap=0.0, causal=False):
    p = _params(q, k_cache, q.shape[3], None, causal, (-1, -1), None, softcap, None)
    return _lib.attn_decode_workspace_size(ctypes.byref(p), int(num_splits))


def fwd_workspace_size(q, k):
    p = _params(q, k, q.shape[3], None, False, (-1, -1), None, 0.0, None)
    return _lib.attn_fwd_workspace_size(ctypes.byref(p))


def bwd_workspace_size(q, k):
    p = _params(q, k, q.shape[3], None, False, (-1, -1), None, 0.0, None)
    return _lib.attn_bwd_workspace_size(ctypes.byref(p))
