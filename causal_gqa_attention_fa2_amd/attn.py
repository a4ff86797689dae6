"""Thin Python binding of libattn.so (include/attn.h).

Argument marshalling only: checks dtypes, shapes, devices and contiguity of
torch tensors, passes raw device pointers and the current HIP stream to the
C ABI, and raises ``AttnError`` on a non-OK status. Every step of the
computation runs in the library's HIP kernels; there is no fallback. If the
library has not been built, every call raises.

Names follow the C ABI: ``fwd`` -> attn_fwd, ``bwd`` -> attn_bwd,
``decode_paged`` -> attn_decode_paged.
"""
import ctypes
import math
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libattn.so")

ATTN_OK = 0
STATUS_NAMES = {0: "ATTN_OK", 1: "ATTN_ERR_INVALID_ARG", 2: "ATTN_ERR_UNSUPPORTED",
                3: "ATTN_ERR_WORKSPACE", 4: "ATTN_ERR_HIP"}
EXPORTED = ("attn_fwd", "attn_bwd", "attn_bwd_workspace_bytes", "attn_decode_paged",
            "attn_decode_workspace_bytes", "attn_kv_append", "attn_prefill_paged",
            "attn_rmsnorm_fwd", "attn_rmsnorm_bwd", "attn_rmsnorm_bwd_workspace_bytes",
            "attn_sample", "attn_rope_tables_init", "attn_rope", "attn_kv_append_rope", "attn_bwd_rope",
            "attn_decode_paged_rope", "attn_decode_paged_noalloc",
            "attn_prefill_paged_rope",
            "attn_status_string", "attn_check_cu_seqlens", "attn_check_paged",
            "attn_check_prefill")


class AttnError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn} returned {STATUS_NAMES.get(status, status)}")


class VarlenDims(ctypes.Structure):
    _fields_ = [("n_seqs", ctypes.c_int32), ("total_tokens", ctypes.c_int32),
                ("max_seqlen", ctypes.c_int32), ("h_q", ctypes.c_int32),
                ("h_kv", ctypes.c_int32), ("head_dim", ctypes.c_int32)]


class PagedDims(ctypes.Structure):
    _fields_ = [("n_seqs", ctypes.c_int32), ("h_q", ctypes.c_int32), ("h_kv", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("max_blocks_per_seq", ctypes.c_int32), ("num_blocks", ctypes.c_int32),
                ("max_ctx_len", ctypes.c_int32)]


class PrefillDims(ctypes.Structure):
    _fields_ = [("paged", PagedDims), ("total_q", ctypes.c_int32),
                ("max_q_len", ctypes.c_int32)]


class SampleDims(ctypes.Structure):
    _fields_ = [("n_rows", ctypes.c_int32), ("vocab", ctypes.c_int32)]


class RopeTables(ctypes.Structure):
    _fields_ = [("cos", ctypes.c_void_p), ("sin", ctypes.c_void_p), ("max_pos", ctypes.c_int32)]


class NormDims(ctypes.Structure):
    _fields_ = [("rows", ctypes.c_int32), ("n", ctypes.c_int32)]


_LIB = None
_vp = ctypes.c_void_p


def load_library():
    """Load libattn.so once (after torch, so both share one HIP runtime)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() or "
                           "python -m causal_gqa_attention_fa2_amd.build")
    lib = ctypes.CDLL(LIB_PATH)
    lib.attn_fwd.argtypes = [ctypes.POINTER(VarlenDims), _vp, _vp, _vp, _vp, ctypes.c_float,
                             _vp, _vp, _vp]
    lib.attn_fwd.restype = ctypes.c_int
    lib.attn_bwd_workspace_bytes.argtypes = [ctypes.POINTER(VarlenDims)]
    lib.attn_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.attn_bwd.argtypes = [ctypes.POINTER(VarlenDims), _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                             _vp, _vp, _vp, ctypes.c_float, _vp, ctypes.c_size_t, _vp]
    lib.attn_bwd.restype = ctypes.c_int
    lib.attn_decode_workspace_bytes.argtypes = [ctypes.POINTER(PagedDims)]
    lib.attn_decode_workspace_bytes.restype = ctypes.c_size_t
    lib.attn_decode_paged.argtypes = [ctypes.POINTER(PagedDims), _vp, _vp, _vp, _vp, _vp, _vp,
                                      ctypes.c_float, _vp, ctypes.c_size_t, _vp]
    lib.attn_decode_paged.restype = ctypes.c_int
    lib.attn_decode_paged_noalloc.argtypes = [ctypes.POINTER(PagedDims), _vp, _vp, _vp, _vp,
                                              _vp, _vp, ctypes.c_float, _vp]
    lib.attn_decode_paged_noalloc.restype = ctypes.c_int
    lib.attn_status_string.argtypes = [ctypes.c_int]
    lib.attn_status_string.restype = ctypes.c_char_p
    lib.attn_check_cu_seqlens.argtypes = [ctypes.POINTER(VarlenDims), _vp]
    lib.attn_check_cu_seqlens.restype = ctypes.c_int
    lib.attn_check_paged.argtypes = [ctypes.POINTER(PagedDims), _vp, _vp]
    lib.attn_check_paged.restype = ctypes.c_int
    lib.attn_kv_append.argtypes = [ctypes.POINTER(PrefillDims), _vp, _vp, _vp, _vp, _vp, _vp,
                                   _vp, _vp]
    lib.attn_kv_append.restype = ctypes.c_int
    lib.attn_prefill_paged.argtypes = [ctypes.POINTER(PrefillDims), _vp, _vp, _vp, _vp, _vp,
                                       _vp, _vp, _vp, ctypes.c_float, _vp]
    lib.attn_prefill_paged.restype = ctypes.c_int
    lib.attn_check_prefill.argtypes = [ctypes.POINTER(PrefillDims), _vp, _vp, _vp]
    lib.attn_check_prefill.restype = ctypes.c_int
    lib.attn_rmsnorm_fwd.argtypes = [ctypes.POINTER(NormDims), _vp, _vp, ctypes.c_float, _vp, _vp,
                                     _vp]
    lib.attn_rmsnorm_fwd.restype = ctypes.c_int
    lib.attn_rmsnorm_bwd_workspace_bytes.argtypes = [ctypes.POINTER(NormDims)]
    lib.attn_rmsnorm_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.attn_rmsnorm_bwd.argtypes = [ctypes.POINTER(NormDims), _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                     ctypes.c_size_t, _vp]
    lib.attn_rmsnorm_bwd.restype = ctypes.c_int
    lib.attn_sample.argtypes = [ctypes.POINTER(SampleDims), _vp, _vp, ctypes.c_float,
                                ctypes.c_int32, ctypes.c_float, _vp, _vp]
    lib.attn_sample.restype = ctypes.c_int
    lib.attn_rope_tables_init.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_double, _vp,
                                          _vp, _vp]
    lib.attn_rope_tables_init.restype = ctypes.c_int
    lib.attn_rope.argtypes = [ctypes.POINTER(VarlenDims), _vp, _vp, _vp, _vp, ctypes.c_int32,
                              ctypes.POINTER(RopeTables), ctypes.c_int32, _vp]
    lib.attn_rope.restype = ctypes.c_int
    lib.attn_decode_paged_rope.argtypes = [ctypes.POINTER(PagedDims), _vp, _vp, _vp, _vp, _vp,
                                           ctypes.POINTER(RopeTables), _vp, ctypes.c_float, _vp,
                                           ctypes.c_size_t, _vp]
    lib.attn_decode_paged_rope.restype = ctypes.c_int
    lib.attn_bwd_rope.argtypes = [ctypes.POINTER(VarlenDims), _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                  ctypes.POINTER(RopeTables), _vp, _vp, _vp, ctypes.c_float, _vp,
                                  ctypes.c_size_t, _vp]
    lib.attn_bwd_rope.restype = ctypes.c_int
    lib.attn_kv_append_rope.argtypes = [ctypes.POINTER(PrefillDims), _vp, _vp, _vp, _vp, _vp,
                                        ctypes.POINTER(RopeTables), _vp, _vp, _vp]
    lib.attn_kv_append_rope.restype = ctypes.c_int
    lib.attn_prefill_paged_rope.argtypes = [ctypes.POINTER(PrefillDims), _vp, _vp, _vp, _vp, _vp,
                                            _vp, ctypes.POINTER(RopeTables), _vp, _vp,
                                            ctypes.c_float, _vp]
    lib.attn_prefill_paged_rope.restype = ctypes.c_int
    _LIB = lib
    return lib


def _ptr(t):
    return None if t is None else _vp(t.data_ptr())


def _stream():
    return _vp(torch.cuda.current_stream().cuda_stream)


def _need(t, name, dtype, ndim=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must live on a GPU")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims")


def _check(fn, status):
    if status != ATTN_OK:
        raise AttnError(fn, status)


def debug_validate_enabled():
    """ATTN_DEBUG_VALIDATE=1: before every launch, copy the device index
    arrays to the host (synchronously) and check their contents with the
    library's host validators. Off by default: the library itself never
    reads them on the host."""
    return os.environ.get("ATTN_DEBUG_VALIDATE", "") == "1"


def validate_varlen(dims, cu_seqlens):
    """Raise AttnError unless cu_seqlens (any device) is valid for dims."""
    _check("attn_check_cu_seqlens", check_cu_seqlens_host(dims, cu_seqlens.cpu()))


def validate_paged(dims, block_table, ctx_lens):
    """Raise AttnError unless block_table and ctx_lens (any device) are valid
    for dims."""
    _check("attn_check_paged", check_paged_host(dims, block_table.cpu(), ctx_lens.cpu()))


def varlen_dims(q, k, cu_seqlens, max_seqlen=None):
    T, h_q, d = q.shape
    if max_seqlen is None:  # host copy: synchronises, meant for tests
        cu = cu_seqlens.cpu()
        max_seqlen = int((cu[1:] - cu[:-1]).max()) if cu.numel() > 1 else 0
    return VarlenDims(cu_seqlens.numel() - 1, T, int(max_seqlen), h_q, k.shape[1], d)


def fwd(q, k, v, cu_seqlens, scale=None, o=None, lse=None, max_seqlen=None):
    """attn_fwd: returns (o fp16 [T, h_q, d], lse fp32 [h_q, T])."""
    lib = load_library()
    dev = q.device
    _need(q, "q", torch.float16, 3)
    _need(k, "k", torch.float16, 3, dev)
    _need(v, "v", torch.float16, 3, dev)
    _need(cu_seqlens, "cu_seqlens", torch.int32, 1, dev)
    T, h_q, d = q.shape
    if k.shape != v.shape or k.shape[0] != T or k.shape[2] != d:
        raise ValueError("k, v must be [T, h_kv, d] matching q")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if o is None:
        o = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((h_q, T), dtype=torch.float32, device=dev)
    _need(o, "o", torch.float16, 3, dev)
    _need(lse, "lse", torch.float32, 2, dev)
    if o.shape != q.shape or lse.shape != (h_q, T):
        raise ValueError("o / lse shape mismatch")
    dims = varlen_dims(q, k, cu_seqlens, max_seqlen)
    if debug_validate_enabled():
        validate_varlen(dims, cu_seqlens)
    _check("attn_fwd", lib.attn_fwd(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v),
                                    _ptr(cu_seqlens), float(scale), _ptr(o), _ptr(lse),
                                    _stream()))
    return o, lse


def bwd_workspace_bytes(dims):
    return int(load_library().attn_bwd_workspace_bytes(ctypes.byref(dims)))


def bwd(q, k, v, o, lse, dout, cu_seqlens, scale=None, dq=None, dk=None, dv=None,
        max_seqlen=None, workspace=None, rope=None):
    """attn_bwd: returns (dq, dk, dv) in fp16. rope=(cos, sin) calls
    attn_bwd_rope: q and k are the rotated tensors and dq, dk come back
    rotated to the unrotated ones (inverse RoPE fused into their stores)."""
    lib = load_library()
    dev = q.device
    _need(q, "q", torch.float16, 3)
    for name, t in (("k", k), ("v", v), ("o", o), ("dout", dout)):
        _need(t, name, torch.float16, 3, dev)
    _need(lse, "lse", torch.float32, 2, dev)
    _need(cu_seqlens, "cu_seqlens", torch.int32, 1, dev)
    T, h_q, d = q.shape
    if o.shape != q.shape or dout.shape != q.shape or k.shape != v.shape or \
            lse.shape != (h_q, T) or k.shape[0] != T or k.shape[2] != d:
        raise ValueError("shape mismatch")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _need(dq, "dq", torch.float16, 3, dev)
    _need(dk, "dk", torch.float16, 3, dev)
    _need(dv, "dv", torch.float16, 3, dev)
    if dq.shape != q.shape or dk.shape != k.shape or dv.shape != v.shape:
        raise ValueError("gradient shape mismatch")
    dims = varlen_dims(q, k, cu_seqlens, max_seqlen)
    if debug_validate_enabled():
        validate_varlen(dims, cu_seqlens)
    need = int(lib.attn_bwd_workspace_bytes(ctypes.byref(dims)))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", torch.uint8, 1, dev)
    if rope is not None:
        tab = _rope_struct(rope, d=d, device=dev)
        _check("attn_bwd_rope",
               lib.attn_bwd_rope(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(o),
                                 _ptr(lse), _ptr(dout), _ptr(cu_seqlens), ctypes.byref(tab),
                                 _ptr(dq), _ptr(dk), _ptr(dv), float(scale), _ptr(workspace),
                                 workspace.numel(), _stream()))
        return dq, dk, dv
    _check("attn_bwd", lib.attn_bwd(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(o),
                                    _ptr(lse), _ptr(dout), _ptr(cu_seqlens), _ptr(dq),
                                    _ptr(dk), _ptr(dv), float(scale), _ptr(workspace),
                                    workspace.numel(), _stream()))
    return dq, dk, dv


def paged_dims(q, k_pool, block_table, max_ctx_len):
    n, h_q, d = q.shape
    nb, bs, h_kv, _ = k_pool.shape
    return PagedDims(n, h_q, h_kv, d, bs, block_table.shape[1], nb, int(max_ctx_len))


def decode_workspace_bytes(dims):
    return int(load_library().attn_decode_workspace_bytes(ctypes.byref(dims)))


def decode_paged(q, k_pool, v_pool, block_table, ctx_lens, scale=None, o=None,
                 max_ctx_len=None, workspace=None, rope=None):
    """attn_decode_paged: returns o fp16 [n, h_q, d]. rope=(cos, sin) calls
    attn_decode_paged_rope, which rotates each query by its position
    ctx_lens[b] - 1 as it loads it (q is not modified)."""
    lib = load_library()
    dev = q.device
    _need(q, "q", torch.float16, 3)
    _need(k_pool, "k_pool", torch.float16, 4, dev)
    _need(v_pool, "v_pool", torch.float16, 4, dev)
    _need(block_table, "block_table", torch.int32, 2, dev)
    _need(ctx_lens, "ctx_lens", torch.int32, 1, dev)
    n, h_q, d = q.shape
    if k_pool.shape != v_pool.shape or k_pool.shape[3] != d or block_table.shape[0] != n or \
            ctx_lens.shape[0] != n:
        raise ValueError("shape mismatch")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if max_ctx_len is None:  # host copy: synchronises, meant for tests
        max_ctx_len = int(ctx_lens.max()) if n else 0
    o = torch.empty_like(q) if o is None else o
    _need(o, "o", torch.float16, 3, dev)
    if o.shape != q.shape:
        raise ValueError("o shape mismatch")
    dims = paged_dims(q, k_pool, block_table, max_ctx_len)
    if debug_validate_enabled():
        validate_paged(dims, block_table, ctx_lens)
    need = int(lib.attn_decode_workspace_bytes(ctypes.byref(dims)))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", torch.uint8, 1, dev)
    if rope is not None:
        tab = _rope_struct(rope, d=d, device=dev)
        _check("attn_decode_paged_rope",
               lib.attn_decode_paged_rope(ctypes.byref(dims), _ptr(q), _ptr(k_pool),
                                          _ptr(v_pool), _ptr(block_table), _ptr(ctx_lens),
                                          ctypes.byref(tab), _ptr(o), float(scale),
                                          _ptr(workspace), workspace.numel(), _stream()))
        return o
    _check("attn_decode_paged",
           lib.attn_decode_paged(ctypes.byref(dims), _ptr(q), _ptr(k_pool), _ptr(v_pool),
                                 _ptr(block_table), _ptr(ctx_lens), _ptr(o), float(scale),
                                 _ptr(workspace), workspace.numel(), _stream()))
    return o


def decode_paged_noalloc(q, k_pool, v_pool, block_table, ctx_lens, o, max_ctx_len, scale=None):
    """attn_decode_paged_noalloc: attn_decode_paged with the library's own
    per-device workspace array, for callers that cannot allocate. The caller
    passes the output o (fp16 [n, h_q, d]) and the host bound max_ctx_len;
    nothing is allocated here or in the library. Returns o."""
    lib = load_library()
    dev = q.device
    _need(q, "q", torch.float16, 3)
    _need(k_pool, "k_pool", torch.float16, 4, dev)
    _need(v_pool, "v_pool", torch.float16, 4, dev)
    _need(block_table, "block_table", torch.int32, 2, dev)
    _need(ctx_lens, "ctx_lens", torch.int32, 1, dev)
    _need(o, "o", torch.float16, 3, dev)
    n, h_q, d = q.shape
    if k_pool.shape != v_pool.shape or k_pool.shape[3] != d or block_table.shape[0] != n or \
            ctx_lens.shape[0] != n or o.shape != q.shape:
        raise ValueError("shape mismatch")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dims = paged_dims(q, k_pool, block_table, max_ctx_len)
    _check("attn_decode_paged_noalloc",
           lib.attn_decode_paged_noalloc(ctypes.byref(dims), _ptr(q), _ptr(k_pool), _ptr(v_pool),
                                         _ptr(block_table), _ptr(ctx_lens), _ptr(o),
                                         float(scale), _stream()))
    return o


def check_cu_seqlens_host(dims, cu_host):
    """attn_check_cu_seqlens on a host int32 tensor."""
    cu_host = cu_host.to(torch.int32).contiguous()
    return int(load_library().attn_check_cu_seqlens(ctypes.byref(dims), _vp(cu_host.data_ptr())))


def check_paged_host(dims, block_table_host, ctx_host):
    """attn_check_paged on host int32 tensors."""
    bt = block_table_host.to(torch.int32).contiguous()
    cx = ctx_host.to(torch.int32).contiguous()
    return int(load_library().attn_check_paged(ctypes.byref(dims), _vp(bt.data_ptr()),
                                               _vp(cx.data_ptr())))


def prefill_dims(q_or_knew, k_pool, block_table, cu_q, max_ctx_len, max_q_len=None):
    """PrefillDims of a chunked prefill; host copies of max_ctx_len and (if
    not given) max_q_len size the launch."""
    n = cu_q.numel() - 1
    nb, bs, h_kv, d = k_pool.shape
    h = q_or_knew.shape[1]
    if max_q_len is None:  # host copy: synchronises, meant for tests
        cu = cu_q.cpu()
        max_q_len = int((cu[1:] - cu[:-1]).max()) if n > 0 else 0
    return PrefillDims(PagedDims(n, h, h_kv, d, bs, block_table.shape[1], nb, int(max_ctx_len)),
                       q_or_knew.shape[0], int(max_q_len))


def validate_prefill(dims, cu_q, block_table, ctx_lens):
    """Raise AttnError unless cu_q, block_table and ctx_lens (any device) are
    valid for dims."""
    _check("attn_check_prefill", check_prefill_host(dims, cu_q.cpu(), block_table.cpu(),
                                                    ctx_lens.cpu()))


def _prefill_args(k_pool, v_pool, block_table, ctx_lens, cu_q, dev):
    _need(k_pool, "k_pool", torch.float16, 4, dev)
    _need(v_pool, "v_pool", torch.float16, 4, dev)
    _need(block_table, "block_table", torch.int32, 2, dev)
    _need(ctx_lens, "ctx_lens", torch.int32, 1, dev)
    _need(cu_q, "cu_q", torch.int32, 1, dev)
    n = cu_q.numel() - 1
    if k_pool.shape != v_pool.shape or block_table.shape[0] != n or ctx_lens.shape[0] != n:
        raise ValueError("shape mismatch")


def kv_append(k_new, v_new, cu_q, block_table, ctx_lens, k_pool, v_pool, max_ctx_len=None,
              max_q_len=None, rope=None):
    """attn_kv_append: writes the new keys/values into k_pool / v_pool in place.
    rope=(cos, sin) (tables from ``rope_tables``) calls attn_kv_append_rope,
    which rotates the keys by their context positions on the way."""
    lib = load_library()
    dev = k_new.device
    _need(k_new, "k_new", torch.float16, 3)
    _need(v_new, "v_new", torch.float16, 3, dev)
    _prefill_args(k_pool, v_pool, block_table, ctx_lens, cu_q, dev)
    if k_new.shape != v_new.shape or k_new.shape[1:] != k_pool.shape[2:]:
        raise ValueError("k_new, v_new must be [total_q, h_kv, d] matching the pools")
    if max_ctx_len is None:  # host copy: synchronises, meant for tests
        max_ctx_len = int(ctx_lens.max()) if ctx_lens.numel() else 0
    dims = prefill_dims(k_new, k_pool, block_table, cu_q, max_ctx_len, max_q_len)
    if debug_validate_enabled():
        validate_prefill(dims, cu_q, block_table, ctx_lens)
    if rope is not None:
        tab = _rope_struct(rope, d=k_new.shape[2], device=dev)
        _check("attn_kv_append_rope",
               lib.attn_kv_append_rope(ctypes.byref(dims), _ptr(k_new), _ptr(v_new), _ptr(cu_q),
                                       _ptr(block_table), _ptr(ctx_lens), ctypes.byref(tab),
                                       _ptr(k_pool), _ptr(v_pool), _stream()))
        return k_pool, v_pool
    _check("attn_kv_append",
           lib.attn_kv_append(ctypes.byref(dims), _ptr(k_new), _ptr(v_new), _ptr(cu_q),
                              _ptr(block_table), _ptr(ctx_lens), _ptr(k_pool), _ptr(v_pool),
                              _stream()))
    return k_pool, v_pool


def prefill_paged(q, k_pool, v_pool, block_table, ctx_lens, cu_q, scale=None, o=None, lse=None,
                  with_lse=True, max_ctx_len=None, max_q_len=None, rope=None):
    """attn_prefill_paged: returns (o fp16 [total_q, h_q, d], lse fp32 [h_q, total_q] or None).
    rope=(cos, sin) calls attn_prefill_paged_rope, which rotates the queries
    by their context positions as it loads them (q is not modified)."""
    lib = load_library()
    dev = q.device
    _need(q, "q", torch.float16, 3)
    _prefill_args(k_pool, v_pool, block_table, ctx_lens, cu_q, dev)
    Tq, h_q, d = q.shape
    if k_pool.shape[3] != d:
        raise ValueError("q and the pools disagree on head_dim")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if max_ctx_len is None:  # host copy: synchronises, meant for tests
        max_ctx_len = int(ctx_lens.max()) if ctx_lens.numel() else 0
    o = torch.empty_like(q) if o is None else o
    _need(o, "o", torch.float16, 3, dev)
    if o.shape != q.shape:
        raise ValueError("o shape mismatch")
    if with_lse and lse is None:
        lse = torch.empty((h_q, Tq), dtype=torch.float32, device=dev)
    if lse is not None:
        _need(lse, "lse", torch.float32, 2, dev)
        if lse.shape != (h_q, Tq):
            raise ValueError("lse shape mismatch")
    dims = prefill_dims(q, k_pool, block_table, cu_q, max_ctx_len, max_q_len)
    if debug_validate_enabled():
        validate_prefill(dims, cu_q, block_table, ctx_lens)
    if rope is not None:
        tab = _rope_struct(rope, d=d, device=dev)
        _check("attn_prefill_paged_rope",
               lib.attn_prefill_paged_rope(ctypes.byref(dims), _ptr(q), _ptr(k_pool),
                                           _ptr(v_pool), _ptr(block_table), _ptr(ctx_lens),
                                           _ptr(cu_q), ctypes.byref(tab), _ptr(o), _ptr(lse),
                                           float(scale), _stream()))
        return o, lse
    _check("attn_prefill_paged",
           lib.attn_prefill_paged(ctypes.byref(dims), _ptr(q), _ptr(k_pool), _ptr(v_pool),
                                  _ptr(block_table), _ptr(ctx_lens), _ptr(cu_q), _ptr(o),
                                  _ptr(lse), float(scale), _stream()))
    return o, lse


def _rope_struct(rope, d, device):
    cos, sin = rope
    _need(cos, "rope cos", torch.float32, 2, device)
    _need(sin, "rope sin", torch.float32, 2, device)
    if cos.shape != sin.shape or cos.shape[1] != d // 2:
        raise ValueError("rope tables must both be [max_pos, head_dim / 2]")
    return RopeTables(cos.data_ptr(), sin.data_ptr(), cos.shape[0])


def rope_tables(max_pos, head_dim, base=1e6, device="cuda"):
    """attn_rope_tables_init: (cos, sin) fp32 [max_pos, head_dim / 2] of the
    angles p * base^(-2j / head_dim), evaluated on the device in fp64."""
    lib = load_library()
    cos = torch.empty((max_pos, head_dim // 2), dtype=torch.float32, device=device)
    sin = torch.empty_like(cos)
    _check("attn_rope_tables_init",
           lib.attn_rope_tables_init(int(max_pos), int(head_dim), float(base), _ptr(cos),
                                     _ptr(sin), _stream()))
    return cos, sin


def rope(q, k, cu_seqlens, tables, ctx_lens=None, max_ctx_len=None, max_seqlen=None,
         inverse=False):
    """attn_rope: rotates q [T, h_q, d] and k [T, h_kv, d] in place (either may
    be None) by their positions within their sequences, or, with ctx_lens,
    by their context positions as the new chunk of a cached sequence.
    inverse=True applies the transposed rotation (the backward of dq, dk)."""
    lib = load_library()
    ref = q if q is not None else k
    if ref is None:
        raise ValueError("nothing to rotate")
    dev = ref.device
    if q is not None:
        _need(q, "q", torch.float16, 3)
    if k is not None:
        _need(k, "k", torch.float16, 3, dev)
    _need(cu_seqlens, "cu_seqlens", torch.int32, 1, dev)
    T, d = ref.shape[0], ref.shape[2]
    h_q = q.shape[1] if q is not None else k.shape[1]
    h_kv = k.shape[1] if k is not None else h_q
    if (q is not None and k is not None) and (q.shape[0] != k.shape[0] or q.shape[2] != k.shape[2]):
        raise ValueError("q and k disagree on tokens or head_dim")
    if max_seqlen is None:  # host copy: synchronises, meant for tests
        c = cu_seqlens.cpu()
        max_seqlen = int((c[1:] - c[:-1]).max()) if c.numel() > 1 else 0
    if ctx_lens is not None:
        _need(ctx_lens, "ctx_lens", torch.int32, 1, dev)
        if max_ctx_len is None:  # host copy: synchronises, meant for tests
            max_ctx_len = int(ctx_lens.max()) if ctx_lens.numel() else 0
    dims = VarlenDims(cu_seqlens.numel() - 1, T, max_seqlen, h_q, h_kv, d)
    tab = _rope_struct(tables, d=d, device=dev)
    _check("attn_rope",
           lib.attn_rope(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(cu_seqlens), _ptr(ctx_lens),
                         int(max_ctx_len or 0), ctypes.byref(tab), int(bool(inverse)), _stream()))
    return q, k


def check_prefill_host(dims, cu_host, block_table_host, ctx_host):
    """attn_check_prefill on host int32 tensors."""
    cu = cu_host.to(torch.int32).contiguous()
    bt = block_table_host.to(torch.int32).contiguous()
    cx = ctx_host.to(torch.int32).contiguous()
    return int(load_library().attn_check_prefill(ctypes.byref(dims), _vp(cu.data_ptr()),
                                                 _vp(bt.data_ptr()), _vp(cx.data_ptr())))


def _norm_dims(x, w):
    _need(x, "x", torch.float16, 2)
    _need(w, "w", torch.float16, 1, x.device)
    if w.shape[0] != x.shape[1]:
        raise ValueError("w must have x.shape[1] entries")
    return NormDims(x.shape[0], x.shape[1])


def rmsnorm_fwd(x, w, eps=1e-6, y=None, rstd=None):
    """attn_rmsnorm_fwd: returns (y fp16 [rows, n], rstd fp32 [rows])."""
    lib = load_library()
    dims = _norm_dims(x, w)
    y = torch.empty_like(x) if y is None else y
    rstd = torch.empty(x.shape[0], dtype=torch.float32, device=x.device) if rstd is None else rstd
    _need(y, "y", torch.float16, 2, x.device)
    _need(rstd, "rstd", torch.float32, 1, x.device)
    if y.shape != x.shape or rstd.shape[0] != x.shape[0]:
        raise ValueError("y / rstd shape mismatch")
    _check("attn_rmsnorm_fwd", lib.attn_rmsnorm_fwd(ctypes.byref(dims), _ptr(x), _ptr(w),
                                                    float(eps), _ptr(y), _ptr(rstd), _stream()))
    return y, rstd


def rmsnorm_bwd_workspace_bytes(rows, n):
    return int(load_library().attn_rmsnorm_bwd_workspace_bytes(ctypes.byref(NormDims(rows, n))))


def rmsnorm_bwd(x, w, rstd, dy, dx=None, dw=None, workspace=None):
    """attn_rmsnorm_bwd: returns (dx fp16 [rows, n], dw fp32 [n])."""
    lib = load_library()
    dims = _norm_dims(x, w)
    _need(rstd, "rstd", torch.float32, 1, x.device)
    _need(dy, "dy", torch.float16, 2, x.device)
    if dy.shape != x.shape or rstd.shape[0] != x.shape[0]:
        raise ValueError("dy / rstd shape mismatch")
    dx = torch.empty_like(x) if dx is None else dx
    dw = torch.empty(x.shape[1], dtype=torch.float32, device=x.device) if dw is None else dw
    _need(dx, "dx", torch.float16, 2, x.device)
    _need(dw, "dw", torch.float32, 1, x.device)
    need = int(lib.attn_rmsnorm_bwd_workspace_bytes(ctypes.byref(dims)))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    _need(workspace, "workspace", torch.uint8, 1, x.device)
    _check("attn_rmsnorm_bwd",
           lib.attn_rmsnorm_bwd(ctypes.byref(dims), _ptr(x), _ptr(w), _ptr(rstd), _ptr(dy),
                                _ptr(dx), _ptr(dw), _ptr(workspace), workspace.numel(),
                                _stream()))
    return dx, dw


def sample(logits, u, temperature=1.0, top_k=50, top_p=1.0, tokens=None):
    """attn_sample: returns tokens int32 [n_rows] (u: fp32 uniforms, one per row)."""
    lib = load_library()
    _need(logits, "logits", torch.float32, 2)
    _need(u, "u", torch.float32, 1, logits.device)
    if u.shape[0] != logits.shape[0]:
        raise ValueError("u must have one entry per row")
    tokens = torch.empty(logits.shape[0], dtype=torch.int32, device=logits.device) \
        if tokens is None else tokens
    _need(tokens, "tokens", torch.int32, 1, logits.device)
    dims = SampleDims(logits.shape[0], logits.shape[1])
    _check("attn_sample", lib.attn_sample(ctypes.byref(dims), _ptr(logits), _ptr(u),
                                          float(temperature), int(top_k), float(top_p),
                                          _ptr(tokens), _stream()))
    return tokens
