"""Host-side tests of the C ABI (no GPU needed).

The library loads, exports every function include/attn.h declares, and
rejects bad arguments with the documented status codes before making any
HIP call. Only failing or empty calls are made here, so no kernel launches.
"""
import ctypes
import os
import re

import pytest
import torch

import causal_gqa_attention_fa2_amd as A
from causal_gqa_attention_fa2_amd.attn import PagedDims, VarlenDims

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3
FAKE = 0x10000  # an aligned non-null address that is never dereferenced


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    return A.load_library()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert {"attn_fwd", "attn_bwd", "attn_decode_paged"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    for code, name in A.attn.STATUS_NAMES.items():
        assert lib.attn_status_string(code).decode() == name
    assert lib.attn_status_string(99).decode() == "ATTN_UNKNOWN_STATUS"


def _fwd(lib, dims, q=FAKE, k=FAKE, v=FAKE, cu=FAKE, o=FAKE, lse=FAKE):
    p = ctypes.c_void_p
    return lib.attn_fwd(ctypes.byref(dims) if dims is not None else None, p(q), p(k), p(v),
                        p(cu), 0.1, p(o), p(lse), None)


def test_fwd_argument_checks(lib):
    good = dict(n_seqs=2, total_tokens=100, max_seqlen=60, h_q=16, h_kv=8, head_dim=128)
    assert _fwd(lib, None) == INVALID
    for field, bad, code in [("h_q", 15, INVALID), ("head_dim", 96, UNSUPPORTED),
                             ("head_dim", 256, UNSUPPORTED), ("h_kv", 0, INVALID),
                             ("n_seqs", -1, INVALID), ("max_seqlen", 101, INVALID),
                             ("max_seqlen", 0, INVALID), ("total_tokens", -5, INVALID)]:
        d = dict(good)
        d[field] = bad
        assert _fwd(lib, VarlenDims(**d)) == code, (field, bad)
    d = dict(good, h_q=17 * 2, h_kv=2)  # group of 17 query heads
    assert _fwd(lib, VarlenDims(**d)) == UNSUPPORTED
    # A batch whose work-item grid would not fit 32 bits: one long sequence
    # next to millions of one-token sequences.
    d = dict(good, n_seqs=2_000_000, total_tokens=4_000_000, max_seqlen=2_000_001)
    assert _fwd(lib, VarlenDims(**d)) == UNSUPPORTED
    dims = VarlenDims(**good)
    assert _fwd(lib, dims, q=0) == INVALID
    assert _fwd(lib, dims, lse=0) == INVALID
    assert _fwd(lib, dims, o=FAKE + 8) == INVALID     # misaligned
    assert _fwd(lib, dims, cu=FAKE + 2) == INVALID    # misaligned int32
    # Empty batches succeed without touching the (null) pointers.
    assert _fwd(lib, VarlenDims(0, 0, 0, 16, 8, 128), 0, 0, 0, 0, 0, 0) == OK
    assert _fwd(lib, VarlenDims(3, 0, 0, 16, 8, 128), 0, 0, 0, 0, 0, 0) == OK


def test_bwd_workspace(lib):
    dims = VarlenDims(2, 100, 60, 16, 8, 128)
    need = lib.attn_bwd_workspace_bytes(ctypes.byref(dims))
    row = (16 * 100 * 4 + 255) // 256 * 256
    assert need == 2 * row
    assert lib.attn_bwd_workspace_bytes(ctypes.byref(VarlenDims(0, 0, 0, 16, 8, 128))) == 0
    # Very unequal lengths (4 * 60 >= 1.25 * 100): room for the fp16 dS blocks too.
    ragged = lib.attn_bwd_workspace_bytes(ctypes.byref(VarlenDims(4, 100, 60, 16, 8, 128)))
    assert ragged == 2 * row + 4 * 16 * 2 * 2 * 32 * 32 * 2
    # Equal lengths keep the recompute path and its small workspace.
    eq = lib.attn_bwd_workspace_bytes(ctypes.byref(VarlenDims(8, 8192, 1024, 16, 8, 128)))
    assert eq == 2 * ((16 * 8192 * 4 + 255) // 256 * 256)
    # The dS blocks are bounded by 4 GiB: 2 sequences x 16 heads x 256^2 blocks
    # of 2 KiB is exactly that and keeps the dS path; one more 32-row block
    # (257^2) or a batch far above it (256 x 2 x 132^2) recomputes instead.
    row_t = lambda h, t: (h * t * 4 + 255) // 256 * 256
    at = lib.attn_bwd_workspace_bytes(ctypes.byref(VarlenDims(2, 8292, 8192, 16, 8, 128)))
    assert at == 2 * row_t(16, 8292) + (4 << 30)
    past = lib.attn_bwd_workspace_bytes(ctypes.byref(VarlenDims(2, 8293, 8193, 16, 8, 128)))
    assert past == 2 * row_t(16, 8293)
    big = lib.attn_bwd_workspace_bytes(ctypes.byref(VarlenDims(256, 11089, 4200, 2, 1, 64)))
    assert big == 2 * row_t(2, 11089)
    p = ctypes.c_void_p
    args = [p(FAKE)] * 7 + [p(FAKE)] * 3

    def call(ws, nbytes):
        return lib.attn_bwd(ctypes.byref(dims), *args, 0.1, p(ws), nbytes, None)

    assert call(0, need) == WORKSPACE
    assert call(FAKE, need - 1) == WORKSPACE
    assert call(FAKE + 16, need) == WORKSPACE  # workspace must be 256-byte aligned
    bad = VarlenDims(2, 100, 60, 16, 8, 80)
    assert lib.attn_bwd(ctypes.byref(bad), *args, 0.1, p(FAKE), need, None) == UNSUPPORTED


def test_decode_argument_checks(lib):
    dims = PagedDims(4, 16, 8, 128, 16, 256, 1000, 4096)
    need = lib.attn_decode_workspace_bytes(ctypes.byref(dims))
    nwg = min(512, 4 * (4096 // 16))  # work-groups of the balanced gather
    slots = (nwg + 4) * 16

    def al(x):
        return (x + 255) // 256 * 256

    assert need == al(slots * 128 * 4) + al(slots * 2 * 4) + al((4 + 1 + nwg) * 4)
    p = ctypes.c_void_p

    def call(d, ws=FAKE, nbytes=None, q=FAKE, bt=FAKE):
        return lib.attn_decode_paged(ctypes.byref(d), p(q), p(FAKE), p(FAKE), p(bt), p(FAKE),
                                     p(FAKE), 0.1, p(ws), need if nbytes is None else nbytes,
                                     None)

    assert call(PagedDims(4, 16, 8, 128, 32, 256, 1000, 4096)) == UNSUPPORTED
    assert call(PagedDims(4, 16, 8, 128, 16, 100, 1000, 4096)) == INVALID  # table too short
    assert call(PagedDims(4, 16, 6, 128, 16, 256, 1000, 4096)) == INVALID
    assert call(PagedDims(4, 16, 8, 128, 16, 256, 0, 4096)) == INVALID
    assert call(dims, q=0) == INVALID
    assert call(dims, bt=FAKE + 1) == INVALID
    assert call(dims, ws=0) == WORKSPACE
    assert call(dims, nbytes=need - 4) == WORKSPACE
    assert call(PagedDims(0, 16, 8, 128, 16, 256, 1000, 4096), ws=0, nbytes=0) == OK


def test_decode_noalloc_argument_checks(lib):
    """The allocation-free decode makes the decode's checks, then refuses a
    batch whose workspace exceeds its 32 MiB device array, all before any
    HIP call."""
    p = ctypes.c_void_p

    def call(d, q=FAKE, bt=FAKE):
        return lib.attn_decode_paged_noalloc(ctypes.byref(d), p(q), p(FAKE), p(FAKE), p(bt),
                                             p(FAKE), p(FAKE), 0.1, None)

    big = PagedDims(4096, 16, 8, 128, 16, 1, 1, 16)
    assert lib.attn_decode_workspace_bytes(ctypes.byref(big)) > (32 << 20)
    assert call(big) == WORKSPACE
    assert call(PagedDims(4, 16, 8, 128, 32, 256, 1000, 4096)) == UNSUPPORTED
    assert call(PagedDims(4, 16, 8, 128, 16, 100, 1000, 4096)) == INVALID
    assert call(PagedDims(4, 16, 8, 128, 16, 256, 1000, 4096), q=0) == INVALID
    assert call(PagedDims(4, 16, 8, 128, 16, 256, 1000, 4096), bt=FAKE + 1) == INVALID
    assert call(PagedDims(0, 16, 8, 128, 16, 256, 1000, 4096)) == OK
    assert lib.attn_decode_paged_noalloc(None, *([p(FAKE)] * 6), 0.1, None) == INVALID


def test_host_validators():
    dims = VarlenDims(3, 10, 7, 4, 2, 64)
    ok = torch.tensor([0, 3, 3, 10], dtype=torch.int32)
    assert A.attn.check_cu_seqlens_host(dims, ok) == OK
    assert A.attn.check_cu_seqlens_host(dims, torch.tensor([1, 3, 3, 10])) == INVALID
    assert A.attn.check_cu_seqlens_host(dims, torch.tensor([0, 3, 2, 10])) == INVALID
    assert A.attn.check_cu_seqlens_host(dims, torch.tensor([0, 3, 3, 9])) == INVALID
    assert A.attn.check_cu_seqlens_host(VarlenDims(3, 10, 6, 4, 2, 64), ok) == INVALID
    pd = PagedDims(2, 4, 2, 64, 16, 3, 5, 40)
    bt = torch.tensor([[4, 0, -1], [1, 2, 3]], dtype=torch.int32)
    assert A.attn.check_paged_host(pd, bt, torch.tensor([17, 40])) == OK
    assert A.attn.check_paged_host(pd, bt, torch.tensor([33, 40])) == INVALID  # entry -1 used
    assert A.attn.check_paged_host(pd, bt, torch.tensor([17, 41])) == INVALID  # > max ctx
    bt2 = bt.clone()
    bt2[1, 2] = 5
    assert A.attn.check_paged_host(pd, bt2, torch.tensor([17, 40])) == INVALID  # out of pool
    assert A.attn.check_paged_host(pd, bt, torch.tensor([0, 0])) == OK


def test_debug_validate_helpers(monkeypatch):
    """The checks ATTN_DEBUG_VALIDATE=1 runs before each launch raise on bad
    index contents (host tensors here; the binding copies device ones)."""
    monkeypatch.delenv("ATTN_DEBUG_VALIDATE", raising=False)
    assert not A.attn.debug_validate_enabled()
    monkeypatch.setenv("ATTN_DEBUG_VALIDATE", "1")
    assert A.attn.debug_validate_enabled()
    dims = VarlenDims(3, 10, 7, 4, 2, 64)
    A.attn.validate_varlen(dims, torch.tensor([0, 3, 3, 10], dtype=torch.int32))
    with pytest.raises(A.attn.AttnError):
        A.attn.validate_varlen(dims, torch.tensor([0, 3, 3, 9], dtype=torch.int32))
    pd = PagedDims(2, 4, 2, 64, 16, 3, 5, 40)
    bt = torch.tensor([[4, 0, -1], [1, 2, 3]], dtype=torch.int32)
    A.attn.validate_paged(pd, bt, torch.tensor([17, 40], dtype=torch.int32))
    with pytest.raises(A.attn.AttnError):
        A.attn.validate_paged(pd, bt, torch.tensor([33, 40], dtype=torch.int32))


def test_binding_rejects_host_tensors():
    q = torch.zeros(4, 2, 64, dtype=torch.float16)
    k = torch.zeros(4, 1, 64, dtype=torch.float16)
    cu = torch.tensor([0, 4], dtype=torch.int32)
    with pytest.raises(ValueError):
        A.fwd(q, k, k, cu)
    with pytest.raises(TypeError):
        A.fwd(q.float(), k, k, cu)


def test_prefill_argument_checks(lib):
    """attn_kv_append / attn_prefill_paged reject bad shapes and pointers
    before any HIP call; an empty batch is a no-op."""
    from causal_gqa_attention_fa2_amd.attn import PrefillDims
    p = ctypes.c_void_p

    def dims(n=4, h_q=16, h_kv=8, d=128, bs=16, maxb=64, nb=1000, max_ctx=1024, tq=300, mq=100):
        return PrefillDims(PagedDims(n, h_q, h_kv, d, bs, maxb, nb, max_ctx), tq, mq)

    def pre(dm, q=FAKE, cu=FAKE, lse=FAKE):
        return lib.attn_prefill_paged(ctypes.byref(dm), p(q), p(FAKE), p(FAKE), p(FAKE), p(FAKE),
                                      p(cu), p(FAKE), p(lse), 0.1, None)

    def app(dm, kn=FAKE, bt=FAKE):
        return lib.attn_kv_append(ctypes.byref(dm), p(kn), p(FAKE), p(FAKE), p(bt), p(FAKE),
                                  p(FAKE), p(FAKE), None)

    assert lib.attn_prefill_paged(None, *([p(FAKE)] * 8), 0.1, None) == INVALID
    for fn in (pre, app):
        assert fn(dims(bs=32)) == UNSUPPORTED
        assert fn(dims(d=96)) == UNSUPPORTED
        assert fn(dims(h_q=12)) == INVALID
        assert fn(dims(maxb=10)) == INVALID           # table shorter than max_ctx
        assert fn(dims(mq=301)) == INVALID            # longer than total_q
        assert fn(dims(mq=2000, tq=3000)) == INVALID  # chunk longer than any context
        assert fn(dims(mq=0)) == INVALID              # tokens but no chunk length
        assert fn(dims(n=0, tq=0, mq=0)) == OK        # empty batch
        assert fn(dims(tq=0, mq=0)) == OK             # no new tokens
    assert pre(dims(), q=0) == INVALID
    assert pre(dims(), cu=FAKE + 2) == INVALID
    assert pre(dims(), lse=FAKE + 4) == INVALID
    assert app(dims(), kn=0) == INVALID
    assert app(dims(), bt=FAKE + 1) == INVALID


def test_prefill_host_validator():
    from causal_gqa_attention_fa2_amd.attn import PrefillDims
    pd = PrefillDims(PagedDims(2, 4, 2, 64, 16, 3, 5, 40), 12, 10)
    bt = torch.tensor([[4, 0, -1], [1, 2, 3]], dtype=torch.int32)
    ctx = torch.tensor([17, 40], dtype=torch.int32)
    chk = A.attn.check_prefill_host
    assert chk(pd, torch.tensor([0, 2, 12]), bt, ctx) == OK
    assert chk(pd, torch.tensor([0, 2, 11]), bt, ctx) == INVALID   # does not end at total_q
    assert chk(pd, torch.tensor([0, 0, 12]), bt, ctx) == INVALID   # chunk above max_q_len
    assert chk(pd, torch.tensor([1, 2, 12]), bt, ctx) == INVALID   # does not start at 0
    small = torch.tensor([1, 40], dtype=torch.int32)
    assert chk(pd, torch.tensor([0, 2, 12]), bt, small) == INVALID  # chunk longer than context
    assert chk(pd, torch.tensor([0, 2, 12]), bt, torch.tensor([33, 40])) == INVALID  # entry -1


def test_debug_validate_prefill_helper():
    """The prefill check that ATTN_DEBUG_VALIDATE=1 runs raises on a chunk
    longer than its context."""
    from causal_gqa_attention_fa2_amd.attn import PrefillDims
    pd = PrefillDims(PagedDims(2, 4, 2, 64, 16, 3, 5, 40), 12, 10)
    bt = torch.tensor([[4, 0, -1], [1, 2, 3]], dtype=torch.int32)
    cu = torch.tensor([0, 2, 12], dtype=torch.int32)
    A.attn.validate_prefill(pd, cu, bt, torch.tensor([17, 40], dtype=torch.int32))
    with pytest.raises(A.attn.AttnError):
        A.attn.validate_prefill(pd, cu, bt, torch.tensor([1, 40], dtype=torch.int32))


def test_rmsnorm_argument_checks(lib):
    from causal_gqa_attention_fa2_amd.attn import NormDims
    p = ctypes.c_void_p

    def fwd(d, x=FAKE, rstd=FAKE, eps=1e-6):
        return lib.attn_rmsnorm_fwd(ctypes.byref(d), p(x), p(FAKE), eps, p(FAKE), p(rstd), None)

    def bwd(d, ws=FAKE, nbytes=1 << 30, dw=FAKE):
        return lib.attn_rmsnorm_bwd(ctypes.byref(d), p(FAKE), p(FAKE), p(FAKE), p(FAKE), p(FAKE),
                                    p(dw), p(ws), nbytes, None)

    assert fwd(NormDims(10, 100)) == UNSUPPORTED   # n % 8
    assert fwd(NormDims(10, 4096)) == UNSUPPORTED  # n above 2048
    assert fwd(NormDims(-1, 128)) == INVALID
    assert fwd(NormDims(10, 0)) == INVALID
    assert fwd(NormDims(10, 128), eps=-1.0) == INVALID
    assert fwd(NormDims(10, 128), x=0) == INVALID
    assert fwd(NormDims(10, 128), rstd=FAKE + 2) == INVALID
    assert fwd(NormDims(0, 128), x=0) == OK        # no rows: nothing to do
    need = lib.attn_rmsnorm_bwd_workspace_bytes(ctypes.byref(NormDims(8192, 1024)))
    assert need == min(8192 // 16, 256) * 1024 * 4  # a partial row per 16 rows, at most 256
    assert lib.attn_rmsnorm_bwd_workspace_bytes(ctypes.byref(NormDims(40, 1024))) == 3 * 4096
    assert lib.attn_rmsnorm_bwd_workspace_bytes(ctypes.byref(NormDims(1 << 20, 1024))) == \
        256 * 1024 * 4
    assert lib.attn_rmsnorm_bwd_workspace_bytes(ctypes.byref(NormDims(0, 1024))) == 0
    assert bwd(NormDims(8192, 1024), ws=0) == WORKSPACE
    assert bwd(NormDims(8192, 1024), nbytes=need - 4) == WORKSPACE
    assert bwd(NormDims(8192, 1024), dw=FAKE + 2) == INVALID
    assert bwd(NormDims(8192, 100)) == UNSUPPORTED


def test_sample_argument_checks(lib):
    from causal_gqa_attention_fa2_amd.attn import SampleDims
    p = ctypes.c_void_p

    def call(d, t=0.7, k=20, tp=0.9, lg=FAKE, u=FAKE, out=FAKE):
        return lib.attn_sample(ctypes.byref(d), p(lg), p(u), t, k, tp, p(out), None)

    d = SampleDims(4, 1000)
    assert call(SampleDims(-1, 1000)) == INVALID
    assert call(SampleDims(4, 0)) == INVALID
    assert call(d, t=0.0) == INVALID
    assert call(d, t=float("nan")) == INVALID
    assert call(d, t=float("inf")) == INVALID
    assert call(d, k=0) == INVALID
    assert call(d, k=1025) == UNSUPPORTED
    assert call(d, tp=0.0) == INVALID
    assert call(d, tp=1.5) == INVALID
    assert call(d, lg=0) == INVALID
    assert call(d, out=FAKE + 2) == INVALID
    assert call(SampleDims(0, 1000), lg=0, u=0, out=0) == OK


def test_rope_argument_checks(lib):
    """attn_rope_tables_init / attn_rope / attn_kv_append_rope /
    attn_prefill_paged_rope reject bad tables, shapes and pointers before any
    HIP call; empty batches are no-ops."""
    from causal_gqa_attention_fa2_amd.attn import PrefillDims, RopeTables
    p = ctypes.c_void_p
    init = lib.attn_rope_tables_init
    assert init(0, 128, 1e6, p(FAKE), p(FAKE), None) == INVALID
    assert init(100, 96, 1e6, p(FAKE), p(FAKE), None) == UNSUPPORTED
    assert init(100, 128, 1.0, p(FAKE), p(FAKE), None) == INVALID
    assert init(100, 128, 1e6, None, p(FAKE), None) == INVALID
    assert init(100, 128, 1e6, p(FAKE), p(FAKE + 4), None) == INVALID

    def tab(mp=4096, c=FAKE, s=FAKE):
        return ctypes.byref(RopeTables(c, s, mp))

    def vd(n=2, T=100, mx=60, h_q=16, h_kv=8, d=128):
        return ctypes.byref(VarlenDims(n, T, mx, h_q, h_kv, d))

    def rope(dm=None, q=FAKE, k=FAKE, cu=FAKE, ctx=None, mctx=0, t=None, inv=0):
        return lib.attn_rope(dm if dm is not None else vd(), p(q), p(k), p(cu), p(ctx), mctx,
                             t if t is not None else tab(), inv, None)

    assert lib.attn_rope(vd(), p(FAKE), p(FAKE), p(FAKE), None, 0, None, 0, None) == INVALID
    assert rope(t=tab(mp=59)) == INVALID            # tables shorter than max_seqlen
    assert rope(t=tab(mp=0)) == INVALID
    assert rope(t=tab(c=0)) == INVALID
    assert rope(t=tab(s=FAKE + 8)) == INVALID       # misaligned table
    assert rope(ctx=FAKE, mctx=50) == INVALID       # max_ctx_len below max_seqlen
    assert rope(ctx=FAKE, mctx=5000) == INVALID     # contexts past the tables
    assert rope(dm=vd(d=96)) == UNSUPPORTED
    assert rope(dm=vd(h_q=12)) == INVALID
    assert rope(q=FAKE + 2) == INVALID
    assert rope(cu=FAKE + 2) == INVALID
    assert rope(dm=vd(n=0, T=0, mx=0)) == OK        # empty batch
    assert rope(q=0, k=0) == OK                     # nothing to rotate

    def dims(n=4, max_ctx=1024, tq=300, mq=100):
        return PrefillDims(PagedDims(n, 16, 8, 128, 16, 64, 1000, max_ctx), tq, mq)

    def app(dm, t):
        return lib.attn_kv_append_rope(ctypes.byref(dm), p(FAKE), p(FAKE), p(FAKE), p(FAKE),
                                       p(FAKE), t, p(FAKE), p(FAKE), None)

    def pre(dm, t):
        return lib.attn_prefill_paged_rope(ctypes.byref(dm), p(FAKE), p(FAKE), p(FAKE), p(FAKE),
                                           p(FAKE), p(FAKE), t, p(FAKE), p(FAKE), 0.1, None)

    for fn in (app, pre):
        assert fn(dims(), None) == INVALID
        assert fn(dims(), tab(mp=1000)) == INVALID  # tables shorter than max_ctx_len
        assert fn(dims(), tab(c=FAKE + 4)) == INVALID
        assert fn(dims(n=0, tq=0, mq=0), tab()) == OK


def test_bwd_rope_argument_checks(lib):
    """attn_bwd_rope: tables required and long enough; otherwise attn_bwd's
    checks (empty batch is a no-op)."""
    from causal_gqa_attention_fa2_amd.attn import RopeTables
    p = ctypes.c_void_p
    dims = VarlenDims(2, 100, 60, 16, 8, 128)

    def call(dm, t, ws_bytes=1 << 30):
        return lib.attn_bwd_rope(ctypes.byref(dm), *([p(FAKE)] * 7), t, p(FAKE), p(FAKE),
                                 p(FAKE), 0.1, p(FAKE), ws_bytes, None)

    assert call(dims, None) == INVALID
    assert call(dims, ctypes.byref(RopeTables(FAKE, FAKE, 59))) == INVALID
    assert call(dims, ctypes.byref(RopeTables(FAKE, FAKE + 4, 100))) == INVALID
    assert call(dims, ctypes.byref(RopeTables(FAKE, FAKE, 100)), ws_bytes=0) == WORKSPACE
    assert call(VarlenDims(0, 0, 0, 16, 8, 128), ctypes.byref(RopeTables(FAKE, FAKE, 100))) == OK


def test_decode_rope_argument_checks(lib):
    """attn_decode_paged_rope: tables required and covering max_ctx_len."""
    from causal_gqa_attention_fa2_amd.attn import RopeTables
    p = ctypes.c_void_p
    dims = PagedDims(4, 16, 8, 128, 16, 64, 1000, 1024)

    def call(dm, t, ws_bytes=1 << 30):
        return lib.attn_decode_paged_rope(ctypes.byref(dm), *([p(FAKE)] * 5), t, p(FAKE), 0.1,
                                          p(FAKE), ws_bytes, None)

    assert call(dims, None) == INVALID
    assert call(dims, ctypes.byref(RopeTables(FAKE, FAKE, 1000))) == INVALID
    assert call(dims, ctypes.byref(RopeTables(FAKE + 8, FAKE, 2048))) == INVALID
    assert call(dims, ctypes.byref(RopeTables(FAKE, FAKE, 2048)), ws_bytes=0) == WORKSPACE
    assert call(PagedDims(0, 16, 8, 128, 16, 64, 1000, 1024),
                ctypes.byref(RopeTables(FAKE, FAKE, 2048))) == OK
