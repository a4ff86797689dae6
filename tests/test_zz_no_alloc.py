"""attn_decode_paged_noalloc, the decode for callers that cannot allocate,
against attn_decode_paged (the workspace entry point) on the same inputs.

Two calls in a row share the library's per-device array: the paged-decode
workload (256 sequences, contexts up to 4096), then a smaller ragged batch
(empty, one-token and block-edge contexts, d = 64) that reuses the array the
first call left its partials in. Both run the same kernels with the same
launch as the workspace entry point, so each output must equal that entry
point's bit for bit; the smaller case is also held to the decode's oracle
tolerance.
"""
import ctypes

import pytest
import torch

from parity import W, attn, check_decode, dev, gpu_decode

CASES = [
    ("paged_decode", lambda: W.decode_workload_inputs()),
    ("ragged_small", lambda: W.make_decode_inputs([0, 1, 15, 16, 17, 300, 1025], 8, 2, 64,
                                                  seed=3301, spare_blocks=5)),
]


def _noalloc(d, o):
    return attn.decode_paged_noalloc(d["q"], d["k_pool"], d["v_pool"], d["block_table"],
                                     d["ctx_lens"], o, d["max_ctx"], d["scale"])


@pytest.mark.gpu
def test_noalloc_decode_matches_workspace_entry(gpu):
    for name, make in CASES:
        print(f"[noalloc] case {name}", flush=True)
        inp = make()
        d = dev(inp, gpu)
        ref = gpu_decode(d)
        o = torch.full_like(d["q"], float("nan"))
        _noalloc(d, o)
        torch.cuda.synchronize()
        assert torch.equal(o, ref), (name, (o.float() - ref.float()).abs().max().item())
        if name == "ragged_small":
            check_decode(f"noalloc {name}", inp, o.cpu())


@pytest.mark.gpu
def test_noalloc_decode_rejects_oversize(gpu):
    """A batch whose workspace would exceed the device array is refused
    before anything is enqueued (the output keeps its contents)."""
    lib = attn.load_library()
    n = 4096
    dims = attn.PagedDims(n, 16, 8, 128, 16, 1, 1, 16)
    assert lib.attn_decode_workspace_bytes(ctypes.byref(dims)) > (32 << 20)
    q = torch.zeros(n, 16, 128, dtype=torch.float16, device=gpu)
    pool = torch.zeros(1, 16, 8, 128, dtype=torch.float16, device=gpu)
    table = torch.zeros(n, 1, dtype=torch.int32, device=gpu)
    ctx = torch.ones(n, dtype=torch.int32, device=gpu)
    o = torch.full_like(q, 7.0)
    with pytest.raises(attn.AttnError) as e:
        attn.decode_paged_noalloc(q, pool, pool, table, ctx, o, 16)
    assert e.value.status == 3  # ATTN_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((o == 7.0).all())
