"""GPU parity of RMSNorm (attn_rmsnorm_fwd / attn_rmsnorm_bwd through the C
ABI) against the fp64 oracle on the same fp16 inputs.

Bars, from the arithmetic: y and dx are computed in fp32 and rounded once to
fp16, so each y element is within one fp16 ulp (2^-10 relative) of the exact
value; dx involves a difference of two fp32 terms, so it is held to a
relative L2 error of 1e-3 and a max error of 2e-3 of its largest entry; rstd
(fp32) to 1e-5 relative; dw (fp32 sums over the rows) to 1e-5 relative L2.
"""
import numpy as np
import pytest
import torch

from parity import W, attn, rel_l2
from oracle import rmsnorm_bwd_ref, rmsnorm_fwd_ref

pytestmark = pytest.mark.gpu

# (rows, n): every lane-group width (8, 16, 32, 64 lanes per row), ragged
# piece counts, one row, and the widest supported row. The last two give the
# backward's row groups one or two rows (more rows than one grid stride of
# 256 work-groups x 16 groups, not a multiple of it), so the loads of a
# group's next row are issued for some groups and not for others.
CASES = [(1, 8), (3, 64), (5, 96), (17, 128), (33, 1024), (7, 2048), (1000, 136), (300, 520),
         (4099, 256), (4500, 1024), (5000, 520)]


def _run(inp, device):
    x, w, dy = (inp[n].to(device) for n in ("x", "w", "dy"))
    y, rstd = attn.rmsnorm_fwd(x, w, inp["eps"])
    dx, dw = attn.rmsnorm_bwd(x, w, rstd, dy)
    torch.cuda.synchronize()
    return y, rstd, dx, dw


def _check(name, inp, y, rstd, dx, dw):
    x, w, dy = (inp[n].numpy() for n in ("x", "w", "dy"))
    y_ref, r_ref = rmsnorm_fwd_ref(x, w, inp["eps"])
    dx_ref, dw_ref = rmsnorm_bwd_ref(x, w, dy, inp["eps"])
    y = y.float().cpu().numpy()
    e_y = float((np.abs(y - y_ref) / (2.0 ** -10 * np.abs(y_ref) + 1e-7)).max())
    e_r = float((np.abs(rstd.cpu().numpy() - r_ref) / r_ref).max())
    dxg = dx.float().cpu().numpy()
    e_dx = rel_l2(dxg, dx_ref)
    e_dxm = float(np.abs(dxg - dx_ref).max() / np.abs(dx_ref).max())
    e_dw = rel_l2(dw.cpu().numpy(), dw_ref)
    print(f"{name}: y/ulp {e_y:.2f}  rstd rel {e_r:.1e}  dx relL2 {e_dx:.1e} max {e_dxm:.1e}  "
          f"dw relL2 {e_dw:.1e}", flush=True)
    assert e_y <= 1.0, f"{name}: y off by more than one fp16 ulp"
    assert e_r <= 1e-5
    assert e_dx <= 1e-3 and e_dxm <= 2e-3
    assert e_dw <= 1e-5


@pytest.mark.parametrize("rows,n", CASES, ids=lambda x: str(x))
def test_rmsnorm_shapes(gpu, rows, n):
    inp = W.make_norm_inputs(rows, n, seed=6000 + rows + n)
    _check(f"rmsnorm {rows}x{n}", inp, *_run(inp, gpu))


@pytest.mark.parametrize("name", ["qwen3_rmsnorm", "qwen3_qknorm"])
def test_rmsnorm_workloads(gpu, name):
    inp = W.norm_workload_inputs(name)
    _check(name, inp, *_run(inp, gpu))


def test_rmsnorm_bwd_reproducible(gpu):
    inp = W.make_norm_inputs(5000, 1024, seed=6100)
    a = _run(inp, gpu)
    b = _run(inp, gpu)
    for t, u in zip(a, b):
        assert torch.equal(t, u)
