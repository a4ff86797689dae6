"""Pins of the RMSNorm oracle against facts that are not its own formula:
PyTorch's CPU fp64 rms_norm and autograd, closed forms (constant rows, eps = 0
scale invariance), the orthogonality of dx to x that scale invariance
implies, and central finite differences. Planted mistakes at the bottom must
fail at least one pin each.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle.rmsnorm as R


def _case(rows, n, seed):
    r = np.random.default_rng(seed)
    return r.standard_normal((rows, n)), 1.0 + 0.5 * r.standard_normal(n), r.standard_normal((rows, n))


def pin_torch_fwd(orc):
    x, w, _ = _case(7, 96, 1)
    y, r = orc.rmsnorm_fwd_ref(x, w, 1e-6)
    yt = F.rms_norm(torch.from_numpy(x), (96,), torch.from_numpy(w), eps=1e-6)
    np.testing.assert_allclose(y, yt.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(r, 1 / np.sqrt((x ** 2).sum(1) / 96 + 1e-6), rtol=1e-14)


def pin_torch_autograd(orc):
    x, w, dy = _case(5, 64, 2)
    dx, dw = orc.rmsnorm_bwd_ref(x, w, dy, 1e-5)
    xt = torch.from_numpy(x).requires_grad_()
    wt = torch.from_numpy(w).requires_grad_()
    (F.rms_norm(xt, (64,), wt, eps=1e-5) * torch.from_numpy(dy)).sum().backward()
    np.testing.assert_allclose(dx, xt.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dw, wt.grad.numpy(), rtol=0, atol=1e-12)


def pin_constant_rows(orc):
    """A row of equal values c has RMS |c|: y = sign(c) w |c| / sqrt(c^2 + eps)."""
    w = np.linspace(0.5, 2.0, 16)
    x = np.array([[3.0] * 16, [-0.25] * 16])
    y, r = orc.rmsnorm_fwd_ref(x, w, 1e-3)
    for i, c in enumerate((3.0, -0.25)):
        np.testing.assert_allclose(y[i], np.sign(c) * w * abs(c) / np.sqrt(c * c + 1e-3),
                                   rtol=1e-14)
        np.testing.assert_allclose(r[i], 1 / np.sqrt(c * c + 1e-3), rtol=1e-14)


def pin_scale_invariance(orc):
    """With eps = 0, y(a x) = y(x) for every a > 0, hence sum_j dx_j x_j = 0."""
    x, w, dy = _case(4, 40, 3)
    y1, _ = orc.rmsnorm_fwd_ref(x, w, 0.0)
    y2, _ = orc.rmsnorm_fwd_ref(7.5 * x, w, 0.0)
    np.testing.assert_allclose(y1, y2, rtol=1e-13, atol=1e-13)
    dx, _ = orc.rmsnorm_bwd_ref(x, w, dy, 0.0)
    np.testing.assert_allclose((dx * x).sum(1), 0.0, atol=1e-12)


def pin_finite_differences(orc):
    x, w, dy = _case(3, 12, 4)
    eps, h = 1e-2, 1e-6
    dx, dw = orc.rmsnorm_bwd_ref(x, w, dy, eps)

    def loss(xx, ww):
        return float((orc.rmsnorm_fwd_ref(xx, ww, eps)[0] * dy).sum())

    for idx in [(0, 0), (1, 5), (2, 11)]:
        xp, xm = x.copy(), x.copy()
        xp[idx] += h
        xm[idx] -= h
        assert abs((loss(xp, w) - loss(xm, w)) / (2 * h) - dx[idx]) < 1e-7
    for j in (0, 6, 11):
        wp, wm = w.copy(), w.copy()
        wp[j] += h
        wm[j] -= h
        assert abs((loss(x, wp) - loss(x, wm)) / (2 * h) - dw[j]) < 1e-7


PINS = [pin_torch_fwd, pin_torch_autograd, pin_constant_rows, pin_scale_invariance,
        pin_finite_differences]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_rmsnorm_oracle_pin(pin):
    pin(R)


def _rrms_sum(x, eps):  # forgets to divide by n
    return 1.0 / np.sqrt((x * x).sum(axis=1) + eps)


def _rrms_eps_outside(x, eps):
    return 1.0 / (np.sqrt((x * x).mean(axis=1)) + eps)


def _bwd_without_projection(x, w, dy, eps):
    r = R._rrms(x, eps)
    return r[:, None] * dy * w[None, :], (dy * x * r[:, None]).sum(axis=0)


MUTANTS = [
    ("_rrms", _rrms_sum, [pin_torch_fwd, pin_constant_rows]),
    ("_rrms", _rrms_eps_outside, [pin_torch_fwd, pin_constant_rows]),
    ("rmsnorm_bwd_ref", _bwd_without_projection, [pin_torch_autograd, pin_scale_invariance,
                                                   pin_finite_differences]),
]


@pytest.mark.parametrize("name,fn,pins", MUTANTS, ids=[f"{m[0]}:{m[1].__name__}" for m in MUTANTS])
def test_rmsnorm_pins_catch_planted_mistake(monkeypatch, name, fn, pins):
    monkeypatch.setattr(R, name, fn)
    for pin in pins:
        with pytest.raises(Exception):
            pin(R)
