"""Pins of the sampling oracle against facts that are not its own formula: a
hand-worked example, argmax and uniform limits, torch.topk as the library
routine for the top-k set, the measure of the uniforms that map to each
token, and masked (-inf) logits. Planted mistakes at the bottom must fail
at least one pin each.
"""
import numpy as np
import pytest
import torch

import oracle.sampling as S


def pin_worked_example(orc):
    """Probabilities (0.1, 0.5, 0.15, 0.25) at temperature 1: ranking
    1, 3, 2, 0 with cumulative mass 0.5, 0.75, 0.9, 1. top_p = 0.7 keeps
    ranks 0..1 (mass 0.75); u = 0.6 -> 0.45 of 0.75 -> token 1, u = 0.7 ->
    0.525 -> token 3. top_k = 3, top_p = 0.8 keeps ranks 0..2 of the top-3
    mass 0.9 (0.8 * 0.9 = 0.72 <= 0.75): u = 0.5 -> 0.375 -> token 1,
    u = 0.95 -> 0.7125 -> token 3."""
    lg = np.log(np.array([[0.1, 0.5, 0.15, 0.25]] * 2))
    t, cut, _ = orc.sample_ref(lg, [0.6, 0.7], 1.0, 4, 0.7)
    assert list(t) == [1, 3] and list(cut) == [1, 1]
    t, cut, _ = orc.sample_ref(lg, [0.5, 0.95], 1.0, 3, 0.8)
    assert list(t) == [1, 3] and list(cut) == [1, 1]
    t, cut, _ = orc.sample_ref(lg, [0.0, 0.999], 1.0, 4, 1.0)
    assert list(t) == [1, 0] and list(cut) == [3, 3]


def pin_top1_is_argmax(orc):
    r = np.random.default_rng(1)
    lg = r.standard_normal((6, 50))
    lg[2, [7, 30]] = lg[2].max() + 1.0  # tie at the maximum: lowest index wins
    t, _, _ = orc.sample_ref(lg, r.random(6), 0.8, 1, 0.9)
    expect = lg.argmax(1)
    assert list(t) == list(expect) and t[2] == 7


def pin_temperature_limits(orc):
    """A tiny temperature gives the argmax; a huge one makes the top-k
    weights equal, so u picks rank floor(u k) of the ranking."""
    r = np.random.default_rng(2)
    lg = r.standard_normal((5, 40))
    u = np.array([0.05, 0.31, 0.55, 0.77, 0.93])  # u k away from integers
    t, _, _ = orc.sample_ref(lg, u, 1e-6, 10, 1.0)
    assert list(t) == list(lg.argmax(1))
    t, _, _ = orc.sample_ref(lg, u, 1e12, 10, 1.0)
    for b in range(5):
        rank = np.argsort(-lg[b], kind="stable")
        assert t[b] == rank[int(u[b] * 10)]


def pin_topk_set_torch(orc):
    """With top_p = 1 every drawn token lies in torch.topk's set, and sweeping
    u reaches every member of it."""
    r = np.random.default_rng(3)
    lg = r.standard_normal((1, 200)) * 3
    k = 12
    top = set(torch.topk(torch.from_numpy(lg[0]), k).indices.tolist())
    us = np.linspace(0, 1, 20001)[:-1]
    t, _, _ = orc.sample_ref(np.repeat(lg, len(us), 0), us, 1.0, k, 1.0)
    # tokens of tiny mass may be missed by the grid; the heavy ones are hit
    assert set(t.tolist()) <= top and len(set(t.tolist())) >= 6


def pin_interval_measure(orc):
    """The uniforms mapping to a kept token form an interval of length
    p_t / (mass kept), with p from scipy's softmax of logits / T over the
    top-k set (tokens outside the kept prefix get none)."""
    from scipy.special import softmax
    r = np.random.default_rng(4)
    V, k, T, top_p = 30, 8, 0.7, 0.85
    lg = r.standard_normal(V) * 1.5
    top = np.argsort(-lg, kind="stable")[:k]
    p = softmax(lg[top] / T)
    keep = int(np.searchsorted(np.cumsum(p), top_p)) + 1
    q = p[:keep] / p[:keep].sum()
    us = (np.arange(200000) + 0.5) / 200000
    t, _, _ = orc.sample_ref(np.repeat(lg[None], len(us), 0), us, T, k, top_p)
    for i, tok in enumerate(top):
        frac = float((t == tok).mean())
        assert abs(frac - (q[i] if i < keep else 0.0)) < 2e-5, (i, frac)


def pin_masked_logits(orc):
    """-inf logits carry no weight and are never drawn, even inside top-k."""
    lg = np.full((3, 10), -np.inf)
    lg[:, 4] = 0.3
    lg[1, 6] = 0.1
    t, _, _ = orc.sample_ref(lg, [0.0, 0.99, 0.5], 1.0, 5, 1.0)
    assert t[0] == 4 and t[2] == 4 and t[1] in (4, 6)
    t, _, _ = orc.sample_ref(lg[1:2], [0.9999], 1.0, 5, 1.0)
    assert t[0] == 6


PINS = [pin_worked_example, pin_top1_is_argmax, pin_temperature_limits, pin_topk_set_torch,
        pin_interval_measure, pin_masked_logits]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_sampling_oracle_pin(pin):
    pin(S)


def _ranking_ascending(z):
    return np.lexsort((np.arange(z.shape[0]), z))


def _ranking_ties_high_index(z):
    return np.lexsort((-np.arange(z.shape[0]), -z))


MUTANTS = [
    ("ranking", _ranking_ascending, [pin_worked_example, pin_top1_is_argmax]),
    ("ranking", _ranking_ties_high_index, [pin_top1_is_argmax]),
]


@pytest.mark.parametrize("name,fn,pins", MUTANTS, ids=[f"{m[0]}:{m[1].__name__}" for m in MUTANTS])
def test_sampling_pins_catch_planted_mistake(monkeypatch, name, fn, pins):
    monkeypatch.setattr(S, name, fn)
    for pin in pins:
        with pytest.raises(Exception):
            pin(S)


def test_sampling_pins_catch_unnormalised_draw(monkeypatch):
    """A draw against the whole top-k mass instead of the kept prefix's mass
    changes the measure of each token's interval."""
    orig = S.sample_ref

    def mutant(logits, u, temperature, top_k, top_p):
        logits = np.asarray(logits, dtype=np.float64)
        n, V = logits.shape
        k = min(int(top_k), V)
        toks, cuts, cums = orig(logits, u, temperature, top_k, top_p)
        for b in range(n):
            z = logits[b] / temperature
            order = S.ranking(z)[:k]
            c = cums[b]
            j = int(np.searchsorted(c[:cuts[b] + 1], u[b] * c[-1], side="right"))
            toks[b] = order[min(j, cuts[b])]
        return toks, cuts, cums

    monkeypatch.setattr(S, "sample_ref", mutant)
    with pytest.raises(Exception):
        pin_interval_measure(S)
