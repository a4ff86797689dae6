"""Pins of the fp64 CPU oracle against facts that do not come from the oracle.

Each ``pin_*`` function checks the oracle module it is given against one of:
a hand-derived worked example (tests/golden), a closed form, an invariant of
softmax attention, central finite differences, or PyTorch's own CPU fp64
attention routine. The mutation tests at the bottom plant plausible mistakes
into the oracle (on the CPU) and check that the pins catch each of them.
"""
import json
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle.attention as OA

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")


def _rng(seed):
    return np.random.default_rng(seed)


def _cu(lens):
    return np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)


def _train_case(lens, h_q, h_kv, d, seed):
    r = _rng(seed)
    T = int(sum(lens))
    return (r.standard_normal((T, h_q, d)), r.standard_normal((T, h_kv, d)),
            r.standard_normal((T, h_kv, d)), r.standard_normal((T, h_q, d)), _cu(lens))


def _arr(x):
    return np.array(x, dtype=np.float64)


def _golden(name):
    with open(GOLDEN) as f:
        return json.load(f)[name]


# ----------------------------------------------------------------------------- forward pins

def pin_golden_fwd_bwd(orc):
    ex = _golden("two_token_fwd_bwd")
    q, k, v, do = (_arr(ex[n]) for n in ("q", "k", "v", "dout"))
    o, lse = orc.attn_fwd_ref(q, k, v, ex["cu_seqlens"], ex["scale"])
    np.testing.assert_allclose(o, _arr(ex["o"]), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, _arr(ex["lse"]), rtol=0, atol=1e-12)
    dq, dk, dv = orc.attn_bwd_ref(q, k, v, do, ex["cu_seqlens"], ex["scale"])
    np.testing.assert_allclose(dq, _arr(ex["dq"]), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dk, _arr(ex["dk"]), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dv, _arr(ex["dv"]), rtol=0, atol=1e-12)


def pin_row0_single_key(orc):
    """The first query of a sequence sees only its own key: O = v exactly and
    LSE = its scaled score."""
    lens = [1, 5, 3]
    q, k, v, _, cu = _train_case(lens, 4, 2, 8, 1)
    scale = 0.3
    o, lse = orc.attn_fwd_ref(q, k, v, cu, scale)
    for s in cu[:-1]:
        for h in range(4):
            g = h // 2
            assert np.array_equal(o[s, h], v[s, g])
            assert abs(lse[h, s] - scale * np.dot(q[s, h], k[s, g])) < 1e-12


def pin_zero_query(orc):
    """q = 0 makes every allowed score 0: O_i is the mean of v_0..v_i and
    LSE_i = ln(i + 1)."""
    lens = [7, 4]
    _, k, v, _, cu = _train_case(lens, 2, 1, 5, 2)
    q = np.zeros((sum(lens), 2, 5))
    o, lse = orc.attn_fwd_ref(q, k, v, cu, 0.9)
    for b, L in enumerate(lens):
        s = cu[b]
        counts = np.arange(1, L + 1)[:, None]
        mean = np.cumsum(v[s:s + L, 0], axis=0) / counts
        for h in range(2):
            np.testing.assert_allclose(o[s:s + L, h], mean, rtol=0, atol=1e-12)
            np.testing.assert_allclose(lse[h, s:s + L], np.log(np.arange(1, L + 1)),
                                       rtol=0, atol=1e-12)


def pin_identical_keys(orc):
    """All keys of a sequence equal to c: every allowed score of row i is
    s_i = scale <q_i, c>, so O_i is the prefix mean of v and
    LSE_i = s_i + ln(i + 1)."""
    L, d, scale = 9, 6, 0.5
    r = _rng(3)
    q = r.standard_normal((L, 2, d))
    c = r.standard_normal(d)
    k = np.tile(c, (L, 1, 1))
    v = r.standard_normal((L, 1, d))
    o, lse = orc.attn_fwd_ref(q, k, v, [0, L], scale)
    mean = np.cumsum(v[:, 0], axis=0) / np.arange(1, L + 1)[:, None]
    for h in range(2):
        np.testing.assert_allclose(o[:, h], mean, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse[h], scale * (q[:, h] @ c) + np.log(np.arange(1, L + 1)),
                                   rtol=0, atol=1e-12)


def pin_rows_sum_to_one(orc):
    """With every value vector equal to ones, O_i = sum_j P_ij must be 1."""
    lens = [13, 6]
    q, k, _, _, cu = _train_case(lens, 4, 1, 4, 4)
    v = np.ones_like(k)
    o, _ = orc.attn_fwd_ref(q, k, v, cu, 1.7)
    np.testing.assert_allclose(o, 1.0, rtol=0, atol=1e-12)


def pin_causality(orc):
    """Changing q, k or v at positions after p leaves O and LSE at positions
    up to p bitwise unchanged; it does change a later row."""
    lens = [12]
    q, k, v, _, cu = _train_case(lens, 2, 1, 8, 5)
    o, lse = orc.attn_fwd_ref(q, k, v, cu, 0.4)
    p = 6
    r = _rng(6)
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    q2[p + 1:] += r.standard_normal(q2[p + 1:].shape)
    k2[p + 1:] += r.standard_normal(k2[p + 1:].shape)
    v2[p + 1:] += r.standard_normal(v2[p + 1:].shape)
    o2, lse2 = orc.attn_fwd_ref(q2, k2, v2, cu, 0.4)
    assert np.array_equal(o[:p + 1], o2[:p + 1])
    assert np.array_equal(lse[:, :p + 1], lse2[:, :p + 1])
    assert not np.allclose(o[p + 1:], o2[p + 1:])


def pin_gqa_equals_repeat(orc):
    """GQA equals ordinary multi-head attention on K/V whose heads are
    repeat-interleaved G times; the GQA gradient of a K/V head is the sum of
    the repeated heads' gradients."""
    lens = [5, 8]
    h_q, h_kv, d, G = 6, 2, 4, 3
    q, k, v, do, cu = _train_case(lens, h_q, h_kv, d, 7)
    kr, vr = np.repeat(k, G, axis=1), np.repeat(v, G, axis=1)
    o, lse = orc.attn_fwd_ref(q, k, v, cu, 0.6)
    o_r, lse_r = orc.attn_fwd_ref(q, kr, vr, cu, 0.6)
    assert np.array_equal(o, o_r) and np.array_equal(lse, lse_r)
    dq, dk, dv = orc.attn_bwd_ref(q, k, v, do, cu, 0.6)
    dq_r, dk_r, dv_r = orc.attn_bwd_ref(q, kr, vr, do, cu, 0.6)
    T = sum(lens)
    np.testing.assert_allclose(dq, dq_r, rtol=0, atol=1e-12)
    np.testing.assert_allclose(dk, dk_r.reshape(T, h_kv, G, d).sum(2), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dv, dv_r.reshape(T, h_kv, G, d).sum(2), rtol=0, atol=1e-12)


def pin_varlen_concat(orc):
    """A packed batch (with empty sequences) equals its sequences run one by
    one and concatenated."""
    lens = [3, 0, 5, 1, 0]
    q, k, v, do, cu = _train_case(lens, 4, 2, 6, 8)
    o, lse = orc.attn_fwd_ref(q, k, v, cu, 0.45)
    dq, dk, dv = orc.attn_bwd_ref(q, k, v, do, cu, 0.45)
    for b, L in enumerate(lens):
        s = cu[b]
        sl = slice(s, s + L)
        o1, lse1 = orc.attn_fwd_ref(q[sl], k[sl], v[sl], [0, L], 0.45)
        assert np.array_equal(o[sl], o1) and np.array_equal(lse[:, sl], lse1)
        g1 = orc.attn_bwd_ref(q[sl], k[sl], v[sl], do[sl], [0, L], 0.45)
        for a, b1 in zip((dq, dk, dv), g1):
            assert np.array_equal(a[sl], b1)


def _torch_seq(x, s, L):
    return torch.from_numpy(np.ascontiguousarray(x[s:s + L].transpose(1, 0, 2)))[None]


def pin_torch_sdpa_fwd(orc):
    """PyTorch's CPU fp64 scaled_dot_product_attention (causal, GQA) and
    torch.logsumexp of its masked scores, per sequence."""
    lens = [17, 1, 30]
    h_q, h_kv, d, scale = 8, 2, 16, 0.21
    q, k, v, _, cu = _train_case(lens, h_q, h_kv, d, 9)
    o, lse = orc.attn_fwd_ref(q, k, v, cu, scale)
    for b, L in enumerate(lens):
        s = cu[b]
        tq, tk, tv = _torch_seq(q, s, L), _torch_seq(k, s, L), _torch_seq(v, s, L)
        ot = F.scaled_dot_product_attention(tq, tk, tv, is_causal=True, scale=scale,
                                            enable_gqa=True)
        np.testing.assert_allclose(o[s:s + L], ot[0].permute(1, 0, 2).numpy(), rtol=0,
                                   atol=1e-12)
        sc = scale * tq[0] @ tk[0].repeat_interleave(h_q // h_kv, 0).transpose(1, 2)
        sc = sc.masked_fill(torch.ones(L, L, dtype=torch.bool).triu(1), float("-inf"))
        np.testing.assert_allclose(lse[:, s:s + L], torch.logsumexp(sc, -1).numpy(), rtol=0,
                                   atol=1e-12)


# ----------------------------------------------------------------------------- backward pins

def pin_torch_autograd_bwd(orc):
    """Gradients of <O, dO> from torch autograd through fp64 SDPA."""
    lens = [11, 4]
    h_q, h_kv, d, scale = 4, 2, 8, 0.33
    q, k, v, do, cu = _train_case(lens, h_q, h_kv, d, 10)
    dq, dk, dv = orc.attn_bwd_ref(q, k, v, do, cu, scale)
    for b, L in enumerate(lens):
        s = cu[b]
        tq, tk, tv = (_torch_seq(x, s, L).requires_grad_() for x in (q, k, v))
        ot = F.scaled_dot_product_attention(tq, tk, tv, is_causal=True, scale=scale,
                                            enable_gqa=True)
        (ot * _torch_seq(do, s, L)).sum().backward()
        for mine, t in ((dq, tq), (dk, tk), (dv, tv)):
            np.testing.assert_allclose(mine[s:s + L], t.grad[0].permute(1, 0, 2).numpy(),
                                       rtol=0, atol=1e-11)


def pin_finite_differences(orc):
    """Central differences (h = 1e-6) of L = <O, W> against the analytic
    gradients, on a tiny two-sequence GQA case."""
    lens = [3, 2]
    q, k, v, w, cu = _train_case(lens, 2, 1, 3, 11)
    scale = 0.7

    def loss(q_, k_, v_):
        return float((orc.attn_fwd_ref(q_, k_, v_, cu, scale)[0] * w).sum())

    grads = orc.attn_bwd_ref(q, k, v, w, cu, scale)
    h = 1e-6
    for which, g in zip(range(3), grads):
        args = [q, k, v]
        num = np.zeros_like(args[which])
        for idx in np.ndindex(num.shape):
            plus = [a.copy() for a in args]
            minus = [a.copy() for a in args]
            plus[which][idx] += h
            minus[which][idx] -= h
            num[idx] = (loss(*plus) - loss(*minus)) / (2 * h)
        err = np.abs(num - g).max() / max(np.abs(num).max(), 1e-30)
        assert err <= 1e-6, (which, err)


def pin_bwd_invariants(orc):
    """Rows of dS sum to 0, so sum_j dK_j = 0 per (sequence, K/V head); rows
    of P sum to 1, so sum_j dV_j = sum over the group's heads and rows of dO;
    equal keys give dQ = 0."""
    lens = [9, 14]
    h_q, h_kv, d = 4, 2, 5
    q, k, v, do, cu = _train_case(lens, h_q, h_kv, d, 12)
    dq, dk, dv = orc.attn_bwd_ref(q, k, v, do, cu, 0.5)
    for b, L in enumerate(lens):
        sl = slice(cu[b], cu[b] + L)
        np.testing.assert_allclose(dk[sl].sum(0), 0.0, rtol=0, atol=1e-11)
        grp = do[sl].reshape(L, h_kv, h_q // h_kv, d).sum(axis=(0, 2))
        np.testing.assert_allclose(dv[sl].sum(0), grp, rtol=0, atol=1e-11)
    kc = np.tile(_rng(13).standard_normal(d), (sum(lens), h_kv, 1))
    dq0, _, _ = orc.attn_bwd_ref(q, kc, v, do, cu, 0.5)
    np.testing.assert_allclose(dq0, 0.0, rtol=0, atol=1e-12)


# ----------------------------------------------------------------------------- decode pins

def _parse_nan(x):
    if isinstance(x, list):
        return [_parse_nan(e) for e in x]
    return float(x)


def pin_golden_decode(orc):
    ex = _golden("paged_decode_five_positions")
    o = orc.attn_decode_ref(_arr(ex["q"]), np.array(_parse_nan(ex["k_pool"])),
                            np.array(_parse_nan(ex["v_pool"])), ex["block_table"],
                            ex["ctx_lens"], ex["scale"])
    np.testing.assert_allclose(o, _arr(ex["o"]), rtol=0, atol=1e-12)


def _paged_case(ctx, h_q, h_kv, d, bs, seed, spare=3):
    """Contiguous per-sequence K/V plus the same data scattered into a pool
    through a random block permutation; unused slots and spare blocks hold
    NaN and unused table entries -1."""
    r = _rng(seed)
    nblk = [-(-c // bs) for c in ctx]
    nb = sum(nblk) + spare
    perm = r.permutation(nb)
    kp = np.full((nb, bs, h_kv, d), np.nan)
    vp = np.full((nb, bs, h_kv, d), np.nan)
    table = np.full((len(ctx), max(nblk) + 2), -1, dtype=np.int64)
    ks, vs, pos = [], [], 0
    for b, c in enumerate(ctx):
        K = r.standard_normal((c, h_kv, d))
        V = r.standard_normal((c, h_kv, d))
        ks.append(K)
        vs.append(V)
        for lb in range(nblk[b]):
            phys = perm[pos]
            pos += 1
            table[b, lb] = phys
            n = min(bs, c - lb * bs)
            kp[phys, :n] = K[lb * bs:lb * bs + n]
            vp[phys, :n] = V[lb * bs:lb * bs + n]
    q = r.standard_normal((len(ctx), h_q, d))
    return q, kp, vp, table, np.array(ctx), ks, vs


def pin_decode_last_row(orc):
    """Decode of query q against a context equals the last row of causal
    attention whose final query is q (the final row sees every key); and the
    result is finite although unused slots hold NaN."""
    ctx = [1, 15, 16, 17, 40]
    h_q, h_kv, d, bs, scale = 4, 2, 8, 16, 0.35
    q, kp, vp, table, ctxa, ks, vs = _paged_case(ctx, h_q, h_kv, d, bs, 14)
    o = orc.attn_decode_ref(q, kp, vp, table, ctxa, scale)
    assert np.all(np.isfinite(o))
    r = _rng(15)
    for b, c in enumerate(ctx):
        qs = r.standard_normal((c, h_q, d))
        qs[-1] = q[b]
        of, _ = orc.attn_fwd_ref(qs, ks[b], vs[b], [0, c], scale)
        np.testing.assert_allclose(o[b], of[-1], rtol=0, atol=1e-12)


def pin_decode_torch(orc):
    """PyTorch fp64 SDPA of the one query against the gathered context."""
    ctx = [33, 2, 64]
    h_q, h_kv, d, bs, scale = 8, 4, 16, 16, 0.25
    q, kp, vp, table, ctxa, ks, vs = _paged_case(ctx, h_q, h_kv, d, bs, 16)
    o = orc.attn_decode_ref(q, kp, vp, table, ctxa, scale)
    for b in range(len(ctx)):
        tq = torch.from_numpy(q[b][:, None, :])[None]
        tk = torch.from_numpy(ks[b].transpose(1, 0, 2).copy())[None]
        tv = torch.from_numpy(vs[b].transpose(1, 0, 2).copy())[None]
        ot = F.scaled_dot_product_attention(tq, tk, tv, scale=scale, enable_gqa=True)
        np.testing.assert_allclose(o[b], ot[0, :, 0].numpy(), rtol=0, atol=1e-12)


def pin_decode_block_permutation(orc):
    """Relabelling physical blocks (moving the data and updating the table)
    leaves every output bitwise unchanged."""
    ctx = [20, 50, 3]
    q, kp, vp, table, ctxa, _, _ = _paged_case(ctx, 4, 1, 8, 16, 17)
    o = orc.attn_decode_ref(q, kp, vp, table, ctxa, 0.4)
    perm = _rng(18).permutation(kp.shape[0])
    kp2, vp2 = np.empty_like(kp), np.empty_like(vp)
    kp2[perm], vp2[perm] = kp, vp
    table2 = np.where(table >= 0, perm[np.maximum(table, 0)], -1)
    o2 = orc.attn_decode_ref(q, kp2, vp2, table2, ctxa, 0.4)
    assert np.array_equal(o, o2)


def pin_decode_degenerate(orc):
    """ctx = 1 gives o = v_0 exactly; ctx = 0 gives a zero row."""
    q, kp, vp, table, ctxa, ks, vs = _paged_case([1, 5], 2, 1, 4, 16, 19)
    ctxa = np.array([1, 0])
    o = orc.attn_decode_ref(q, kp, vp, table, ctxa, 0.5)
    for h in range(2):
        assert np.array_equal(o[0, h], vs[0][0, 0])
    assert np.array_equal(o[1], np.zeros_like(o[1]))


PINS = [pin_golden_fwd_bwd, pin_row0_single_key, pin_zero_query, pin_identical_keys,
        pin_rows_sum_to_one, pin_causality, pin_gqa_equals_repeat, pin_varlen_concat,
        pin_torch_sdpa_fwd, pin_torch_autograd_bwd, pin_finite_differences,
        pin_bwd_invariants, pin_golden_decode, pin_decode_last_row, pin_decode_torch,
        pin_decode_block_permutation, pin_decode_degenerate]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin):
    pin(OA)


# ----------------------------------------------------------------------------- planted mistakes

def _mask_without_diagonal(q_rows, keys, row0, scale):
    s = scale * (q_rows @ keys.T)
    qpos = np.arange(row0, row0 + q_rows.shape[0])[:, None]
    kpos = np.arange(keys.shape[0])[None, :]
    return np.where(kpos < qpos, s, -np.inf)


def _mask_leaking_next(q_rows, keys, row0, scale):
    # query i also sees key i + 1 (where that key is among those passed in)
    s = scale * (q_rows @ keys.T)
    qpos = np.arange(row0, row0 + q_rows.shape[0])[:, None]
    kpos = np.arange(keys.shape[0])[None, :]
    return np.where(kpos <= qpos + 1, s, -np.inf)


def _softmax_rows_log2(s):
    m = s.max(axis=1, keepdims=True)
    tot = np.exp(s - m).sum(axis=1)
    lse = m[:, 0] + np.log(tot)
    return np.exp(s - lse[:, None]), m[:, 0] + np.log2(tot)


def _paged_positions_swapped(table_row, ctx, bs):
    t = np.arange(ctx)
    return table_row[t % bs], t // bs


def _gqa_modulo(h, h_q, h_kv):
    return h % h_kv


MUTANTS = [
    ("kv_head_of", _gqa_modulo, [pin_gqa_equals_repeat, pin_torch_sdpa_fwd,
                                 pin_torch_autograd_bwd]),
    ("_masked_scores", _mask_without_diagonal, [pin_row0_single_key, pin_golden_fwd_bwd]),
    ("_masked_scores", _mask_leaking_next, [pin_torch_sdpa_fwd]),
    ("_softmax_rows", _softmax_rows_log2, [pin_golden_fwd_bwd, pin_zero_query,
                                           pin_torch_sdpa_fwd]),
    ("_softmax_grad", lambda p, dp: p * dp, [pin_finite_differences, pin_bwd_invariants,
                                             pin_golden_fwd_bwd]),
    ("_paged_positions", _paged_positions_swapped, [pin_golden_decode, pin_decode_torch]),
]


@pytest.mark.parametrize("name,fn,pins", MUTANTS,
                         ids=[f"{m[0]}:{m[1].__name__}" for m in MUTANTS])
def test_pins_catch_planted_mistake(monkeypatch, name, fn, pins):
    monkeypatch.setattr(OA, name, fn)
    with np.errstate(all="ignore"):
        for pin in pins:
            with pytest.raises(Exception):
                pin(OA)
