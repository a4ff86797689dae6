"""Pins of the oracle's paged prefill and key/value append.

Each pin checks ``attn_prefill_ref`` / ``kv_append_ref`` against something
that is not their own formula: the independently pinned forward and decode
oracles (prefill of one-token chunks is decode; prefill into an empty cache
is the causal forward), PyTorch's CPU fp64 attention routine with an explicit
offset-causal mask, the chunking invariant of causal attention, relabelling of
physical blocks, and a slot-by-slot check of the append. The mutation test at
the bottom plants plausible mistakes into the oracle (on the CPU) and checks
that the pins catch each one.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle.attention as OA


def _rng(seed):
    return np.random.default_rng(seed)


def _cu(lens):
    return np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)


def _pool_case(ctx, h_kv, d, bs, seed, spare=3):
    """Per-sequence contiguous K/V of ``ctx`` tokens and the same data in a
    pool through a random block permutation; unused slots and spare blocks
    hold NaN, unused table entries -1."""
    r = _rng(seed)
    nblk = [-(-c // bs) for c in ctx]
    nb = sum(nblk) + spare
    perm = r.permutation(nb)
    kp = np.full((nb, bs, h_kv, d), np.nan)
    vp = np.full((nb, bs, h_kv, d), np.nan)
    table = np.full((len(ctx), max(nblk + [1]) + 2), -1, dtype=np.int64)
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
    return kp, vp, table, ks, vs


def pin_prefill_one_token_chunks_are_decode(orc):
    """A chunk of one new token per sequence is exactly a decode step."""
    ctx = [1, 15, 16, 17, 40]
    h_q, h_kv, d, bs, scale = 4, 2, 8, 16, 0.35
    kp, vp, table, _, _ = _pool_case(ctx, h_kv, d, bs, 31)
    q = _rng(32).standard_normal((len(ctx), h_q, d))
    o, lse = orc.attn_prefill_ref(q, kp, vp, table, ctx, _cu([1] * len(ctx)), scale)
    od = orc.attn_decode_ref(q, kp, vp, table, ctx, scale)
    np.testing.assert_allclose(o, od, rtol=0, atol=1e-12)
    assert np.all(np.isfinite(lse))


def pin_prefill_empty_cache_is_forward(orc):
    """With no cached tokens (ctx = q_len) every sequence is plain causal
    attention over its own tokens."""
    lens = [5, 1, 33, 17]
    h_q, h_kv, d, bs, scale = 6, 2, 8, 16, 0.3
    kp, vp, table, ks, vs = _pool_case(lens, h_kv, d, bs, 33)
    cu = _cu(lens)
    q = _rng(34).standard_normal((int(cu[-1]), h_q, d))
    o, lse = orc.attn_prefill_ref(q, kp, vp, table, lens, cu, scale)
    of, lf = orc.attn_fwd_ref(q, np.concatenate(ks), np.concatenate(vs), cu, scale)
    np.testing.assert_allclose(o, of, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lf, rtol=0, atol=1e-12)


def pin_prefill_torch(orc):
    """PyTorch fp64 SDPA of each chunk against its gathered context with an
    explicit mask: new token i sees positions 0 .. ctx - q_len + i."""
    ctx = [40, 19, 64, 7]
    qlen = [9, 19, 1, 3]
    h_q, h_kv, d, bs, scale = 8, 4, 16, 16, 0.25
    kp, vp, table, ks, vs = _pool_case(ctx, h_kv, d, bs, 35)
    cu = _cu(qlen)
    q = _rng(36).standard_normal((int(cu[-1]), h_q, d))
    o, lse = orc.attn_prefill_ref(q, kp, vp, table, ctx, cu, scale)
    for b, (c, L) in enumerate(zip(ctx, qlen)):
        tq = torch.from_numpy(q[cu[b]:cu[b + 1]].transpose(1, 0, 2).copy())[None]
        tk = torch.from_numpy(ks[b].transpose(1, 0, 2).copy())[None]
        tv = torch.from_numpy(vs[b].transpose(1, 0, 2).copy())[None]
        allow = torch.arange(c)[None, :] <= (c - L + torch.arange(L))[:, None]
        ot = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=allow, scale=scale,
                                            enable_gqa=True)
        np.testing.assert_allclose(o[cu[b]:cu[b + 1]], ot[0].transpose(0, 1).numpy(),
                                   rtol=0, atol=1e-12)
        s = scale * np.einsum("hd,khd->hk", q[cu[b] + L - 1], np.repeat(ks[b], h_q // h_kv, 1))
        np.testing.assert_allclose(lse[:, cu[b] + L - 1], np.log(np.exp(s).sum(1)),
                                   rtol=0, atol=1e-10)


def pin_prefill_chunking(orc):
    """Causal attention does not depend on how the new tokens are chunked:
    one chunk of c tokens equals a first chunk of c1 tokens (context c1)
    followed by a second chunk of c - c1 tokens (context c)."""
    c, c1 = 45, 18
    h_q, h_kv, d, bs, scale = 4, 1, 8, 16, 0.4
    kp, vp, table, _, _ = _pool_case([c], h_kv, d, bs, 37)
    q = _rng(38).standard_normal((c, h_q, d))
    o, lse = orc.attn_prefill_ref(q, kp, vp, table, [c], [0, c], scale)
    oa, la = orc.attn_prefill_ref(q[:c1], kp, vp, table, [c1], [0, c1], scale)
    ob, lb = orc.attn_prefill_ref(q[c1:], kp, vp, table, [c], [0, c - c1], scale)
    np.testing.assert_allclose(o, np.concatenate([oa, ob]), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, np.concatenate([la, lb], axis=1), rtol=0, atol=1e-12)


def pin_prefill_block_permutation(orc):
    """Relabelling physical blocks leaves every output bitwise unchanged."""
    ctx, qlen = [20, 50, 3], [4, 50, 2]
    kp, vp, table, _, _ = _pool_case(ctx, 1, 8, 16, 39)
    cu = _cu(qlen)
    q = _rng(40).standard_normal((int(cu[-1]), 4, 8))
    o, lse = orc.attn_prefill_ref(q, kp, vp, table, ctx, cu, 0.4)
    perm = _rng(41).permutation(kp.shape[0])
    kp2, vp2 = np.empty_like(kp), np.empty_like(vp)
    kp2[perm], vp2[perm] = kp, vp
    table2 = np.where(table >= 0, perm[np.maximum(table, 0)], -1)
    o2, lse2 = orc.attn_prefill_ref(q, kp2, vp2, table2, ctx, cu, 0.4)
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2)


def pin_append_slots(orc):
    """Append writes new token i of sequence b to slot t % 16 of block
    table[b][t // 16], t = ctx - q_len + i (checked slot by slot), and leaves
    every other slot bitwise as it was (NaN included)."""
    ctx, qlen = [20, 16, 33, 5], [4, 16, 1, 0]
    h_kv, d, bs = 2, 4, 16
    kp, vp, table, _, _ = _pool_case(ctx, h_kv, d, bs, 42)
    cu = _cu(qlen)
    r = _rng(43)
    kn = r.standard_normal((int(cu[-1]), h_kv, d))
    vn = r.standard_normal((int(cu[-1]), h_kv, d))
    kp2, vp2 = orc.kv_append_ref(kp, vp, kn, vn, cu, table, ctx)
    written = np.zeros(kp.shape[:2], dtype=bool)
    for b, (c, L) in enumerate(zip(ctx, qlen)):
        for i in range(L):
            t = c - L + i
            blk, slot = table[b][t // bs], t % bs
            assert np.array_equal(kp2[blk, slot], kn[cu[b] + i])
            assert np.array_equal(vp2[blk, slot], vn[cu[b] + i])
            written[blk, slot] = True
    same_k = (kp2[~written] == kp[~written]) | (np.isnan(kp2[~written]) & np.isnan(kp[~written]))
    same_v = (vp2[~written] == vp[~written]) | (np.isnan(vp2[~written]) & np.isnan(vp[~written]))
    assert same_k.all() and same_v.all()
    assert written.sum() == sum(qlen)


def pin_append_then_prefill_is_forward(orc):
    """Appending whole sequences to an empty (NaN) pool and then prefilling
    them equals the causal forward on the contiguous data."""
    lens = [17, 3, 40]
    h_q, h_kv, d, bs, scale = 4, 2, 8, 16, 0.3
    nblk = [-(-c // bs) for c in lens]
    perm = _rng(44).permutation(sum(nblk) + 2)
    table = np.full((len(lens), max(nblk)), -1, dtype=np.int64)
    pos = 0
    for b, n in enumerate(nblk):
        table[b, :n] = perm[pos:pos + n]
        pos += n
    kp = np.full((len(perm), bs, h_kv, d), np.nan)
    vp = np.full_like(kp, np.nan)
    cu = _cu(lens)
    r = _rng(45)
    q = r.standard_normal((int(cu[-1]), h_q, d))
    k = r.standard_normal((int(cu[-1]), h_kv, d))
    v = r.standard_normal((int(cu[-1]), h_kv, d))
    kp, vp = orc.kv_append_ref(kp, vp, k, v, cu, table, lens)
    o, lse = orc.attn_prefill_ref(q, kp, vp, table, lens, cu, scale)
    of, lf = orc.attn_fwd_ref(q, k, v, cu, scale)
    np.testing.assert_allclose(o, of, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lf, rtol=0, atol=1e-12)


PINS = [pin_prefill_one_token_chunks_are_decode, pin_prefill_empty_cache_is_forward,
        pin_prefill_torch, pin_prefill_chunking, pin_prefill_block_permutation,
        pin_append_slots, pin_append_then_prefill_is_forward]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_prefill_oracle_pin(pin):
    pin(OA)


def _offset_one_late(ctx, q_len):
    return ctx - q_len + 1 if q_len < ctx else ctx - q_len


def _offset_from_start(ctx, q_len):
    return 0


MUTANTS = [
    ("_chunk_offset", _offset_one_late, [pin_prefill_torch, pin_prefill_chunking,
                                         pin_append_slots]),
    ("_chunk_offset", _offset_from_start, [pin_prefill_one_token_chunks_are_decode,
                                           pin_prefill_torch, pin_append_slots]),
]


@pytest.mark.parametrize("name,fn,pins", MUTANTS,
                         ids=[f"{m[0]}:{m[1].__name__}" for m in MUTANTS])
def test_prefill_pins_catch_planted_mistake(monkeypatch, name, fn, pins):
    monkeypatch.setattr(OA, name, fn)
    with np.errstate(all="ignore"):
        for pin in pins:
            with pytest.raises(Exception):
                pin(OA)
