"""GPU parity of the chunked prefill over the paged cache: attn_kv_append and
attn_prefill_paged (through the C ABI) against the fp64 oracle.

The append is pure data movement and must match the oracle bit for bit
(NaN-poisoned unused slots included). The prefill is compared with the
oracle's prefill over the oracle-appended pools: O max abs <= 2e-3, LSE max
abs <= 1e-4. With no cached tokens the prefill must reproduce attn_fwd on
the contiguous data bit for bit (same kernel, only the addressing differs).
"""
import numpy as np
import pytest
import torch

from parity import LSE_TOL, O_TOL, W, attn, max_abs
from oracle import attn_prefill_ref, kv_append_ref

pytestmark = pytest.mark.gpu

# (cached tokens, new tokens) per sequence: chunks of 0, 1 and 16/32/64/128
# tile edges, empty caches, block-edge contexts and one long cache.
PRIOR = [0, 0, 5, 15, 16, 17, 100, 300, 0, 1000, 64, 511, 3, 31]
NEW = [1, 17, 1, 17, 16, 63, 64, 129, 300, 1, 65, 0, 128, 33]

HEAD_CONFIGS = [(16, 8, 128), (8, 2, 64), (4, 4, 128), (12, 4, 64), (2, 1, 128), (6, 2, 128)]


def _np(t):
    return t.numpy() if isinstance(t, torch.Tensor) else t


def _oracle(inp, seqs=None):
    """Oracle append of the whole batch, then the oracle prefill of the
    sampled sequences (each alone). Returns {b: (o, lse)}, the pools."""
    kp, vp = kv_append_ref(_np(inp["k_pool"]), _np(inp["v_pool"]), _np(inp["k_new"]),
                           _np(inp["v_new"]), _np(inp["cu_q"]), _np(inp["block_table"]),
                           _np(inp["ctx_lens"]))
    cu = inp["cu_q"].tolist()
    out = {}
    for b in (range(inp["n"]) if seqs is None else seqs):
        s, e = cu[b], cu[b + 1]
        if e == s:
            continue
        o, lse = attn_prefill_ref(_np(inp["q"])[s:e], kp, vp, _np(inp["block_table"])[b:b + 1],
                                  [int(inp["ctx_lens"][b])], [0, e - s], inp["scale"])
        out[b] = (o, lse)
    return out, kp, vp


def _gpu(inp, device, with_lse=True):
    d = {k: (v.to(device) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    attn.kv_append(d["k_new"], d["v_new"], d["cu_q"], d["block_table"], d["ctx_lens"],
                   d["k_pool"], d["v_pool"], max_ctx_len=inp["max_ctx"],
                   max_q_len=inp["max_q_len"])
    o, lse = attn.prefill_paged(d["q"], d["k_pool"], d["v_pool"], d["block_table"],
                                d["ctx_lens"], d["cu_q"], inp["scale"], with_lse=with_lse,
                                max_ctx_len=inp["max_ctx"], max_q_len=inp["max_q_len"])
    torch.cuda.synchronize()
    return d, o, lse


def _check(name, inp, o, lse, ref):
    cu = inp["cu_q"].tolist()
    o = o.float().cpu().numpy()
    lse = lse.cpu().numpy()
    worst_o = worst_l = 0.0
    for b, (o_ref, lse_ref) in ref.items():
        s, e = cu[b], cu[b + 1]
        worst_o = max(worst_o, max_abs(o[s:e], o_ref))
        worst_l = max(worst_l, max_abs(lse[:, s:e], lse_ref))
    print(f"{name}: O max abs {worst_o:.2e}, LSE max abs {worst_l:.2e}", flush=True)
    assert worst_o <= O_TOL, f"{name}: O error {worst_o}"
    assert worst_l <= LSE_TOL, f"{name}: LSE error {worst_l}"


def _same_bits(a, b):
    return torch.equal(a.cpu().view(torch.int16), torch.as_tensor(b).view(torch.int16))


@pytest.mark.parametrize("h_q,h_kv,d", HEAD_CONFIGS, ids=lambda x: str(x))
def test_append_and_prefill_edge_cases(gpu, h_q, h_kv, d):
    inp = W.poison_unused_prefill(W.make_prefill_inputs(PRIOR, NEW, h_q, h_kv, d,
                                                        seed=5000 + 7 * h_q + d,
                                                        spare_blocks=3))
    name = f"prefill hq{h_q} hkv{h_kv} d{d}"
    print(name, flush=True)
    dd, o, lse = _gpu(inp, gpu)
    ref, kp, vp = _oracle(inp)
    # The append moves bytes: bitwise equal pools, poisoned slots included.
    assert _same_bits(dd["k_pool"], torch.from_numpy(kp)), "k_pool differs"
    assert _same_bits(dd["v_pool"], torch.from_numpy(vp)), "v_pool differs"
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()
    _check(name, inp, o, lse, ref)


def test_prefill_without_cache_is_the_forward_bitwise(gpu):
    """No cached tokens: every sequence is the plain causal forward over its
    chunk, and the paged kernel reproduces attn_fwd bit for bit."""
    lens = [1, 17, 64, 65, 300, 129, 0, 33]
    inp = W.make_prefill_inputs([0] * len(lens), lens, 16, 8, 128, seed=5100)
    _, o, lse = _gpu(inp, gpu)
    q, k, v, cu = (inp[n].to(gpu) for n in ("q", "k_new", "v_new", "cu_q"))
    of, lf = attn.fwd(q, k, v, cu, inp["scale"], max_seqlen=inp["max_q_len"])
    torch.cuda.synchronize()
    assert torch.equal(o, of)
    assert torch.equal(lse, lf)


def test_prefill_lse_optional(gpu):
    """With lse = NULL the kernel skips the LSE store; O is unchanged."""
    inp = W.make_prefill_inputs([40, 0, 300], [20, 64, 100], 8, 2, 128, seed=5200)
    _, o1, lse1 = _gpu(inp, gpu, with_lse=True)
    _, o2, lse2 = _gpu(inp, gpu, with_lse=False)
    assert lse2 is None
    assert torch.equal(o1, o2)


def test_prefill_workload_sampled(gpu):
    """The full paged_prefill workload, launched as the benchmark launches
    it, compared on sampled sequences."""
    inp = W.prefill_workload_inputs("paged_prefill")
    _, o, lse = _gpu(inp, gpu)
    ref, _, _ = _oracle(inp, seqs=[0, 7, 13, 22, 31])
    _check("paged_prefill sampled", inp, o, lse, ref)


def test_prefill_empty_batches(gpu):
    """No sequences, or sequences without new tokens: nothing is launched and
    the call succeeds."""
    inp = W.make_prefill_inputs([5, 17], [0, 0], 4, 2, 64, seed=5300)
    d = {k: (v.to(gpu) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    before = d["k_pool"].clone()
    attn.kv_append(d["k_new"], d["v_new"], d["cu_q"], d["block_table"], d["ctx_lens"],
                   d["k_pool"], d["v_pool"], max_ctx_len=inp["max_ctx"], max_q_len=0)
    o, lse = attn.prefill_paged(d["q"], d["k_pool"], d["v_pool"], d["block_table"],
                                d["ctx_lens"], d["cu_q"], max_ctx_len=inp["max_ctx"],
                                max_q_len=0)
    torch.cuda.synchronize()
    assert o.shape[0] == 0 and lse.shape[1] == 0
    assert torch.equal(before, d["k_pool"])


def _random_prefill_cases(n, seed):
    """Seeded random chunked-prefill batches: 1-6 sequences, cached 0-700,
    new 0-300 tokens, KV heads 1-4, group size 1-8, d 64 or 128."""
    g = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        m = int(g.integers(1, 7))
        prior = [int(x) for x in g.integers(0, 701, size=m)]
        new = [int(x) for x in g.integers(0, 301, size=m)]
        if sum(new) == 0:
            new[0] = 1
        h_kv = int(g.choice([1, 2, 4]))
        G = int(g.choice([1, 2, 3, 4, 8]))
        d = int(g.choice([64, 128]))
        cases.append((prior, new, G * h_kv, h_kv, d, 5400 + i))
    return cases


@pytest.mark.parametrize("h_q,h_kv,d", [(16, 8, 128), (8, 2, 64)], ids=lambda x: str(x))
def test_prefill_long_context(gpu, h_q, h_kv, d):
    """Contexts past 4096 keys take the eight-wave prefill (the cases above,
    all shorter, take the four-wave shape): a cache of 4200 and one ending
    just past the threshold, next to short and empty caches."""
    prior, new = [4200, 4090, 0, 300], [33, 10, 17, 129]
    inp = W.poison_unused_prefill(W.make_prefill_inputs(prior, new, h_q, h_kv, d,
                                                        seed=5600 + h_q + d, spare_blocks=2))
    name = f"prefill long hq{h_q} hkv{h_kv} d{d}"
    print(name, flush=True)
    dd, o, lse = _gpu(inp, gpu)
    ref, kp, vp = _oracle(inp)
    assert _same_bits(dd["k_pool"], torch.from_numpy(kp))
    assert _same_bits(dd["v_pool"], torch.from_numpy(vp))
    _check(name, inp, o, lse, ref)


@pytest.mark.parametrize("prior,new,h_q,h_kv,d,seed", _random_prefill_cases(8, 91),
                         ids=lambda x: str(x))
def test_prefill_random_batches(gpu, prior, new, h_q, h_kv, d, seed):
    inp = W.poison_unused_prefill(W.make_prefill_inputs(prior, new, h_q, h_kv, d, seed=seed,
                                                        spare_blocks=2))
    name = f"prefill random seed {seed}"
    print(name, flush=True)
    dd, o, lse = _gpu(inp, gpu)
    ref, kp, vp = _oracle(inp)
    assert _same_bits(dd["k_pool"], torch.from_numpy(kp))
    _check(name, inp, o, lse, ref)


def test_prefill_one_token_chunks_match_decode(gpu):
    """One new token per sequence: the prefill (forward kernel, paged) and the
    decode (split-K gather) are different kernels computing the same row;
    both must agree within the output bar."""
    prior = [0, 15, 16, 100, 1000, 2047]
    inp = W.make_prefill_inputs(prior, [1] * len(prior), 16, 8, 128, seed=5500)
    dd, o, _ = _gpu(inp, gpu)
    od = attn.decode_paged(dd["q"], dd["k_pool"], dd["v_pool"], dd["block_table"],
                           dd["ctx_lens"], inp["scale"], max_ctx_len=inp["max_ctx"])
    torch.cuda.synchronize()
    assert max_abs(o.float().cpu().numpy(), od.float().cpu().numpy()) <= 2 * O_TOL
