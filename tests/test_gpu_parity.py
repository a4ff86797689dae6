"""GPU parity: the HIP kernels (through the C ABI) against the fp64 oracle.

Every case draws seeded fp16 inputs on the CPU, runs the library on the GPU
and compares with the oracle on the same inputs. Small cases are compared
in full; the full-size workloads run exactly as the benchmark launches them
and are compared on sampled (sequence, KV-head group) slices.
"""
import math

import numpy as np
import pytest
import torch

from parity import (GRAD_TOL, O_TOL, W, attn, check_bwd, check_decode, check_fwd, dev,
                    gpu_bwd, gpu_decode, gpu_fwd, rel_l2)
from oracle import attn_fwd_ref

pytestmark = pytest.mark.gpu

# Lengths around the 16/32/64/128 tile edges plus an empty sequence.
EDGE_LENS = [1, 2, 15, 16, 17, 31, 32, 33, 63, 64, 65, 127, 128, 129, 300, 0, 511]

HEAD_CONFIGS = [  # (h_q, h_kv, d)
    (2, 1, 64), (2, 1, 128), (4, 4, 128), (8, 2, 64), (8, 2, 128), (6, 2, 128),
    (16, 2, 128), (16, 1, 64), (12, 4, 64),
]


@pytest.mark.parametrize("h_q,h_kv,d", HEAD_CONFIGS, ids=lambda x: str(x))
def test_fwd_bwd_edge_lengths(gpu, h_q, h_kv, d):
    name = f"edge hq{h_q} hkv{h_kv} d{d}"
    inp = W.make_train_inputs(EDGE_LENS, h_q, h_kv, d, seed=2000 + 31 * h_q + h_kv + d)
    dd = dev(inp, gpu)
    o, lse = gpu_fwd(dd)
    torch.cuda.synchronize()
    check_fwd(name, inp, o, lse)
    dq, dk, dv = gpu_bwd(dd, o, lse)
    torch.cuda.synchronize()
    check_bwd(name, inp, dq, dk, dv)


def _random_cases(n, seed):
    """Seeded random varlen batches: 1-5 sequences of 0-400 tokens, KV heads
    1-4, group size 1-8 (including non powers of two) and d 64 or 128."""
    g = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        lens = [int(x) for x in g.integers(0, 401, size=int(g.integers(1, 6)))]
        h_kv = int(g.choice([1, 2, 4]))
        G = int(g.choice([1, 2, 3, 4, 5, 8]))
        d = int(g.choice([64, 128]))
        cases.append((lens, G * h_kv, h_kv, d, 3000 + i))
    return cases


@pytest.mark.parametrize("lens,h_q,h_kv,d,seed", _random_cases(10, 77),
                         ids=lambda x: str(x))
def test_random_shapes(gpu, lens, h_q, h_kv, d, seed):
    """Forward and backward on random ragged batches, every sequence and KV
    group compared with the oracle."""
    name = f"random {lens} hq{h_q} hkv{h_kv} d{d}"
    inp = W.make_train_inputs(lens, h_q, h_kv, d, seed=seed)
    if inp["total_tokens"] == 0:
        pytest.skip("empty batch (covered by the zero-length test)")
    dd = dev(inp, gpu)
    o, lse = gpu_fwd(dd)
    dq, dk, dv = gpu_bwd(dd, o, lse)
    torch.cuda.synchronize()
    check_fwd(name, inp, o, lse)
    check_bwd(name, inp, dq, dk, dv)


@pytest.mark.parametrize("h_q,h_kv,d", [(2, 2, 128), (6, 2, 64), (16, 1, 64), (8, 1, 128)],
                         ids=lambda x: str(x))
def test_long_batch_group_sizes(gpu, h_q, h_kv, d):
    """A batch longer than 4096 keys takes the eight-wave forward (shorter
    ones the four-wave shape, covered above): group sizes 1, 3, 16 and 8 and
    both head dims, a sequence just past the threshold plus a short one and
    an edge length, compared in full with the oracle."""
    lens = [4100, 65, 300]
    name = f"long hq{h_q} hkv{h_kv} d{d}"
    inp = W.make_train_inputs(lens, h_q, h_kv, d, seed=2300 + h_q + 7 * h_kv + d)
    dd = dev(inp, gpu)
    o, lse = gpu_fwd(dd)
    dq, dk, dv = gpu_bwd(dd, o, lse)
    torch.cuda.synchronize()
    check_fwd(name, inp, o, lse)
    check_bwd(name, inp, dq, dk, dv)


@pytest.mark.parametrize("n_seqs,h_q,h_kv,d,longest", [
    (150, 4, 2, 64, 0), (256, 8, 2, 128, 0), (257, 2, 1, 64, 0), (256, 2, 1, 64, 4200)],
    ids=lambda x: str(x))
def test_many_unequal_sequences(gpu, n_seqs, h_q, h_kv, d, longest):
    """Many short sequences and four long ones: the work-sorted lists of
    query and key tiles span several groups of 64 sequences (256 is the most
    they take; 257 falls back to the static order). With one sequence of
    4200 tokens the forward walks its list in the eight-wave shape, the dS
    blocks would pass their 4 GiB bound (so the backward recomputes), and
    the key-tile list passes its size bound (256 sequences x 3 groups of 64
    query blocks), so dK/dV falls back to the static order. Compared in
    full."""
    g = np.random.default_rng(2400 + n_seqs + longest)
    lens = [int(x) for x in g.integers(0, 41, size=n_seqs)]
    for i in g.choice(n_seqs, size=4, replace=False):
        lens[int(i)] = int(g.integers(300, 700))
    if longest:
        lens[int(g.integers(0, n_seqs))] = longest
    name = f"{n_seqs} seqs hq{h_q} hkv{h_kv} d{d} longest {max(lens)}"
    inp = W.make_train_inputs(lens, h_q, h_kv, d, seed=2400 + n_seqs + longest)
    dd = dev(inp, gpu)
    o, lse = gpu_fwd(dd)
    dq, dk, dv = gpu_bwd(dd, o, lse)
    torch.cuda.synchronize()
    check_fwd(name, inp, o, lse)
    check_bwd(name, inp, dq, dk, dv)


def test_tiny_workload(gpu):
    inp = W.workload_inputs("tiny")
    dd = dev(inp, gpu)
    o, lse = gpu_fwd(dd)
    dq, dk, dv = gpu_bwd(dd, o, lse)
    torch.cuda.synchronize()
    check_fwd("tiny", inp, o, lse)
    check_bwd("tiny", inp, dq, dk, dv)
    # Row 0 of every head sees one key: its output is v_0 exactly.
    assert torch.equal(o[0].cpu(), inp["v"][0].repeat_interleave(2, 0))


def test_debug_validate_mode(gpu, monkeypatch):
    """With ATTN_DEBUG_VALIDATE=1 the binding checks host copies of the index
    arrays before each launch; valid inputs give bitwise the same results.
    (Invalid contents are covered on the CPU: they must never reach a kernel.)"""
    inp = W.make_train_inputs([100, 1, 64], 4, 2, 64, seed=2200)
    dd = dev(inp, gpu)
    o0, lse0 = gpu_fwd(dd)
    g0 = gpu_bwd(dd, o0, lse0)
    dec = W.make_decode_inputs([1, 17, 40], 4, 2, 64, seed=2201)
    dd_dec = dev(dec, gpu)
    od0 = gpu_decode(dd_dec)
    monkeypatch.setenv("ATTN_DEBUG_VALIDATE", "1")
    o1, lse1 = gpu_fwd(dd)
    g1 = gpu_bwd(dd, o1, lse1)
    od1 = gpu_decode(dd_dec)
    torch.cuda.synchronize()
    assert torch.equal(o0, o1) and torch.equal(lse0, lse1)
    assert all(torch.equal(a, b) for a, b in zip(g0, g1))
    assert torch.equal(od0, od1)


def test_isolated_bwd_from_oracle_forward(gpu):
    """The backward fed the oracle's O (rounded to fp16) and LSE."""
    inp = W.make_train_inputs([200, 77, 129], 8, 2, 128, seed=2100)
    o_ref, lse_ref = attn_fwd_ref(inp["q"].numpy(), inp["k"].numpy(), inp["v"].numpy(),
                                  inp["cu_seqlens"].numpy(), inp["scale"])
    dd = dev(inp, gpu)
    o = torch.from_numpy(o_ref).half().to(gpu)
    lse = torch.from_numpy(lse_ref).float().to(gpu)
    dq, dk, dv = gpu_bwd(dd, o, lse)
    torch.cuda.synchronize()
    check_bwd("isolated bwd", inp, dq, dk, dv)


@pytest.mark.parametrize("workload,seqs,groups", [
    ("qwen3_train", [0, 7], [0, 5]),
    ("grpo_varlen", None, [3]),
    ("long_context", [2], [6]),
    ("long_context_tp8", [1], [0]),
])
def test_workload_sampled(gpu, workload, seqs, groups):
    """Full-size workload on the GPU (the benchmark's launch), compared with the
    oracle on sampled sequences and KV groups."""
    inp = W.workload_inputs(workload)
    if seqs is None:  # the longest and the shortest sequence of the batch
        lens = inp["seqlens"]
        seqs = [int(np.argmax(lens)), int(np.argmin(lens))]
    dd = dev(inp, gpu)
    o, lse = gpu_fwd(dd)
    dq, dk, dv = gpu_bwd(dd, o, lse)
    torch.cuda.synchronize()
    for t in (o, lse, dq, dk, dv):
        assert torch.isfinite(t).all()
    check_fwd(workload, inp, o, lse, seqs, groups)
    check_bwd(workload, inp, dq, dk, dv, seqs, groups)


@pytest.mark.parametrize("workload", ["qwen3_train", "long_context"])
def test_workload_gradient_sums(gpu, workload):
    """Properties that hold at any size, over every (sequence, KV head):
    sum_j dK_j = 0 (rows of dS sum to zero) and sum_j dV_j equals the sum of
    dO over the group's heads and rows (rows of P sum to one)."""
    inp = W.workload_inputs(workload)
    dd = dev(inp, gpu)
    o, lse = gpu_fwd(dd)
    dq, dk, dv = gpu_bwd(dd, o, lse)
    torch.cuda.synchronize()
    cu = inp["cu_seqlens"].tolist()
    h_q, h_kv = inp["h_q"], inp["h_kv"]
    G = h_q // h_kv
    dk64, dv64 = dk.double().cpu(), dv.double().cpu()
    do64 = inp["dout"].double()
    for b in range(len(cu) - 1):
        s, e = cu[b], cu[b + 1]
        want = do64[s:e].view(e - s, h_kv, G, -1).sum(dim=(0, 2))
        got = dv64[s:e].sum(0)
        assert rel_l2(got.numpy(), want.numpy()) <= GRAD_TOL
        # dK sums to zero up to rounding: compare with the size of its terms.
        scale_ref = dk64[s:e].abs().sum(0).mean()
        assert float(dk64[s:e].sum(0).abs().max() / scale_ref) <= GRAD_TOL


def test_zero_length_and_empty_batches(gpu):
    inp = W.make_train_inputs([0, 5, 0, 70, 0], 4, 2, 64, seed=2200)
    dd = dev(inp, gpu)
    o, lse = gpu_fwd(dd)
    dq, dk, dv = gpu_bwd(dd, o, lse)
    torch.cuda.synchronize()
    check_fwd("zero-length seqs", inp, o, lse)
    check_bwd("zero-length seqs", inp, dq, dk, dv)
    # An empty batch is a valid no-op.
    empty = W.make_train_inputs([0, 0], 4, 2, 128, seed=2201)
    de = dev(empty, gpu)
    o, lse = attn.fwd(de["q"], de["k"], de["v"], de["cu_seqlens"], max_seqlen=0)
    dq, dk, dv = attn.bwd(de["q"], de["k"], de["v"], o, lse, de["dout"], de["cu_seqlens"],
                          max_seqlen=0)
    torch.cuda.synchronize()
    assert o.numel() == 0 and dq.numel() == 0


def test_fwd_bitwise_reproducible(gpu):
    inp = W.make_train_inputs([1000, 333, 64], 16, 8, 128, seed=2300)
    dd = dev(inp, gpu)
    o1, l1 = gpu_fwd(dd)
    o2, l2 = gpu_fwd(dd)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def _guarded(shape, dtype, device, fill, pad=4096):
    n = math.prod(shape)
    buf = torch.full((n + 2 * pad,), fill, dtype=dtype, device=device)
    return buf, buf[pad:pad + n].view(shape), pad


def _untouched(buf, pad, n, fill):
    return bool((buf[:pad] == fill).all()) and bool((buf[pad + n:] == fill).all())


def test_outputs_stay_in_bounds(gpu):
    """Canaries around every output buffer stay untouched."""
    inp = W.make_train_inputs([129, 1, 64, 250], 8, 2, 128, seed=2400)
    dd = dev(inp, gpu)
    T, h_q, d = inp["q"].shape
    h_kv = inp["k"].shape[1]
    ob, o, po = _guarded((T, h_q, d), torch.float16, gpu, 7.0)
    lb, lse, pl = _guarded((h_q, T), torch.float32, gpu, 7.0)
    attn.fwd(dd["q"], dd["k"], dd["v"], dd["cu_seqlens"], dd["scale"], o=o, lse=lse,
             max_seqlen=dd["max_seqlen"])
    qb, dq, _ = _guarded((T, h_q, d), torch.float16, gpu, 7.0)
    kb, dk, _ = _guarded((T, h_kv, d), torch.float16, gpu, 7.0)
    vb, dv, _ = _guarded((T, h_kv, d), torch.float16, gpu, 7.0)
    attn.bwd(dd["q"], dd["k"], dd["v"], o, lse, dd["dout"], dd["cu_seqlens"], dd["scale"],
             dq=dq, dk=dk, dv=dv, max_seqlen=dd["max_seqlen"])
    torch.cuda.synchronize()
    for buf, t in ((ob, o), (lb, lse), (qb, dq), (kb, dk), (vb, dv)):
        assert _untouched(buf, 4096, t.numel(), 7.0)
    check_fwd("guarded", inp, o, lse)
    check_bwd("guarded", inp, dq, dk, dv)


# ----------------------------------------------------------------------------- decode

DECODE_CTX = [1, 15, 16, 17, 100, 511, 512, 513, 1500, 0, 2049]


@pytest.mark.parametrize("h_q,h_kv,d", [(2, 1, 64), (16, 8, 128), (8, 2, 128), (8, 8, 64),
                                        (16, 2, 128), (6, 3, 64)], ids=lambda x: str(x))
def test_decode_edge_contexts(gpu, h_q, h_kv, d):
    """Ragged contexts around block and split edges, with NaN in every unused
    pool slot and spare block (they must never reach the output)."""
    inp = W.make_decode_inputs(DECODE_CTX, h_q, h_kv, d, seed=2500 + h_q + d, spare_blocks=7)
    inp = W.poison_unused(inp)
    dd = dev(inp, gpu)
    o = gpu_decode(dd)
    torch.cuda.synchronize()
    check_decode(f"decode edge hq{h_q} hkv{h_kv} d{d}", inp, o)
    assert torch.equal(o[DECODE_CTX.index(0)].cpu(), torch.zeros(h_q, d, dtype=torch.float16))


def test_decode_workload(gpu):
    """The paged-decode workload in full (256 sequences, ctx up to 4096)."""
    inp = W.decode_workload_inputs()
    dd = dev(inp, gpu)
    o = gpu_decode(dd)
    torch.cuda.synchronize()
    check_decode("paged_decode", inp, o)


def test_decode_block_permutation_gpu(gpu):
    """Relabelling the physical blocks gives bitwise the same GPU output."""
    inp = W.make_decode_inputs([700, 33, 1024], 16, 8, 128, seed=2600, spare_blocks=3)
    dd = dev(inp, gpu)
    o1 = gpu_decode(dd)
    g = torch.Generator().manual_seed(2601)
    perm = torch.randperm(inp["num_blocks"], generator=g)
    kp = torch.empty_like(inp["k_pool"])
    vp = torch.empty_like(inp["v_pool"])
    kp[perm] = inp["k_pool"]
    vp[perm] = inp["v_pool"]
    bt = inp["block_table"].clone().long()
    bt = torch.where(bt >= 0, perm[bt.clamp(min=0)], bt).int()
    d2 = dict(dd)
    d2.update(k_pool=kp.to(gpu), v_pool=vp.to(gpu), block_table=bt.to(gpu))
    o2 = gpu_decode(d2)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    check_decode("decode permuted", inp, o1)


def test_decode_clamps_bad_indices(gpu):
    """Contexts outside [0, max_ctx_len] and table entries outside
    [0, num_blocks) are clamped inside the kernels: the output equals, bit for
    bit, the decode of the clamped (valid) inputs, which matches the oracle.
    The index math was checked on the CPU first (every access in bounds)."""
    inp = W.make_decode_inputs([300, 40, 700, 64], 16, 8, 128, seed=2700, max_blocks=50,
                               spare_blocks=2)
    nb = inp["num_blocks"]
    max_ctx = 800  # 50 blocks of 16
    bad_ctx = torch.tensor([300, -5, 900, 64], dtype=torch.int32)
    bad_bt = inp["block_table"].clone()
    bad_bt[0, 2] = -7
    bad_bt[0, 5] = nb + 3
    bad_bt[3, 1] = 2 ** 31 - 1
    good_ctx = torch.tensor([300, 0, 800, 64], dtype=torch.int32)
    good_bt = bad_bt.clamp(0, nb - 1)
    good = dict(inp, ctx_lens=good_ctx, block_table=good_bt, max_ctx=max_ctx)
    bad = dict(inp, ctx_lens=bad_ctx, block_table=bad_bt, max_ctx=max_ctx)
    o_bad = gpu_decode(dev(bad, gpu))
    o_good = gpu_decode(dev(good, gpu))
    torch.cuda.synchronize()
    assert torch.equal(o_bad, o_good)
    assert torch.equal(o_bad[1].cpu(), torch.zeros(16, 128, dtype=torch.float16))
    check_decode("decode clamped", good, o_good)
