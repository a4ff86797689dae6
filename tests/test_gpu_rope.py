"""GPU parity of the RoPE entry points (through the C ABI) against the fp64
oracle.

The kernels rotate in fp64 and round once to fp16, and the oracle rounds its
fp64 rotation to fp16 the same way, so rotated tensors must match bit for
bit (same fp32 tables on both sides: the oracle's, rounded to fp32). The
table kernel itself is compared with the oracle's tables within one fp32
unit in the last place (its fp64 pow / cos / sin are not the CPU's). Every
entry point that rotates must give the same bits as the standalone pass;
attention on rotated inputs keeps the attention bars (O max abs <= 2e-3,
LSE max abs <= 1e-4, gradients rel L2 <= 1e-2).
"""
import numpy as np
import pytest
import torch

from parity import GRAD_TOL, LSE_TOL, O_TOL, W, attn, max_abs, rel_l2
from oracle import (attn_bwd_ref, attn_fwd_ref, attn_prefill_ref, chunk_positions,
                    kv_append_ref, rope_fp16_ref, rope_ref, rope_tables_ref, varlen_positions)

pytestmark = pytest.mark.gpu

BASE = 1e6  # Qwen3's frequency base


def _tables(max_pos, d, device, base=BASE):
    c, s = rope_tables_ref(max_pos, d, base)
    c32, s32 = c.astype(np.float32), s.astype(np.float32)
    return (c32, s32), (torch.from_numpy(c32).to(device), torch.from_numpy(s32).to(device))


def _bits_equal(got, ref16):
    g = got.detach().cpu().contiguous().view(torch.int16)
    r = torch.from_numpy(np.ascontiguousarray(ref16)).view(torch.int16)
    return torch.equal(g, r)


@pytest.mark.parametrize("max_pos,d,base", [(40960, 128, 1e6), (5000, 64, 1e4), (1, 128, 500.0)])
def test_rope_tables(gpu, max_pos, d, base):
    cos, sin = attn.rope_tables(max_pos, d, base, device=gpu)
    torch.cuda.synchronize()
    c, s = rope_tables_ref(max_pos, d, base)
    for got, ref in ((cos, c), (sin, s)):
        g = got.cpu().numpy().view(np.int32).astype(np.int64)
        r = ref.astype(np.float32).view(np.int32).astype(np.int64)
        ulps = np.abs(g - r)
        print(f"tables {max_pos}x{d}: {int((ulps > 0).sum())} entries 1 ulp off", flush=True)
        assert ulps.max() <= 1


SEQS = [1, 17, 64, 65, 0, 130, 33, 300]


@pytest.mark.parametrize("h_q,h_kv,d", [(16, 8, 128), (8, 2, 64), (4, 4, 128)],
                         ids=lambda x: str(x))
def test_rope_varlen_bitwise(gpu, h_q, h_kv, d):
    """Standalone pass over packed sequences, forward and inverse, q and k
    together and each alone."""
    inp = W.make_train_inputs(SEQS, h_q, h_kv, d, seed=6000 + d + h_q, with_dout=False)
    pos = varlen_positions(inp["cu_seqlens"].numpy())
    (c, s), tab = _tables(max(SEQS), d, gpu)
    q, k, cu = inp["q"].to(gpu), inp["k"].to(gpu), inp["cu_seqlens"].to(gpu)
    attn.rope(q, k, cu, tab, max_seqlen=max(SEQS))
    torch.cuda.synchronize()
    assert _bits_equal(q, rope_fp16_ref(inp["q"].numpy(), pos, c, s))
    assert _bits_equal(k, rope_fp16_ref(inp["k"].numpy(), pos, c, s))
    # Inverse of the rotated tensors (as the backward applies it to dq, dk).
    qi, ki = q.clone(), k.clone()
    attn.rope(qi, None, cu, tab, max_seqlen=max(SEQS), inverse=True)
    attn.rope(None, ki, cu, tab, max_seqlen=max(SEQS), inverse=True)
    torch.cuda.synchronize()
    assert _bits_equal(qi, rope_fp16_ref(q.cpu().numpy(), pos, c, s, inverse=True))
    assert _bits_equal(ki, rope_fp16_ref(k.cpu().numpy(), pos, c, s, inverse=True))


def test_rope_chunk_positions_bitwise(gpu):
    """With ctx_lens the tokens are the last L_b positions of each context."""
    prior, new = [0, 5, 300, 1000, 16, 0], [17, 1, 64, 129, 0, 3]
    inp = W.make_prefill_inputs(prior, new, 16, 8, 128, seed=6100)
    pos = chunk_positions(inp["cu_q"].numpy(), inp["ctx_lens"].numpy())
    (c, s), tab = _tables(inp["max_ctx"], 128, gpu)
    q, k = inp["q"].to(gpu), inp["k_new"].to(gpu)
    attn.rope(q, k, inp["cu_q"].to(gpu), tab, ctx_lens=inp["ctx_lens"].to(gpu),
              max_ctx_len=inp["max_ctx"], max_seqlen=inp["max_q_len"])
    torch.cuda.synchronize()
    assert _bits_equal(q, rope_fp16_ref(inp["q"].numpy(), pos, c, s))
    assert _bits_equal(k, rope_fp16_ref(inp["k_new"].numpy(), pos, c, s))
    # And back, at the same positions.
    qi = q.clone()
    attn.rope(qi, None, inp["cu_q"].to(gpu), tab, ctx_lens=inp["ctx_lens"].to(gpu),
              max_ctx_len=inp["max_ctx"], max_seqlen=inp["max_q_len"], inverse=True)
    torch.cuda.synchronize()
    assert _bits_equal(qi, rope_fp16_ref(q.cpu().numpy(), pos, c, s, inverse=True))


PRIOR = [0, 0, 5, 15, 16, 17, 100, 300, 0, 1000, 64, 511, 3, 31]
NEW = [1, 17, 1, 17, 16, 63, 64, 129, 300, 1, 65, 0, 128, 33]


@pytest.mark.parametrize("h_q,h_kv,d", [(16, 8, 128), (8, 2, 64), (12, 4, 128)],
                         ids=lambda x: str(x))
def test_append_and_prefill_with_rope(gpu, h_q, h_kv, d):
    """attn_kv_append_rope writes the oracle's rotated keys (bitwise, unused
    slots untouched); attn_prefill_paged_rope equals attn_rope on q followed
    by attn_prefill_paged bit for bit, and the oracle's prefill on the
    rotated tensors within the attention bars."""
    _prefill_with_rope(gpu, PRIOR, NEW, h_q, h_kv, d, 6200 + h_q + d,
                       f"prefill rope hq{h_q} hkv{h_kv} d{d}")


@pytest.mark.parametrize("h_q,h_kv,d", [(16, 8, 128), (8, 2, 64)], ids=lambda x: str(x))
def test_append_and_prefill_with_rope_long_context(gpu, h_q, h_kv, d):
    """The same checks with contexts past 4096 keys (the eight-wave prefill)."""
    _prefill_with_rope(gpu, [4200, 4090, 0, 300], [33, 10, 17, 129], h_q, h_kv, d,
                       6250 + h_q + d, f"prefill rope long hq{h_q} hkv{h_kv} d{d}")


def _prefill_with_rope(gpu, prior, new, h_q, h_kv, d, seed, name):
    inp = W.poison_unused_prefill(W.make_prefill_inputs(prior, new, h_q, h_kv, d,
                                                        seed=seed, spare_blocks=2))
    print(name, flush=True)
    pos = chunk_positions(inp["cu_q"].numpy(), inp["ctx_lens"].numpy())
    (c, s), tab = _tables(inp["max_ctx"], d, gpu)
    dd = {k: (v.to(gpu) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    attn.kv_append(dd["k_new"], dd["v_new"], dd["cu_q"], dd["block_table"], dd["ctx_lens"],
                   dd["k_pool"], dd["v_pool"], max_ctx_len=inp["max_ctx"],
                   max_q_len=inp["max_q_len"], rope=tab)
    o, lse = attn.prefill_paged(dd["q"], dd["k_pool"], dd["v_pool"], dd["block_table"],
                                dd["ctx_lens"], dd["cu_q"], inp["scale"],
                                max_ctx_len=inp["max_ctx"], max_q_len=inp["max_q_len"], rope=tab)
    torch.cuda.synchronize()
    assert torch.equal(dd["q"].cpu(), inp["q"])  # q itself is not modified

    qr = rope_fp16_ref(inp["q"].numpy(), pos, c, s)
    kr = rope_fp16_ref(inp["k_new"].numpy(), pos, c, s)
    kp, vp = kv_append_ref(inp["k_pool"].numpy(), inp["v_pool"].numpy(), kr,
                           inp["v_new"].numpy(), inp["cu_q"].numpy(), inp["block_table"].numpy(),
                           inp["ctx_lens"].numpy())
    assert _bits_equal(dd["k_pool"], kp), "k_pool differs"
    assert _bits_equal(dd["v_pool"], vp), "v_pool differs"

    # Same bits as the unfused order: rotate q with attn_rope, then prefill.
    q2 = dd["q"].clone()
    attn.rope(q2, None, dd["cu_q"], tab, ctx_lens=dd["ctx_lens"], max_ctx_len=inp["max_ctx"],
              max_seqlen=inp["max_q_len"])
    o2, lse2 = attn.prefill_paged(q2, dd["k_pool"], dd["v_pool"], dd["block_table"],
                                  dd["ctx_lens"], dd["cu_q"], inp["scale"],
                                  max_ctx_len=inp["max_ctx"], max_q_len=inp["max_q_len"])
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)

    cu = inp["cu_q"].tolist()
    o_np, lse_np = o.float().cpu().numpy(), lse.cpu().numpy()
    worst_o = worst_l = 0.0
    for b in range(inp["n"]):
        st, en = cu[b], cu[b + 1]
        if en == st:
            continue
        o_ref, lse_ref = attn_prefill_ref(qr[st:en], kp, vp, inp["block_table"].numpy()[b:b + 1],
                                          [int(inp["ctx_lens"][b])], [0, en - st], inp["scale"])
        worst_o = max(worst_o, max_abs(o_np[st:en], o_ref))
        worst_l = max(worst_l, max_abs(lse_np[:, st:en], lse_ref))
    print(f"{name}: O max abs {worst_o:.2e}, LSE max abs {worst_l:.2e}", flush=True)
    assert worst_o <= O_TOL and worst_l <= LSE_TOL


@pytest.mark.parametrize("h_q,h_kv,d", [(16, 8, 128), (8, 2, 64)], ids=lambda x: str(x))
def test_training_chain_with_rope(gpu, h_q, h_kv, d):
    """rope(q, k) -> attn_fwd -> attn_bwd -> inverse rope(dq, dk) against the
    oracle chain: fp16 rotation, fp64 attention and backward, fp64 inverse
    rotation of the gradients."""
    seqs = [1, 17, 64, 65, 130, 0, 33]
    inp = W.make_train_inputs(seqs, h_q, h_kv, d, seed=6300 + d)
    pos = varlen_positions(inp["cu_seqlens"].numpy())
    (c, s), tab = _tables(max(seqs), d, gpu)
    dd = {k: (v.to(gpu) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    q, k = dd["q"].clone(), dd["k"].clone()
    attn.rope(q, k, dd["cu_seqlens"], tab, max_seqlen=max(seqs))
    o, lse = attn.fwd(q, k, dd["v"], dd["cu_seqlens"], inp["scale"], max_seqlen=max(seqs))
    dq, dk, dv = attn.bwd(q, k, dd["v"], o, lse, dd["dout"], dd["cu_seqlens"], inp["scale"],
                          max_seqlen=max(seqs))
    attn.rope(dq, dk, dd["cu_seqlens"], tab, max_seqlen=max(seqs), inverse=True)
    torch.cuda.synchronize()

    qr = rope_fp16_ref(inp["q"].numpy(), pos, c, s)
    kr = rope_fp16_ref(inp["k"].numpy(), pos, c, s)
    assert _bits_equal(q, qr) and _bits_equal(k, kr)
    cu = inp["cu_seqlens"].numpy()
    v, dout = inp["v"].numpy(), inp["dout"].numpy()
    o_ref, lse_ref = attn_fwd_ref(qr, kr, v, cu, inp["scale"])
    dq_r, dk_r, dv_ref = attn_bwd_ref(qr, kr, v, dout, cu, inp["scale"])
    dq_ref = rope_ref(dq_r, pos, c, s, inverse=True)
    dk_ref = rope_ref(dk_r, pos, c, s, inverse=True)
    errs = dict(o=max_abs(o.float().cpu().numpy(), o_ref),
                lse=max_abs(lse.cpu().numpy(), lse_ref),
                dq=rel_l2(dq.float().cpu().numpy(), dq_ref),
                dk=rel_l2(dk.float().cpu().numpy(), dk_ref),
                dv=rel_l2(dv.float().cpu().numpy(), dv_ref))
    print(f"rope chain hq{h_q} d{d}: " + ", ".join(f"{n} {e:.2e}" for n, e in errs.items()),
          flush=True)
    assert errs["o"] <= O_TOL and errs["lse"] <= LSE_TOL
    assert max(errs["dq"], errs["dk"], errs["dv"]) <= GRAD_TOL


def test_rope_workload_bitwise(gpu):
    """The qwen3_train shape (8 x 1024 tokens, 16 query and 8 key heads,
    d = 128) as the benchmark rotates it: every element against the oracle."""
    inp = W.workload_inputs("qwen3_train", with_dout=False)
    pos = varlen_positions(inp["cu_seqlens"].numpy())
    (c, s), tab = _tables(inp["max_seqlen"], inp["d"], gpu)
    q, k = inp["q"].to(gpu), inp["k"].to(gpu)
    attn.rope(q, k, inp["cu_seqlens"].to(gpu), tab, max_seqlen=inp["max_seqlen"])
    torch.cuda.synchronize()
    assert _bits_equal(q, rope_fp16_ref(inp["q"].numpy(), pos, c, s))
    assert _bits_equal(k, rope_fp16_ref(inp["k"].numpy(), pos, c, s))


@pytest.mark.parametrize("h_q,h_kv,d", [(16, 8, 128), (8, 2, 64), (6, 6, 64)],
                         ids=lambda x: str(x))
def test_decode_step_with_rope(gpu, h_q, h_kv, d):
    """One rollout decode step with RoPE: attn_kv_append_rope stores the new
    token's rotated key, attn_rope (ctx_lens) rotates its query, and
    attn_decode_paged attends; attn_decode_paged_rope (rotating the query at
    load) must give the same bits. The result must agree with the prefill
    that rotates one-token chunks itself (two different kernels), and with
    the oracle decode over the oracle-rotated tensors."""
    from oracle import attn_decode_ref
    prior = [0, 15, 16, 100, 1000, 2047]
    inp = W.make_prefill_inputs(prior, [1] * len(prior), h_q, h_kv, d, seed=6400 + d + h_q)
    pos = chunk_positions(inp["cu_q"].numpy(), inp["ctx_lens"].numpy())
    (c, s), tab = _tables(inp["max_ctx"], d, gpu)
    dd = {k: (v.to(gpu) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    kw = dict(max_ctx_len=inp["max_ctx"], max_q_len=1)
    attn.kv_append(dd["k_new"], dd["v_new"], dd["cu_q"], dd["block_table"], dd["ctx_lens"],
                   dd["k_pool"], dd["v_pool"], rope=tab, **kw)
    op, _ = attn.prefill_paged(dd["q"], dd["k_pool"], dd["v_pool"], dd["block_table"],
                               dd["ctx_lens"], dd["cu_q"], inp["scale"], rope=tab, **kw)
    qd = dd["q"].clone()
    attn.rope(qd, None, dd["cu_q"], tab, ctx_lens=dd["ctx_lens"], max_ctx_len=inp["max_ctx"],
              max_seqlen=1)
    od = attn.decode_paged(qd, dd["k_pool"], dd["v_pool"], dd["block_table"], dd["ctx_lens"],
                           inp["scale"], max_ctx_len=inp["max_ctx"])
    # The decode that rotates its queries itself: the same bits.
    of = attn.decode_paged(dd["q"], dd["k_pool"], dd["v_pool"], dd["block_table"],
                           dd["ctx_lens"], inp["scale"], max_ctx_len=inp["max_ctx"], rope=tab)
    torch.cuda.synchronize()
    assert torch.equal(of, od)
    assert torch.equal(dd["q"].cpu(), inp["q"])
    qr = rope_fp16_ref(inp["q"].numpy(), pos, c, s)
    assert _bits_equal(qd, qr)
    kr = rope_fp16_ref(inp["k_new"].numpy(), pos, c, s)
    kp, vp = kv_append_ref(inp["k_pool"].numpy(), inp["v_pool"].numpy(), kr,
                           inp["v_new"].numpy(), inp["cu_q"].numpy(), inp["block_table"].numpy(),
                           inp["ctx_lens"].numpy())
    o_ref = attn_decode_ref(qr, kp, vp, inp["block_table"].numpy(), inp["ctx_lens"].numpy(),
                            inp["scale"])
    e_dec = max_abs(od.float().cpu().numpy(), o_ref)
    e_pre = max_abs(op.float().cpu().numpy(), o_ref)
    e_both = max_abs(od.float().cpu().numpy(), op.float().cpu().numpy())
    print(f"decode with rope: decode {e_dec:.2e}, prefill {e_pre:.2e}, between {e_both:.2e}",
          flush=True)
    assert e_dec <= O_TOL and e_pre <= O_TOL and e_both <= 2 * O_TOL


@pytest.mark.parametrize("seqs,h_q,h_kv,d", [
    ([1, 17, 64, 65, 130, 0, 33], 16, 8, 128),  # ragged: the dS path
    ([128, 128], 16, 8, 128),                   # equal lengths: the recompute path
    ([300, 64, 1], 8, 2, 64),
    ([256, 256], 8, 2, 64),
], ids=lambda x: str(x))
def test_bwd_with_fused_inverse_rope(gpu, seqs, h_q, h_kv, d):
    """attn_bwd_rope (inverse rotation of dq, dk in fp32 at their stores, one
    fp16 rounding) against the oracle chain within the gradient bar, no less
    accurate than attn_bwd + inverse attn_rope (two fp16 roundings) and within
    about one fp16 unit of it; dv is attn_bwd's bit for bit."""
    inp = W.make_train_inputs(seqs, h_q, h_kv, d, seed=6500 + sum(seqs) + d)
    ms = max(seqs)
    pos = varlen_positions(inp["cu_seqlens"].numpy())
    (c, s), tab = _tables(ms, d, gpu)
    dd = {k: (v.to(gpu) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    q, k = dd["q"].clone(), dd["k"].clone()
    attn.rope(q, k, dd["cu_seqlens"], tab, max_seqlen=ms)
    o, lse = attn.fwd(q, k, dd["v"], dd["cu_seqlens"], inp["scale"], max_seqlen=ms)
    args = (q, k, dd["v"], o, lse, dd["dout"], dd["cu_seqlens"], inp["scale"])
    dq1, dk1, dv1 = attn.bwd(*args, max_seqlen=ms, rope=tab)
    dq2, dk2, dv2 = attn.bwd(*args, max_seqlen=ms)
    attn.rope(dq2, dk2, dd["cu_seqlens"], tab, max_seqlen=ms, inverse=True)
    torch.cuda.synchronize()
    assert torch.equal(dv1, dv2)

    qr = rope_fp16_ref(inp["q"].numpy(), pos, c, s)
    kr = rope_fp16_ref(inp["k"].numpy(), pos, c, s)
    cu = inp["cu_seqlens"].numpy()
    dq_r, dk_r, _ = attn_bwd_ref(qr, kr, inp["v"].numpy(), inp["dout"].numpy(), cu,
                                 inp["scale"])
    dq_ref = rope_ref(dq_r, pos, c, s, inverse=True)
    dk_ref = rope_ref(dk_r, pos, c, s, inverse=True)
    res = []
    for name, fused, unfused, ref in (("dq", dq1, dq2, dq_ref), ("dk", dk1, dk2, dk_ref)):
        f, u = fused.float().cpu().numpy(), unfused.float().cpu().numpy()
        e_f, e_u, between = rel_l2(f, ref), rel_l2(u, ref), rel_l2(f, u)
        res.append(f"{name} fused {e_f:.2e} unfused {e_u:.2e} between {between:.2e}")
        assert e_f <= GRAD_TOL and e_f <= e_u * 1.02 + 1e-6 and between <= 1e-3, res[-1]
    print(f"bwd rope {seqs} d{d}: " + "; ".join(res), flush=True)


def test_rope_prefill_workload(gpu):
    """The paged_prefill workload (32 sequences, cached 0-1536, new 128-512
    tokens) with RoPE, launched as the benchmark launches it: the pools
    against the oracle's append of the oracle-rotated keys (every element),
    the fused prefill against attn_rope + attn_prefill_paged (bit for bit) and
    against the oracle on sampled sequences."""
    inp = W.prefill_workload_inputs("paged_prefill")
    pos = chunk_positions(inp["cu_q"].numpy(), inp["ctx_lens"].numpy())
    (c, s), tab = _tables(inp["max_ctx"], inp["d"], gpu)
    dd = {k: (v.to(gpu) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    kw = dict(max_ctx_len=inp["max_ctx"], max_q_len=inp["max_q_len"])
    attn.kv_append(dd["k_new"], dd["v_new"], dd["cu_q"], dd["block_table"], dd["ctx_lens"],
                   dd["k_pool"], dd["v_pool"], rope=tab, **kw)
    o, lse = attn.prefill_paged(dd["q"], dd["k_pool"], dd["v_pool"], dd["block_table"],
                                dd["ctx_lens"], dd["cu_q"], inp["scale"], rope=tab, **kw)
    q2 = dd["q"].clone()
    attn.rope(q2, None, dd["cu_q"], tab, ctx_lens=dd["ctx_lens"], max_ctx_len=inp["max_ctx"],
              max_seqlen=inp["max_q_len"])
    o2, lse2 = attn.prefill_paged(q2, dd["k_pool"], dd["v_pool"], dd["block_table"],
                                  dd["ctx_lens"], dd["cu_q"], inp["scale"], **kw)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)
    qr = rope_fp16_ref(inp["q"].numpy(), pos, c, s)
    assert _bits_equal(q2, qr)
    kr = rope_fp16_ref(inp["k_new"].numpy(), pos, c, s)
    kp, vp = kv_append_ref(inp["k_pool"].numpy(), inp["v_pool"].numpy(), kr,
                           inp["v_new"].numpy(), inp["cu_q"].numpy(), inp["block_table"].numpy(),
                           inp["ctx_lens"].numpy())
    assert _bits_equal(dd["k_pool"], kp) and _bits_equal(dd["v_pool"], vp)
    cu = inp["cu_q"].tolist()
    o_np, lse_np = o.float().cpu().numpy(), lse.cpu().numpy()
    worst_o = worst_l = 0.0
    for b in (0, 9, 20, 31):
        st, en = cu[b], cu[b + 1]
        o_ref, lse_ref = attn_prefill_ref(qr[st:en], kp, vp, inp["block_table"].numpy()[b:b + 1],
                                          [int(inp["ctx_lens"][b])], [0, en - st], inp["scale"])
        worst_o = max(worst_o, max_abs(o_np[st:en], o_ref))
        worst_l = max(worst_l, max_abs(lse_np[:, st:en], lse_ref))
    print(f"paged_prefill with rope: O {worst_o:.2e}, LSE {worst_l:.2e}", flush=True)
    assert worst_o <= O_TOL and worst_l <= LSE_TOL


def test_bwd_rope_workload(gpu):
    """qwen3_train (8 x 1024, H_q 16, H_kv 8, d 128) through attn_bwd_rope as
    the benchmark launches it, against attn_bwd + inverse attn_rope (about one
    fp16 unit apart) and dv bit for bit; the oracle on one sampled sequence
    and KV group."""
    inp = W.workload_inputs("qwen3_train")
    ms = inp["max_seqlen"]
    (c, s), tab = _tables(ms, inp["d"], gpu)
    dd = {k: (v.to(gpu) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    q, k = dd["q"].clone(), dd["k"].clone()
    attn.rope(q, k, dd["cu_seqlens"], tab, max_seqlen=ms)
    o, lse = attn.fwd(q, k, dd["v"], dd["cu_seqlens"], inp["scale"], max_seqlen=ms)
    args = (q, k, dd["v"], o, lse, dd["dout"], dd["cu_seqlens"], inp["scale"])
    dq1, dk1, dv1 = attn.bwd(*args, max_seqlen=ms, rope=tab)
    dq2, dk2, dv2 = attn.bwd(*args, max_seqlen=ms)
    attn.rope(dq2, dk2, dd["cu_seqlens"], tab, max_seqlen=ms, inverse=True)
    torch.cuda.synchronize()
    assert torch.equal(dv1, dv2)
    for a, b in ((dq1, dq2), (dk1, dk2)):
        assert rel_l2(a.float().cpu().numpy(), b.float().cpu().numpy()) <= 1e-3
    # Oracle: sequence 5, KV head 3 and its two query heads.
    seq, g = 5, 3
    rows = slice(seq * 1024, (seq + 1) * 1024)
    heads = slice(2 * g, 2 * g + 2)
    pos = np.arange(1024)
    qr = q[rows, heads].cpu().numpy()
    kr = k[rows, g:g + 1].cpu().numpy()
    cu1 = np.array([0, 1024])
    dq_r, dk_r, _ = attn_bwd_ref(qr, kr, inp["v"].numpy()[rows, g:g + 1],
                                 inp["dout"].numpy()[rows, heads], cu1, inp["scale"])
    e_q = rel_l2(dq1[rows, heads].float().cpu().numpy(), rope_ref(dq_r, pos, c, s, inverse=True))
    # dK sums over the group's query heads; with G = 2 both are in the sample.
    e_k = rel_l2(dk1[rows, g:g + 1].float().cpu().numpy(), rope_ref(dk_r, pos, c, s, inverse=True))
    print(f"qwen3_train bwd rope: dq {e_q:.2e}, dk {e_k:.2e}", flush=True)
    assert e_q <= GRAD_TOL and e_k <= GRAD_TOL


def test_decode_rope_workload(gpu):
    """The paged_decode workload (256 sequences, context 128-4096) with RoPE,
    launched as the benchmark launches it: attn_decode_paged_rope equals
    attn_rope on q followed by attn_decode_paged bit for bit, and matches the
    oracle decode on sampled sequences."""
    from oracle import attn_decode_ref
    inp = W.decode_workload_inputs("paged_decode")
    n = inp["q"].shape[0]
    ctx = inp["ctx_lens"].numpy()
    (c, s), tab = _tables(int(ctx.max()), inp["q"].shape[2], gpu)
    dd = {k: (v.to(gpu) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    of = attn.decode_paged(dd["q"], dd["k_pool"], dd["v_pool"], dd["block_table"],
                           dd["ctx_lens"], inp["scale"], max_ctx_len=int(ctx.max()), rope=tab)
    cu1 = torch.arange(n + 1, dtype=torch.int32, device=gpu)
    qd = dd["q"].clone()
    attn.rope(qd, None, cu1, tab, ctx_lens=dd["ctx_lens"], max_ctx_len=int(ctx.max()),
              max_seqlen=1)
    od = attn.decode_paged(qd, dd["k_pool"], dd["v_pool"], dd["block_table"], dd["ctx_lens"],
                           inp["scale"], max_ctx_len=int(ctx.max()))
    torch.cuda.synchronize()
    assert torch.equal(of, od)
    qr = rope_fp16_ref(inp["q"].numpy(), ctx - 1, c, s)
    assert _bits_equal(qd, qr)
    rows = [0, 77, 128, 255]
    o_ref = attn_decode_ref(qr[rows], inp["k_pool"].numpy(), inp["v_pool"].numpy(),
                            inp["block_table"].numpy()[rows], ctx[rows], inp["scale"])
    err = max_abs(of.float().cpu().numpy()[rows], o_ref)
    print(f"paged_decode with rope: O {err:.2e}", flush=True)
    assert err <= O_TOL
