"""Shared helpers of the GPU parity tests (not collected by pytest).

Tolerances (from the attention build's stated bar): forward O and decode O
max abs error <= 2e-3, LSE max abs error <= 1e-4, dQ/dK/dV relative L2
error <= 1e-2, all against the fp64 CPU oracle on the same fp16 inputs.
"""
import numpy as np
import torch

import causal_gqa_attention_fa2_amd as attn
from causal_gqa_attention_fa2_amd import workloads as W
from oracle import attn_bwd_ref, attn_decode_ref, attn_fwd_ref

O_TOL = 2e-3
LSE_TOL = 1e-4
GRAD_TOL = 1e-2


def rel_l2(x, ref):
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(x - ref) / (den if den > 0 else 1.0))


def max_abs(x, ref):
    d = np.abs(np.asarray(x, dtype=np.float64) - np.asarray(ref, dtype=np.float64))
    return float(d.max()) if d.size else 0.0


def fp16_floor(ref):
    """max |fp16(ref) - ref|: the error of storing the exact result in fp16."""
    r = np.asarray(ref, dtype=np.float64)
    return max_abs(r.astype(np.float16).astype(np.float64), r) if r.size else 0.0


def dev(inp, device):
    return {k: (v.to(device) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}


def gpu_fwd(d):
    return attn.fwd(d["q"], d["k"], d["v"], d["cu_seqlens"], d["scale"],
                    max_seqlen=d["max_seqlen"])


def gpu_bwd(d, o, lse):
    return attn.bwd(d["q"], d["k"], d["v"], o, lse, d["dout"], d["cu_seqlens"], d["scale"],
                    max_seqlen=d["max_seqlen"])


def _slices(inp, seqs, groups):
    """(name, q, k, v, dout, heads, group) slices of sampled sequences and KV
    groups: the oracle sees each sampled sequence alone, with the G query
    heads of one KV head."""
    cu = inp["cu_seqlens"].tolist()
    h_q, h_kv = inp["q"].shape[1], inp["k"].shape[1]
    G = h_q // h_kv
    seqs = range(len(cu) - 1) if seqs is None else seqs
    groups = range(h_kv) if groups is None else groups
    for b in seqs:
        s, e = cu[b], cu[b + 1]
        if e == s:
            continue
        for g in groups:
            hs = slice(g * G, (g + 1) * G)
            dout = inp["dout"][s:e, hs].numpy() if inp.get("dout") is not None else None
            yield (s, e, hs, g, inp["q"][s:e, hs].numpy(), inp["k"][s:e, g:g + 1].numpy(),
                   inp["v"][s:e, g:g + 1].numpy(), dout)


def check_fwd(name, inp, o, lse, seqs=None, groups=None):
    """Compare GPU O/LSE with the oracle on all (or the sampled) sequences and
    KV groups."""
    o = o.float().cpu().numpy()
    lse = lse.cpu().numpy()
    worst_o = worst_l = floor = 0.0
    for s, e, hs, g, q, k, v, _ in _slices(inp, seqs, groups):
        o_ref, lse_ref = attn_fwd_ref(q, k, v, [0, e - s], inp["scale"])
        worst_o = max(worst_o, max_abs(o[s:e, hs], o_ref))
        worst_l = max(worst_l, max_abs(lse[hs, s:e], lse_ref))
        floor = max(floor, fp16_floor(o_ref))
    print(f"[{name}] fwd: O max abs {worst_o:.3e} (fp16 floor {floor:.3e}), "
          f"LSE max abs {worst_l:.3e}", flush=True)
    assert np.isfinite(worst_o) and worst_o <= O_TOL, (name, worst_o)
    assert np.isfinite(worst_l) and worst_l <= LSE_TOL, (name, worst_l)
    return worst_o, worst_l


def check_bwd(name, inp, dq, dk, dv, seqs=None, groups=None):
    """Relative L2 error of dq, dk, dv over all (or the sampled) sequences and
    KV groups; dk/dv of a KV head sum over its G query heads on both sides."""
    dq, dk, dv = (t.float().cpu().numpy() for t in (dq, dk, dv))
    refs = [[], [], []]
    gots = [[], [], []]
    for s, e, hs, g, q, k, v, do in _slices(inp, seqs, groups):
        ref = attn_bwd_ref(q, k, v, do, [0, e - s], inp["scale"])
        for i, (mine, r) in enumerate(zip((dq[s:e, hs], dk[s:e, g:g + 1], dv[s:e, g:g + 1]), ref)):
            refs[i].append(r.ravel())
            gots[i].append(mine.ravel())
    errs = [rel_l2(np.concatenate(gots[i]), np.concatenate(refs[i])) if refs[i] else 0.0
            for i in range(3)]
    print(f"[{name}] bwd: rel L2 dq {errs[0]:.3e} dk {errs[1]:.3e} dv {errs[2]:.3e}", flush=True)
    for nm, e in zip(("dq", "dk", "dv"), errs):
        assert np.isfinite(e) and e <= GRAD_TOL, (name, nm, e)
    return errs


def check_decode(name, inp, o):
    o = o.float().cpu().numpy()
    ref = attn_decode_ref(inp["q"].numpy(), inp["k_pool"].numpy(), inp["v_pool"].numpy(),
                          inp["block_table"].numpy(), inp["ctx_lens"].numpy(), inp["scale"])
    err = max_abs(o, ref)
    print(f"[{name}] decode: O max abs {err:.3e} (fp16 floor {fp16_floor(ref):.3e})", flush=True)
    assert np.all(np.isfinite(o)), name
    assert err <= O_TOL, (name, err)
    return err


def gpu_decode(d):
    return attn.decode_paged(d["q"], d["k_pool"], d["v_pool"], d["block_table"], d["ctx_lens"],
                             d["scale"], max_ctx_len=d["max_ctx"])


__all__ = ["W", "attn", "check_fwd", "check_bwd", "check_decode", "dev", "gpu_fwd", "gpu_bwd",
           "gpu_decode", "rel_l2", "max_abs", "O_TOL", "LSE_TOL", "GRAD_TOL"]
