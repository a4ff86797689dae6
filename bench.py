#!/usr/bin/env python3
"""Benchmark of the causal GQA attention hot path on one MI355X.

One step = one pass over every stage of the path on resident synthetic
inputs: attn_fwd + attn_bwd on the long-context training workload (B=4,
S=8192, H_q=16, H_kv=8, d=128, fp16; the largest training workload that one
GPU holds) and attn_decode_paged on the rollout decode workload (256
sequences, ctx U{128..4096}, 16-token blocks).

Prints ONE JSON line. ``value`` is the forward+backward attention
throughput in TFLOP/s (causal FLOP count: 4*d*H_q per unmasked (query, key)
pair for the forward, 2.5x that for the backward) from HIP events on the
launch stream; the decode bandwidth (algorithmic bytes / event time) rides
along in ``decode``. ``configs`` holds every workload: the tiny case (µs),
the 1024-token, GRPO varlen and long-context training batches (fwd and bwd
µs as median / min / max: over the timed steps for long_context, else over
5 groups of 20 back-to-back launches, each group timed by one event pair;
TFLOP/s on the median
and its fraction of the dense fp16 MFMA peak) and the decode (GB/s, fraction
of HBM peak). ``roofline`` reports the entry point that takes the most time
per step against its bound; ``cpu_baseline`` times the fp64 CPU oracle on a
bounded sample of the long-context workload, with the host's CPU model,
core counts and BLAS library. ``prefill`` times the rollout
engine's chunked prefill (attn_kv_append + attn_prefill_paged on the
paged_prefill workload) separately, after the timed steps; it is not part of
``value``. ``measured_peaks`` holds this GPU's measured dense fp16 MFMA rate,
the shader clock under it and its streaming-read rate (probe kernels of
libattn_probe.so), the second denominators beside the published peaks.
``rmsnorm`` likewise times RMSNorm forward and backward on the
training batch's layer norm and per-head query norm (HBM-bound, GB/s),
``sampling`` the rollout batch's temperature / top-k / top-p sampling, and
``rope`` the rotary embedding pass over the training batch's q and k plus
the append and prefill with the rotation fused in.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--no-cpu-baseline]
"""
import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_F16_PEAK_TFLOPS = 2516.6  # 256 CU x 2.4 GHz x 4096 FLOP/clk, dense fp16
HBM_PEAK_GBPS = 8000.0
TRAIN_WORKLOAD = "long_context"
DECODE_WORKLOAD = "paged_decode"
ROPE_WORKLOAD = "qwen3_train"
KERNEL_SOURCES = ["attn_fwd.hip", "attn_bwd.hip", "attn_decode.hip", "attn_cache.hip",
                  "attn_norm.hip", "attn_sample.hip", "attn_rope.hip", "probe_peaks.hip", "cdna4.h",
                  "kernels.h", "attn_api.cpp"]


def causal_pairs(seqlens):
    return sum(L * (L + 1) // 2 for L in seqlens)


def train_costs(inp):
    d, h_q, h_kv, T = inp["d"], inp["h_q"], inp["h_kv"], inp["total_tokens"]
    pairs = causal_pairs(inp["seqlens"])
    f_fwd = 4 * d * h_q * pairs
    f_bwd = 2.5 * f_fwd
    qo = T * h_q * d * 2
    kv = T * h_kv * d * 2
    lse = h_q * T * 4
    b_fwd = qo + 2 * kv + qo + lse                       # read q,k,v; write o,lse
    b_bwd = qo + 2 * kv + qo + qo + lse + qo + 2 * kv     # read q,k,v,o,dO,lse; write dq,dk,dv
    return f_fwd, f_bwd, b_fwd, b_bwd


def decode_costs(inp):
    ctx = [int(c) for c in inp["ctx_lens"]]
    d, h_q, h_kv, n = inp["d"], inp["h_q"], inp["h_kv"], inp["n"]
    kv = sum(ctx) * h_kv * d * 2 * 2
    qo = 2 * n * h_q * d * 2
    table = sum(math.ceil(c / inp["block_size"]) for c in ctx) * 4 + n * 4
    flops = 4 * d * h_q * sum(ctx)
    return flops, kv + qo + table


def source_digest():
    h = hashlib.sha256()
    paths = [os.path.join(ROOT, "causal_gqa_attention_fa2_amd", "csrc", f) for f in KERNEL_SOURCES]
    paths.append(os.path.join(ROOT, "causal_gqa_attention_fa2_amd", "build.py"))  # flags
    for path in paths:
        with open(path, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def read_traffic(kernel, workload):
    """HBM bytes per launch of entry point `kernel` on `workload` from the
    committed rocprofv3 counter summary, if it was taken on the current kernel
    sources (else None)."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.md")
    if not os.path.exists(path):
        return None
    txt = open(path).read()
    m_src = re.search(r"source_digest:\s*([0-9a-f]+)", txt)
    m_b = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", txt)
    if not m_src or not m_b or m_src.group(1) != source_digest():
        return None
    return float(m_b.group(1))


def host_facts():
    """CPU model, logical CPUs, CPUs this process may run on, and the BLAS
    library NumPy calls with its thread count."""
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:  # pragma: no cover
        pass
    blas = []
    try:
        import numpy  # noqa: F401  (loads the BLAS library threadpoolctl inspects)
        from threadpoolctl import threadpool_info
        for i in threadpool_info():
            if i.get("user_api") == "blas":
                blas.append({"library": i.get("internal_api"), "version": i.get("version"),
                             "threads": i.get("num_threads"),
                             "arch": i.get("architecture")})
    except Exception:  # pragma: no cover
        pass
    return {"cpu_model": model, "os_cpu_count": os.cpu_count(),
            "sched_affinity": len(os.sched_getaffinity(0)), "blas": blas}


def cpu_baseline(budget_s):
    """The fp64 oracle (as it stands) on whole (sequence, KV-group) slices of the
    long-context workload, forward + backward, until `budget_s` seconds pass
    (at least one slice)."""
    from causal_gqa_attention_fa2_amd import workloads as W
    from oracle import attn_bwd_ref, attn_fwd_ref
    facts = host_facts()
    threads = max([b["threads"] or 1 for b in facts["blas"]] or [1])
    inp = W.workload_inputs(TRAIN_WORKLOAD)
    cu = inp["cu_seqlens"].tolist()
    G = inp["h_q"] // inp["h_kv"]
    flops = 0.0
    n = 0
    slices = [(b, g) for b in range(len(cu) - 1) for g in range(inp["h_kv"])]
    t0 = time.perf_counter()
    while n == 0 or time.perf_counter() - t0 < budget_s:  # whole slices, then stop
        for b, g in slices:
            s, e = cu[b], cu[b + 1]
            hs = slice(g * G, (g + 1) * G)
            q = inp["q"][s:e, hs].numpy()
            k = inp["k"][s:e, g:g + 1].numpy()
            v = inp["v"][s:e, g:g + 1].numpy()
            do = inp["dout"][s:e, hs].numpy()
            attn_fwd_ref(q, k, v, [0, e - s], inp["scale"])
            attn_bwd_ref(q, k, v, do, [0, e - s], inp["scale"])
            flops += 3.5 * 4 * inp["d"] * G * causal_pairs([e - s])
            n += 1
            if time.perf_counter() - t0 >= budget_s:
                break
    dt = time.perf_counter() - t0
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{n} (sequence, KV-group) slices of {TRAIN_WORKLOAD} "
                      f"({len(slices)} per batch: one sequence, its 2 query heads and 1 KV "
                      f"head), fwd+bwd in fp64, {dt:.1f} s wall",
            "host": facts, "seconds": dt}


PREFILL_WORKLOAD = "paged_prefill"


def prefill_costs(inp):
    """Causal FLOPs of a chunked prefill (query i of sequence b sees
    prior_b + i + 1 positions) and the append's algorithmic bytes."""
    d, h_q, h_kv = inp["d"], inp["h_q"], inp["h_kv"]
    pairs = sum(L * p + L * (L + 1) // 2 for p, L in zip(inp["prior_lens"], inp["new_lens"]))
    append_bytes = 2 * 2 * inp["total_q"] * h_kv * d * 2  # k and v, read and write
    return 4 * d * h_q * pairs, append_bytes


def bench_prefill(attn, W, dev, iters):
    """The rollout engine's chunked prefill on the paged_prefill workload,
    timed on its own (not part of `value`): attn_kv_append and
    attn_prefill_paged, each averaged over back-to-back launches."""
    import torch
    inp = W.prefill_workload_inputs(PREFILL_WORKLOAD)
    q, kn, vn, cu, kp, vp, bt, ctx = (inp[n].to(dev) for n in (
        "q", "k_new", "v_new", "cu_q", "k_pool", "v_pool", "block_table", "ctx_lens"))
    o = torch.empty_like(q)
    lse = torch.empty((q.shape[1], q.shape[0]), dtype=torch.float32, device=dev)
    kw = dict(max_ctx_len=inp["max_ctx"], max_q_len=inp["max_q_len"])

    def append():
        attn.kv_append(kn, vn, cu, bt, ctx, kp, vp, **kw)

    def prefill():
        attn.prefill_paged(q, kp, vp, bt, ctx, cu, inp["scale"], o=o, lse=lse, **kw)

    def timed(fn):
        """Mean time of `iters` back-to-back launches, queued behind a spin
        kernel so that the GPU never waits for the host."""
        return time_launches([fn], iters)[0][0]

    t_app = timed(append)  # rewrites the same slots: idempotent
    t_att = timed(prefill)
    flops, app_bytes = prefill_costs(inp)
    return {"workload": "paged_prefill (32 seqs, cached U{0..1536} + new U{128..512}, "
                        "block 16, H_q=16, H_kv=8, d=128)",
            "append_us": round(t_app * 1e6, 2),
            "append_GB/s": round(app_bytes / t_app / 1e9, 1),
            "attn_us": round(t_att * 1e6, 2),
            "attn_TFLOP/s": round(flops / t_att / 1e12, 2),
            "attn_mfma_peak_frac": round(flops / t_att / 1e12 / MFMA_F16_PEAK_TFLOPS, 4)}


def bench_rope(attn, W, dev, iters):
    """RoPE, timed on its own (not part of `value`): the standalone pass over
    the training batch's q and k (qwen3_train: 8 x 1024 tokens, 16 + 8 heads,
    d = 128), forward and inverse, HBM-bound against 8 TB/s; the training
    backward with the inverse rotation fused into its dq / dk stores, beside
    attn_bwd alone; and on the paged_prefill workload the append and the
    prefill with the rotation fused in, beside the same calls without it."""
    import torch
    inp = W.workload_inputs(ROPE_WORKLOAD, with_dout=False)
    q, k, cu = inp["q"].to(dev), inp["k"].to(dev), inp["cu_seqlens"].to(dev)
    T, h_q, d = q.shape
    h_kv = k.shape[1]
    pre = W.prefill_workload_inputs(PREFILL_WORKLOAD)
    max_pos = max(inp["max_seqlen"], pre["max_ctx"])
    tab = attn.rope_tables(max_pos, d, 1e6, device=dev)

    def timed(fn):
        """Mean time of `iters` back-to-back launches, queued behind a spin
        kernel so that the GPU never waits for the host."""
        return time_launches([fn], iters)[0][0]

    ms = inp["max_seqlen"]
    t_f = timed(lambda: attn.rope(q, k, cu, tab, max_seqlen=ms))
    t_i = timed(lambda: attn.rope(q, k, cu, tab, max_seqlen=ms, inverse=True))
    # q and k read and written once, one table row (cos and sin) per token.
    nbytes = 2 * T * (h_q + h_kv) * d * 2 + T * d * 4
    out = {"workload": f"{ROPE_WORKLOAD} q+k ({T} tokens, H_q={h_q}, H_kv={h_kv}, d={d})",
           "fwd_us": round(t_f * 1e6, 2), "fwd_GB/s": round(nbytes / t_f / 1e9, 1),
           "inv_us": round(t_i * 1e6, 2), "inv_GB/s": round(nbytes / t_i / 1e9, 1),
           "fwd_hbm_peak_frac": round(nbytes / t_f / 1e9 / HBM_PEAK_GBPS, 4)}

    # Training step on the rotated q and k: attn_bwd_rope (inverse rotation of
    # dq, dk fused into the stores) against attn_bwd with and without the
    # separate inverse pass.
    tr_v = W.workload_inputs(ROPE_WORKLOAD)
    v, dout = tr_v["v"].to(dev), tr_v["dout"].to(dev)
    o, lse = attn.fwd(q, k, v, cu, inp["scale"], max_seqlen=ms)
    dq, dk, dv = (torch.empty_like(t) for t in (q, k, v))
    ws = torch.empty(max(1, attn.bwd_workspace_bytes(attn.varlen_dims(q, k, cu, ms))),
                     dtype=torch.uint8, device=dev)
    bargs = (q, k, v, o, lse, dout, cu, inp["scale"])

    def fwd():
        attn.fwd(q, k, v, cu, inp["scale"], o=o, lse=lse, max_seqlen=ms)

    def bwd(rope=None):
        attn.bwd(*bargs, dq=dq, dk=dk, dv=dv, max_seqlen=ms, workspace=ws, rope=rope)

    def unfused():
        fwd()
        bwd()
        attn.rope(dq, dk, cu, tab, max_seqlen=ms, inverse=True)

    # Whole training steps (forward, then backward), as the timed steps run
    # them: the plain backward, the fused one, and the plain one followed by
    # the separate inverse pass. The three alternate over five rounds and each
    # keeps its best round, so that a clock still settling does not favour
    # whichever runs last.
    variants = {"step_fwd_bwd_us": lambda: (fwd(), bwd()),
                "step_fwd_bwd_rope_us": lambda: (fwd(), bwd(tab)),
                "step_fwd_bwd_then_inverse_pass_us": unfused}
    best = {name: float("inf") for name in variants}
    for _ in range(5):
        for name, fn in variants.items():
            best[name] = min(best[name], timed(fn))
    out.update({name: round(t * 1e6, 2) for name, t in best.items()})

    qp, kn, vn, cq, kp, vp, bt, ctx = (pre[n].to(dev) for n in (
        "q", "k_new", "v_new", "cu_q", "k_pool", "v_pool", "block_table", "ctx_lens"))
    o = torch.empty_like(qp)
    lse = torch.empty((qp.shape[1], qp.shape[0]), dtype=torch.float32, device=dev)
    kw = dict(max_ctx_len=pre["max_ctx"], max_q_len=pre["max_q_len"])
    t_app = timed(lambda: attn.kv_append(kn, vn, cq, bt, ctx, kp, vp, **kw))
    t_app_r = timed(lambda: attn.kv_append(kn, vn, cq, bt, ctx, kp, vp, rope=tab, **kw))
    t_att = timed(lambda: attn.prefill_paged(qp, kp, vp, bt, ctx, cq, pre["scale"], o=o, lse=lse,
                                             **kw))
    t_att_r = timed(lambda: attn.prefill_paged(qp, kp, vp, bt, ctx, cq, pre["scale"], o=o,
                                               lse=lse, rope=tab, **kw))
    # The rollout decode with the query rotation fused in, beside the plain
    # decode (the pools' keys count as rotated; the timing does not depend on it).
    dinp = W.decode_workload_inputs(DECODE_WORKLOAD)
    dq_, dkp, dvp, dbt, dctx = (dinp[n].to(dev) for n in ("q", "k_pool", "v_pool", "block_table",
                                                          "ctx_lens"))
    dmc = int(dinp["ctx_lens"].max())
    dtab = attn.rope_tables(dmc, d, 1e6, device=dev)
    dout_ = torch.empty_like(dq_)
    dws = torch.empty(max(1, attn.decode_workspace_bytes(attn.paged_dims(dq_, dkp, dbt, dmc))),
                      dtype=torch.uint8, device=dev)
    dvars = {"decode_us": lambda: attn.decode_paged(dq_, dkp, dvp, dbt, dctx, dinp["scale"],
                                                    o=dout_, max_ctx_len=dmc, workspace=dws),
             "decode_rope_us": lambda: attn.decode_paged(dq_, dkp, dvp, dbt, dctx, dinp["scale"],
                                                         o=dout_, max_ctx_len=dmc, workspace=dws,
                                                         rope=dtab)}
    dbest = {name: float("inf") for name in dvars}
    for _ in range(3):
        for name, fn in dvars.items():
            dbest[name] = min(dbest[name], timed(fn))
    out.update({name: round(t * 1e6, 2) for name, t in dbest.items()})
    out.update({"prefill_workload": "paged_prefill",
                "append_us": round(t_app * 1e6, 2), "append_rope_us": round(t_app_r * 1e6, 2),
                "prefill_us": round(t_att * 1e6, 2), "prefill_rope_us": round(t_att_r * 1e6, 2)})
    return out


def norm_bytes(rows, n):
    """Algorithmic HBM bytes of RMSNorm: forward reads x, w and writes y,
    rstd; backward reads x, w, rstd, dy and writes dx, dw."""
    fwd = 2 * rows * n * 2 + n * 2 + rows * 4
    bwd = 3 * rows * n * 2 + n * 2 + rows * 4 + n * 4
    return fwd, bwd


def bench_rmsnorm(attn, W, dev, iters):
    """RMSNorm forward and backward on the training batch's layer norm
    (8192 x 1024) and per-head query norm (131072 x 128), each averaged over
    back-to-back launches; HBM-bound, reported against 8 TB/s."""
    import torch
    out = {}
    for name in ("qwen3_rmsnorm", "qwen3_qknorm"):
        inp = W.norm_workload_inputs(name)
        x, w, dy = (inp[n].to(dev) for n in ("x", "w", "dy"))
        y = torch.empty_like(x)
        rstd = torch.empty(x.shape[0], dtype=torch.float32, device=dev)
        dx = torch.empty_like(x)
        dw = torch.empty(x.shape[1], dtype=torch.float32, device=dev)
        ws = torch.empty(max(1, attn.rmsnorm_bwd_workspace_bytes(x.shape[0], x.shape[1])),
                         dtype=torch.uint8, device=dev)

        def timed(fn):
            """Mean time of `iters` back-to-back launches, queued behind a spin
            kernel so that the GPU never waits for the host."""
            return time_launches([fn], iters)[0][0]

        t_f = timed(lambda: attn.rmsnorm_fwd(x, w, inp["eps"], y=y, rstd=rstd))
        t_b = timed(lambda: attn.rmsnorm_bwd(x, w, rstd, dy, dx=dx, dw=dw, workspace=ws))
        b_f, b_b = norm_bytes(*x.shape)
        out[name] = {"rows": x.shape[0], "n": x.shape[1],
                     "fwd_us": round(t_f * 1e6, 2), "fwd_GB/s": round(b_f / t_f / 1e9, 1),
                     "bwd_us": round(t_b * 1e6, 2), "bwd_GB/s": round(b_b / t_b / 1e9, 1),
                     "fwd_hbm_peak_frac": round(b_f / t_f / 1e9 / HBM_PEAK_GBPS, 4),
                     "bwd_hbm_peak_frac": round(b_b / t_b / 1e9 / HBM_PEAK_GBPS, 4)}
    return out


def bench_sampling(attn, W, dev, iters):
    """Temperature / top-k / top-p sampling of the rollout batch (256 rows of
    the 151936-token vocabulary), averaged over back-to-back launches. The
    algorithmic bytes are one read of the logits (plus u and the tokens); the
    kernel reads each row several times (radix passes), mostly from cache."""
    import torch
    inp = W.sample_workload_inputs("rollout_sampling")
    lg, u = inp["logits"].to(dev), inp["u"].to(dev)
    tok = torch.empty(lg.shape[0], dtype=torch.int32, device=dev)

    def run():
        attn.sample(lg, u, inp["temperature"], inp["top_k"], inp["top_p"], tokens=tok)

    for _ in range(3):
        run()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record()
    for _ in range(iters):
        run()
    ev[1].record()
    ev[1].synchronize()
    t = ev[0].elapsed_time(ev[1]) / iters * 1e-3
    nbytes = lg.numel() * 4 + lg.shape[0] * 8
    return {"workload": "rollout_sampling (256 x 151936 fp32 logits, T 0.6, top-k 20, "
                        "top-p 0.95)",
            "us": round(t * 1e6, 2), "GB/s": round(nbytes / t / 1e9, 1),
            "hbm_peak_frac": round(nbytes / t / 1e9 / HBM_PEAK_GBPS, 4)}


def measured_peaks(dev):
    """Second denominators measured on this GPU by the probe library
    (libattn_probe.so): dense fp16 MFMA rate of independent 32x32x16 chains
    (1024 work-groups of 4 waves, 8 chains each) with the shader clock under
    that load, and the streaming-read rate of 16-byte non-temporal loads over
    2 GiB. Best of three runs each; None if the probe library is not built."""
    import ctypes
    import torch
    path = os.path.join(ROOT, "causal_gqa_attention_fa2_amd", "libattn_probe.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    vp = ctypes.c_void_p
    lib.probe_mfma_flops.argtypes = [ctypes.c_int, ctypes.c_int]
    lib.probe_mfma_flops.restype = ctypes.c_double
    lib.probe_mfma_f16.argtypes = [ctypes.c_int, ctypes.c_int, vp, vp, vp]
    lib.probe_mfma_f16.restype = ctypes.c_int
    lib.probe_stream_read.argtypes = [vp, ctypes.c_size_t, ctypes.c_int, vp, vp]
    lib.probe_stream_read.restype = ctypes.c_int
    stream = vp(torch.cuda.current_stream().cuda_stream)
    n_wg, iters = 1024, 2000
    out = torch.empty(n_wg * 256, dtype=torch.float32, device=dev)
    clocks = torch.zeros(2, dtype=torch.int64, device=dev)

    def timed(fn):
        fn()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record()
        fn()
        ev[1].record()
        ev[1].synchronize()
        return ev[0].elapsed_time(ev[1]) * 1e-3

    best_mfma, clock_ghz = 0.0, None
    for _ in range(3):
        t = timed(lambda: lib.probe_mfma_f16(n_wg, iters, vp(out.data_ptr()),
                                             vp(clocks.data_ptr()), stream))
        rate = lib.probe_mfma_flops(n_wg, iters) / t / 1e12
        if rate > best_mfma:
            best_mfma = rate
            ticks, real = (int(x) for x in clocks.cpu())
            clock_ghz = ticks / (real / 100e6) / 1e9 if real > 0 else None
    nbytes = 2 << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    rwg = 4096
    rout = torch.empty(rwg * 256, dtype=torch.int32, device=dev)
    best_read = 0.0
    for _ in range(3):
        t = timed(lambda: lib.probe_stream_read(vp(buf.data_ptr()), nbytes, rwg,
                                                vp(rout.data_ptr()), stream))
        best_read = max(best_read, nbytes / t / 1e9)
    del buf
    return {"mfma_f16_tflops": round(best_mfma, 1),
            "shader_clock_ghz_under_mfma": round(clock_ghz, 3) if clock_ghz else None,
            "stream_read_gbps": round(best_read, 1),
            "how": "probe_peaks.hip: 1024 x 4 waves x 8 independent 32x32x16 fp16 MFMA chains; "
                   "16-byte non-temporal reads of 2 GiB, 8 in flight per thread; best of 3"}


def _stats(ts):
    """Median / min / max of launch-time samples (seconds) in µs."""
    xs = sorted(ts)
    return {"median": round(xs[len(xs) // 2] * 1e6, 2), "min": round(xs[0] * 1e6, 2),
            "max": round(xs[-1] * 1e6, 2)}


def _rate(alg, ts, peak, scale):
    """Algorithmic work per launch over the median launch time, and its
    fraction of `peak` (`scale` converts to the unit of `peak`)."""
    xs = sorted(ts)
    r = alg / xs[len(xs) // 2] / scale
    return round(r, 2), round(r / peak, 4)


class TrainCase:
    """Resident inputs, outputs and workspace of one training workload, with
    the forward and backward as calls that allocate nothing."""

    def __init__(self, attn, W, name, dev):
        import torch
        self.name = name
        self.inp = W.workload_inputs(name)
        q, k, v, dout = (self.inp[n].to(dev) for n in ("q", "k", "v", "dout"))
        cu = self.inp["cu_seqlens"].to(dev)
        T, h_q, d = q.shape
        o = torch.empty_like(q)
        lse = torch.empty((h_q, T), dtype=torch.float32, device=dev)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        ms, sc = self.inp["max_seqlen"], self.inp["scale"]
        ws = torch.empty(max(attn.bwd_workspace_bytes(attn.varlen_dims(q, k, cu, ms)), 1),
                         dtype=torch.uint8, device=dev)
        self.fwd = lambda: attn.fwd(q, k, v, cu, sc, o=o, lse=lse, max_seqlen=ms)
        self.bwd = lambda: attn.bwd(q, k, v, o, lse, dout, cu, sc, dq=dq, dk=dk, dv=dv,
                                    max_seqlen=ms, workspace=ws)
        self.costs = train_costs(self.inp)


class DecodeCase:
    def __init__(self, attn, W, name, dev):
        import torch
        self.inp = de = W.decode_workload_inputs(name)
        q, kp, vp, bt, ctx = (de[n].to(dev) for n in ("q", "k_pool", "v_pool", "block_table",
                                                      "ctx_lens"))
        od = torch.empty_like(q)
        pdims = attn.paged_dims(q, kp, bt, de["max_ctx"])
        wsd = torch.empty(max(attn.decode_workspace_bytes(pdims), 1), dtype=torch.uint8,
                          device=dev)
        self.run = lambda: attn.decode_paged(q, kp, vp, bt, ctx, de["scale"], o=od,
                                             max_ctx_len=de["max_ctx"], workspace=wsd)
        self.costs = decode_costs(de)


# Length of the spin kernel that the timed launches queue behind (shader
# clock cycles, tens of milliseconds): longer than the host needs to enqueue
# them, so the GPU runs them back to back instead of waiting for each call.
SPIN_CYCLES = 60_000_000
# Samples (groups of back-to-back launches) behind each per-config median / min / max.
CONFIG_REPS = 5


def time_launches(fns, iters, reps=1, warm=2):
    """Mean launch time (seconds) of each function in `fns`: `reps` samples per
    function, each one event pair around `iters` back-to-back launches of it
    (the functions take turns, group by group). Everything is queued behind a
    spin kernel, so the events time the GPU work and not the host's launch
    overhead, and no event sits between two launches of a group (an event
    between kernels adds the drain of one before the next starts, several µs).
    Returns one list of `reps` samples per function."""
    import torch
    for _ in range(warm):
        for f in fns:
            f()
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in fns] for _ in range(reps)]
    torch.cuda.synchronize()
    torch.cuda._sleep(SPIN_CYCLES)
    for r in range(reps):
        for fi, f in enumerate(fns):
            ev[r][fi][0].record()
            for _ in range(iters):
                f()
            ev[r][fi][1].record()
    ev[-1][-1][1].synchronize()
    return [[ev[r][fi][0].elapsed_time(ev[r][fi][1]) * 1e-3 / iters for r in range(reps)]
            for fi in range(len(fns))]


def train_entry(case, t_fwd, t_bwd, with_rates=True):
    """Per-config object: fwd and bwd µs (median / min / max), TFLOP/s on the
    median and its fraction of the dense fp16 MFMA peak; fwd+bwd likewise."""
    f_fwd, f_bwd, b_fwd, b_bwd = case.costs
    e = {"fwd_us": _stats(t_fwd), "bwd_us": _stats(t_bwd),
         "tokens": case.inp["total_tokens"], "max_seqlen": case.inp["max_seqlen"]}
    if with_rates:
        for nm, alg, ts in (("fwd", f_fwd, t_fwd), ("bwd", f_bwd, t_bwd)):
            r, fr = _rate(alg, ts, MFMA_F16_PEAK_TFLOPS, 1e12)
            e[f"{nm}_TFLOP/s"] = r
            e[f"{nm}_mfma_peak_frac"] = fr
        tot = [a + b for a, b in zip(t_fwd, t_bwd)]
        r, fr = _rate(f_fwd + f_bwd, tot, MFMA_F16_PEAK_TFLOPS, 1e12)
        e["fwd+bwd_TFLOP/s"] = r
        e["fwd+bwd_mfma_peak_frac"] = fr
        e["fwd_hbm_GB/s"] = round(b_fwd / sorted(t_fwd)[len(t_fwd) // 2] / 1e9, 1)
    return e


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the measured-peak probes (MFMA rate, streaming read)")
    ap.add_argument("--no-extras", action="store_true",
                    help="time only the step (long_context fwd+bwd, paged_decode) and the "
                         "per-config training rows; skip prefill, RMSNorm, sampling, RoPE")
    ap.add_argument("--warm-seconds", type=float, default=1.0,
                    help="untimed steady-state run before the timed steps")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 256 MiB device-to-device copy (4 launches), the "
                         "known-size kernel that scales the HBM byte counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(the attention path here runs on a single MI355X).", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_calibration:
        n = 256 << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(4):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration": {"bytes_read": n, "bytes_written": n,
                                               "launches": 4}}), flush=True)
        return
    import causal_gqa_attention_fa2_amd as attn
    from causal_gqa_attention_fa2_amd import workloads as W

    dev = torch.device("cuda:0")
    tr = TrainCase(attn, W, TRAIN_WORKLOAD, dev)
    dc = DecodeCase(attn, W, DECODE_WORKLOAD, dev)

    def step(ev=None):
        if ev:
            ev[0].record()
        tr.fwd()
        if ev:
            ev[1].record()
        tr.bwd()
        if ev:
            ev[2].record()
        dc.run()
        if ev:
            ev[3].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # Bring the GPU to its steady clock before the timed steps (a cold GPU
    # runs the first tens of milliseconds ~10% slower).
    t_warm = time.perf_counter()
    while time.perf_counter() - t_warm < args.warm_seconds:
        step()
        torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ts_fwd = [e[0].elapsed_time(e[1]) * 1e-3 for e in evs]
    ts_bwd = [e[1].elapsed_time(e[2]) * 1e-3 for e in evs]
    ts_dec = [e[2].elapsed_time(e[3]) * 1e-3 for e in evs]
    t_fwd = sum(ts_fwd) / args.steps
    t_bwd = sum(ts_bwd) / args.steps
    t_dec = sum(ts_dec) / args.steps

    f_fwd, f_bwd, b_fwd, b_bwd = tr.costs
    f_dec, b_dec = dc.costs
    tflops = (f_fwd + f_bwd) / (t_fwd + t_bwd) / 1e12
    dec_gbps = b_dec / t_dec / 1e9

    parts = {
        "attn_fwd": dict(t=t_fwd, bound="mfma", achieved=f_fwd / t_fwd / 1e12,
                         peak=MFMA_F16_PEAK_TFLOPS, unit="TFLOP/s", alg=f_fwd,
                         launches=["fwd_kernel<128, false, false, 8>"]),
        "attn_bwd": dict(t=t_bwd, bound="mfma", achieved=f_bwd / t_bwd / 1e12,
                         peak=MFMA_F16_PEAK_TFLOPS, unit="TFLOP/s", alg=f_bwd,
                         launches=["dq_kernel<128, false>", "dkdv_kernel<128, false, false>"]),
        "attn_decode_paged": dict(t=t_dec, bound="hbm", achieved=dec_gbps, peak=HBM_PEAK_GBPS,
                                  unit="GB/s", alg=b_dec,
                                  launches=["decode_plan_kernel", "decode_gather_kernel<128, 2>",
                                            "decode_combine_kernel<128>"]),
    }
    dom = max(parts, key=lambda n: parts[n]["t"])
    p = parts[dom]
    wl = DECODE_WORKLOAD if dom == "attn_decode_paged" else TRAIN_WORKLOAD
    roofline = {"kernel": dom, "workload": wl, "launches": p["launches"], "bound": p["bound"],
                "achieved": round(p["achieved"], 2), "peak": p["peak"], "unit": p["unit"],
                "frac": round(p["achieved"] / p["peak"], 4),
                "avg_launch_us": round(p["t"] * 1e6, 2),
                "traffic": read_traffic(dom, wl)}

    configs = {"long_context": train_entry(tr, ts_fwd, ts_bwd)}
    configs["long_context"]["source"] = "the timed steps"
    for name in ("tiny", "qwen3_train", "grpo_varlen", "long_context_tp8"):
        c = TrainCase(attn, W, name, dev)
        tf, tb = time_launches([c.fwd, c.bwd], max(args.steps, 20), reps=CONFIG_REPS)
        configs[name] = train_entry(c, tf, tb, with_rates=name != "tiny")
        del c
    configs[DECODE_WORKLOAD] = {"us": _stats(ts_dec), "GB/s": round(b_dec / sorted(ts_dec)[
        len(ts_dec) // 2] / 1e9, 1), "hbm_peak_frac": round(b_dec / sorted(ts_dec)[
            len(ts_dec) // 2] / 1e9 / HBM_PEAK_GBPS, 4), "alg_bytes": int(b_dec),
        "source": "the timed steps"}
    order = ["tiny", "qwen3_train", "grpo_varlen", "long_context", "long_context_tp8",
             DECODE_WORKLOAD]
    configs = {k: configs[k] for k in order}

    out = {
        "metric": "attn fwd+bwd TFLOP/s & % FP16 MFMA peak; paged-decode HBM GB/s",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic",
        "config": {
            "workload": "long_context fwd+bwd (B=4, S=8192, H_q=16, H_kv=8, d=128, causal) + "
                        "paged_decode (256 seqs, ctx U{128..4096}, block 16, H_q=16, H_kv=8, "
                        "d=128)",
            "global_batch": 4, "seq_len": 8192, "parallelism": "single-gpu",
        },
        "mfma_peak_frac": round(tflops / MFMA_F16_PEAK_TFLOPS, 4),
        "fwd": {"us": round(t_fwd * 1e6, 2), "TFLOP/s": round(parts["attn_fwd"]["achieved"], 2),
                "GB/s": round(b_fwd / t_fwd / 1e9, 1)},
        "bwd": {"us": round(t_bwd * 1e6, 2), "TFLOP/s": round(parts["attn_bwd"]["achieved"], 2),
                "GB/s": round(b_bwd / t_bwd / 1e9, 1), "launches": 2},
        "decode": {"us": round(t_dec * 1e6, 2), "GB/s": round(dec_gbps, 1),
                   "hbm_peak_frac": round(dec_gbps / HBM_PEAK_GBPS, 4),
                   "alg_bytes": int(b_dec), "launches": 3},
        "roofline": roofline,
        "configs": configs,
        "source_digest": source_digest(),
    }
    peaks = None if args.no_peaks else measured_peaks(dev)
    if peaks:
        out["measured_peaks"] = peaks
        out["mfma_measured_frac"] = round(tflops / peaks["mfma_f16_tflops"], 4)
        out["decode"]["hbm_measured_frac"] = round(dec_gbps / peaks["stream_read_gbps"], 4)
    if not args.no_extras:
        out["prefill"] = bench_prefill(attn, W, dev, max(args.steps, 5))
        out["rmsnorm"] = bench_rmsnorm(attn, W, dev, max(args.steps, 5))
        out["sampling"] = bench_sampling(attn, W, dev, max(args.steps, 5))
        out["rope"] = bench_rope(attn, W, dev, max(args.steps, 5))
    if not args.no_cpu_baseline:
        cb = cpu_baseline(args.cpu_budget)
        cb.pop("seconds", None)
        out["cpu_baseline"] = cb
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
