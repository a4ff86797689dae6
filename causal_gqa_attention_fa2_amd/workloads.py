"""Seeded synthetic inputs for the attention workloads.

This module holds no attention arithmetic: it only draws lengths, tensors,
block tables and paged pools. Both the HIP path and the CPU oracle are fed
from it (through the tests, the benchmark and the smoke check), so the two
sides always see bit-identical fp16 inputs.

Recipe. Values are N(0, 1) drawn in fp32 from a CPU ``torch.Generator`` and
rounded to fp16 (round-to-nearest-even). Draw order: lengths (or context
lengths and the block permutation) first, then q, k, v, dO. Packed layouts:
q, dO [T, H_q, d]; k, v [T, H_kv, d]; paged pools [num_blocks, 16, H_kv, d].

Workloads (shapes of the RL.cu stack's Qwen3-0.6B attention; pitchhut
"Project Highlights", mlllm.io "What happened"):

* ``tiny``          B=1, S=64, H_q=2, H_kv=1, d=64
* ``qwen3_train``   B=8, S=1024, H_q=16, H_kv=8, d=128
* ``grpo_varlen``   4 prompts x 8 samples, prompt U{64..256} shared by a
  prompt's samples, completion U{128..1024} per sample, packed prompt-major
* ``long_context``  B=4, S=8192, H_q=16, H_kv=8, d=128
* ``long_context_tp8`` the same batch at one GPU's share of an 8-way split by
  KV head: H_q=2, H_kv=1, d=128
* ``paged_decode``  256 sequences, ctx U{128..4096}, block 16, H_q=16,
  H_kv=8, d=128; the logical blocks of all sequences (in order) receive a
  seeded random permutation of the physical blocks.
* ``paged_prefill`` one chunked-prefill step of a GRPO group: 32 sequences
  with a cached context U{0..1536} and a new chunk U{128..512}, block 16,
  H_q=16, H_kv=8, d=128; blocks permuted as for the decode.
* ``rollout_sampling`` 256 rows of Qwen3's 151936-token vocabulary, logits
  3 N(0,1), temperature 0.6, top-k 20, top-p 0.95, one uniform per row.
* ``qwen3_rmsnorm`` the layer RMSNorm of the training batch: 8192 rows
  (B=8 x S=1024) of hidden size 1024; ``qwen3_qknorm`` the per-head
  query norm: 8192 x 16 rows of 128. x, dy ~ N(0,1); w = 1 + 0.1 N(0,1).
"""
import math

import torch

TRAIN_WORKLOADS = {
    "tiny": dict(seqlens=[64], h_q=2, h_kv=1, d=64, seed=1000),
    "qwen3_train": dict(seqlens=[1024] * 8, h_q=16, h_kv=8, d=128, seed=1001),
    "grpo_varlen": dict(seqlens=None, h_q=16, h_kv=8, d=128, seed=1002),
    "long_context": dict(seqlens=[8192] * 4, h_q=16, h_kv=8, d=128, seed=1003),
    # One GPU's share of long_context split 8 ways by KV head (tensor
    # parallel): one KV head and its two query heads.
    "long_context_tp8": dict(seqlens=[8192] * 4, h_q=2, h_kv=1, d=128, seed=1007),
}
DECODE_WORKLOADS = {
    "paged_decode": dict(n=256, ctx_lo=128, ctx_hi=4096, block_size=16,
                         h_q=16, h_kv=8, d=128, seed=1004),
}
SAMPLE_WORKLOADS = {
    "rollout_sampling": dict(n=256, vocab=151936, scale=3.0, temperature=0.6, top_k=20,
                             top_p=0.95, seed=1008),
}
NORM_WORKLOADS = {
    "qwen3_rmsnorm": dict(rows=8192, n=1024, seed=1006),
    "qwen3_qknorm": dict(rows=8192 * 16, n=128, seed=1007),
}
PREFILL_WORKLOADS = {
    "paged_prefill": dict(n=32, prior_lo=0, prior_hi=1536, new_lo=128, new_hi=512,
                          block_size=16, h_q=16, h_kv=8, d=128, seed=1005),
}
BLOCK_SIZE = 16


def _gen(seed):
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return g


def _randn_f16(shape, g, chunk=1 << 24):
    """N(0,1) in fp32 rounded to fp16, drawn in chunks to bound host memory."""
    out = torch.empty(shape, dtype=torch.float16)
    flat = out.view(-1)
    for i in range(0, flat.numel(), chunk):
        n = min(chunk, flat.numel() - i)
        flat[i:i + n] = torch.randn(n, generator=g, dtype=torch.float32).half()
    return out


def grpo_seqlens(g, prompts=4, samples=8, prompt_range=(64, 256),
                 completion_range=(128, 1024)):
    """Sequence lengths of a GRPO group batch: one prompt length per prompt
    shared by its samples, one completion length per sample."""
    lens = []
    for _ in range(prompts):
        p = int(torch.randint(prompt_range[0], prompt_range[1] + 1, (1,), generator=g))
        for _ in range(samples):
            c = int(torch.randint(completion_range[0], completion_range[1] + 1, (1,),
                                  generator=g))
            lens.append(p + c)
    return lens


def cu_from_lens(seqlens):
    cu = [0]
    for L in seqlens:
        cu.append(cu[-1] + int(L))
    return torch.tensor(cu, dtype=torch.int32)


def make_train_inputs(seqlens, h_q, h_kv, d, seed, with_dout=True):
    """Packed varlen q, k, v (and dO) in fp16 with their ``cu_seqlens``."""
    g = _gen(seed)
    if seqlens is None:
        seqlens = grpo_seqlens(g)
    cu = cu_from_lens(seqlens)
    T = int(cu[-1])
    q = _randn_f16((T, h_q, d), g)
    k = _randn_f16((T, h_kv, d), g)
    v = _randn_f16((T, h_kv, d), g)
    dout = _randn_f16((T, h_q, d), g) if with_dout else None
    return dict(q=q, k=k, v=v, dout=dout, cu_seqlens=cu, seqlens=list(seqlens),
                max_seqlen=max(seqlens) if seqlens else 0, total_tokens=T,
                h_q=h_q, h_kv=h_kv, d=d, scale=1.0 / math.sqrt(d))


def workload_inputs(name, with_dout=True):
    w = TRAIN_WORKLOADS[name]
    return make_train_inputs(w["seqlens"], w["h_q"], w["h_kv"], w["d"], w["seed"],
                             with_dout=with_dout)


def make_decode_inputs(ctx_lens, h_q, h_kv, d, seed, block_size=BLOCK_SIZE,
                       max_blocks=None, spare_blocks=0):
    """Single-token queries and a paged pool holding each sequence's context.

    Physical blocks: num_blocks = sum(ceil(ctx/bs)) + ``spare_blocks``. The
    logical blocks of all sequences, taken in order, map through a seeded
    random permutation; table entries past a sequence's last block hold -1.
    """
    g = _gen(seed)
    ctx = [int(c) for c in ctx_lens]
    nblk = [math.ceil(c / block_size) for c in ctx]
    used = sum(nblk)
    num_blocks = used + int(spare_blocks)
    if max_blocks is None:
        max_blocks = max(1, max(nblk) if nblk else 1)
    perm = torch.randperm(num_blocks, generator=g)[:used].to(torch.int32)
    table = torch.full((len(ctx), max_blocks), -1, dtype=torch.int32)
    pos = 0
    for b, nb in enumerate(nblk):
        table[b, :nb] = perm[pos:pos + nb]
        pos += nb
    n = len(ctx)
    q = _randn_f16((n, h_q, d), g)
    k_pool = _randn_f16((num_blocks, block_size, h_kv, d), g)
    v_pool = _randn_f16((num_blocks, block_size, h_kv, d), g)
    return dict(q=q, k_pool=k_pool, v_pool=v_pool, block_table=table,
                ctx_lens=torch.tensor(ctx, dtype=torch.int32), n=n, h_q=h_q,
                h_kv=h_kv, d=d, block_size=block_size, num_blocks=num_blocks,
                max_blocks=max_blocks, max_ctx=max(ctx) if ctx else 0,
                scale=1.0 / math.sqrt(d))


def decode_workload_inputs(name="paged_decode"):
    w = DECODE_WORKLOADS[name]
    g = _gen(w["seed"])
    ctx = torch.randint(w["ctx_lo"], w["ctx_hi"] + 1, (w["n"],), generator=g).tolist()
    max_blocks = math.ceil(w["ctx_hi"] / w["block_size"])
    return make_decode_inputs(ctx, w["h_q"], w["h_kv"], w["d"], w["seed"] + 7919,
                              block_size=w["block_size"], max_blocks=max_blocks)


def poison_unused(inp):
    """NaN into every pool slot no sequence uses (tail slots of last blocks,
    spare blocks). Returns a new dict with cloned pools."""
    k_pool = inp["k_pool"].clone()
    v_pool = inp["v_pool"].clone()
    bs = inp["block_size"]
    used = torch.zeros(k_pool.shape[0], bs, dtype=torch.bool)
    for b in range(inp["n"]):
        c = int(inp["ctx_lens"][b])
        for lb in range(math.ceil(c / bs)):
            phys = int(inp["block_table"][b, lb])
            used[phys, :min(bs, c - lb * bs)] = True
    k_pool[~used] = float("nan")
    v_pool[~used] = float("nan")
    out = dict(inp)
    out.update(k_pool=k_pool, v_pool=v_pool)
    return out


def make_prefill_inputs(prior_lens, new_lens, h_q, h_kv, d, seed, block_size=BLOCK_SIZE,
                        max_blocks=None, spare_blocks=0):
    """A chunked prefill step: sequence b has ``prior_lens[b]`` cached tokens
    and ``new_lens[b]`` new ones (ctx_lens = prior + new, the new tokens are
    the last positions). Draw order: block permutation, then q, k_new, v_new
    [total_q, heads, d] packed by cu_q, then the pools. The pools hold random
    values everywhere, including the slots the new tokens will be appended
    to (stale data the append must overwrite); table entries past a
    sequence's last block hold -1.
    """
    g = _gen(seed)
    prior = [int(c) for c in prior_lens]
    new = [int(c) for c in new_lens]
    ctx = [a + b for a, b in zip(prior, new)]
    nblk = [math.ceil(c / block_size) for c in ctx]
    used = sum(nblk)
    num_blocks = used + int(spare_blocks)
    if max_blocks is None:
        max_blocks = max(1, max(nblk) if nblk else 1)
    perm = torch.randperm(num_blocks, generator=g)[:used].to(torch.int32)
    table = torch.full((len(ctx), max_blocks), -1, dtype=torch.int32)
    pos = 0
    for b, nb in enumerate(nblk):
        table[b, :nb] = perm[pos:pos + nb]
        pos += nb
    cu_q = cu_from_lens(new)
    Tq = int(cu_q[-1])
    q = _randn_f16((Tq, h_q, d), g)
    k_new = _randn_f16((Tq, h_kv, d), g)
    v_new = _randn_f16((Tq, h_kv, d), g)
    k_pool = _randn_f16((num_blocks, block_size, h_kv, d), g)
    v_pool = _randn_f16((num_blocks, block_size, h_kv, d), g)
    return dict(q=q, k_new=k_new, v_new=v_new, cu_q=cu_q, k_pool=k_pool, v_pool=v_pool,
                block_table=table, ctx_lens=torch.tensor(ctx, dtype=torch.int32),
                prior_lens=prior, new_lens=new, n=len(ctx), total_q=Tq,
                max_q_len=max(new) if new else 0, max_ctx=max(ctx) if ctx else 0,
                h_q=h_q, h_kv=h_kv, d=d, block_size=block_size, num_blocks=num_blocks,
                max_blocks=max_blocks, scale=1.0 / math.sqrt(d))


def prefill_workload_inputs(name="paged_prefill"):
    w = PREFILL_WORKLOADS[name]
    g = _gen(w["seed"])
    prior = torch.randint(w["prior_lo"], w["prior_hi"] + 1, (w["n"],), generator=g).tolist()
    new = torch.randint(w["new_lo"], w["new_hi"] + 1, (w["n"],), generator=g).tolist()
    max_blocks = math.ceil((w["prior_hi"] + w["new_hi"]) / w["block_size"])
    return make_prefill_inputs(prior, new, w["h_q"], w["h_kv"], w["d"], w["seed"] + 7919,
                               block_size=w["block_size"], max_blocks=max_blocks)


def poison_unused_prefill(inp):
    """NaN into every pool slot outside all contexts (tail slots of last
    blocks, spare blocks). Returns a new dict with cloned pools."""
    k_pool = inp["k_pool"].clone()
    v_pool = inp["v_pool"].clone()
    bs = inp["block_size"]
    used = torch.zeros(k_pool.shape[0], bs, dtype=torch.bool)
    for b in range(inp["n"]):
        c = int(inp["ctx_lens"][b])
        for lb in range(math.ceil(c / bs)):
            phys = int(inp["block_table"][b, lb])
            used[phys, :min(bs, c - lb * bs)] = True
    k_pool[~used] = float("nan")
    v_pool[~used] = float("nan")
    out = dict(inp)
    out.update(k_pool=k_pool, v_pool=v_pool)
    return out


def make_norm_inputs(rows, n, seed):
    """RMSNorm inputs: x [rows, n], dy [rows, n] ~ N(0,1) and a weight
    w [n] = 1 + 0.1 N(0,1), all fp16 (draw order w, x, dy)."""
    g = _gen(seed)
    w = (1.0 + 0.1 * torch.randn(n, generator=g, dtype=torch.float32)).half()
    x = _randn_f16((rows, n), g)
    dy = _randn_f16((rows, n), g)
    return dict(x=x, w=w, dy=dy, rows=rows, n=n, eps=1e-6)


def norm_workload_inputs(name):
    w = NORM_WORKLOADS[name]
    return make_norm_inputs(w["rows"], w["n"], w["seed"])


def make_sample_inputs(n, vocab, scale, seed, step=None, masked=0.0, offset=0.0):
    """Logits [n, vocab] = offset + scale N(0,1) in fp32 (rounded to multiples of
    `step` when given, which creates ties; a `masked` fraction set to -inf,
    never the first entry of a row) and uniforms u [n] in [0, 1). Draw
    order: logits, mask, u."""
    g = _gen(seed)
    logits = torch.randn(n, vocab, generator=g, dtype=torch.float32) * scale + offset
    if step:
        logits = torch.round(logits / step) * step
    if masked > 0:
        m = torch.rand(n, vocab, generator=g) < masked
        m[:, 0] = False
        logits[m] = float("-inf")
    u = torch.rand(n, generator=g, dtype=torch.float32)
    return dict(logits=logits, u=u, n=n, vocab=vocab)


def sample_workload_inputs(name="rollout_sampling"):
    w = SAMPLE_WORKLOADS[name]
    inp = make_sample_inputs(w["n"], w["vocab"], w["scale"], w["seed"])
    inp.update(temperature=w["temperature"], top_k=w["top_k"], top_p=w["top_p"])
    return inp
