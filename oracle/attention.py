"""fp64 reference for causal GQA attention: forward, backward, paged decode.

TEST INFRASTRUCTURE ONLY (see the package docstring). Nothing in the HIP
library or its binding may import this module.

Sources. The RL.cu pages (pitchhut "Project Highlights"; mlllm.io "What
happened") name FlashAttention-2 forward and backward kernels and a paged
key/value cache (pitchhut "Key Features", item 2); they print no formula.
FlashAttention-2 computes exact softmax attention, so each function below is
that definition written out, one (sequence, query head) at a time, with no
online softmax, no tiling over keys and no fusion. Readings of points the
pages leave open:

* causal mask keeps key j for query i iff j <= i, positions counted from each
  sequence's start (queries and keys of a sequence have the same length);
* attention never crosses a sequence boundary of the packed batch
  (``cu_seqlens`` gives the boundaries, shared by queries and keys);
* grouped-query head map: query head h reads key/value head h // G with
  G = H_q / H_kv (contiguous groups);
* ``scale`` multiplies q.k before masking and softmax; the saved log-sum-exp
  is the natural logarithm of sum_j exp(scaled score);
* the backward cotangent is dO only (no gradient flows into the LSE);
* decode: the single query of sequence b attends to context positions
  t < ctx_lens[b]; position t lives in physical block block_table[b][t // bs]
  at slot t % bs; a context of length 0 yields a zero output row.

Layouts (all row-major): q, o, dO, dq [T, H_q, d]; k, v, dk, dv [T, H_kv, d];
lse [H_q, T]; pools [num_blocks, bs, H_kv, d]; block_table [n, max_blocks].
Rows are processed in chunks of at most ``ROW_CHUNK`` queries only to bound
memory; every row still sees its full score vector at once.
"""
import numpy as np

ROW_CHUNK = 1024


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def kv_head_of(h, h_q, h_kv):
    """Key/value head read by query head ``h``: contiguous groups of
    G = h_q // h_kv query heads share one key/value head."""
    return h // (h_q // h_kv)


def _masked_scores(q_rows, keys, row0, scale):
    """scale * q_rows @ keys^T with the causal mask applied.

    ``q_rows`` are the sequence's queries at local positions row0.., ``keys``
    its keys at local positions 0..len(keys)-1. Disallowed pairs (key position
    greater than query position) become -inf.
    """
    s = scale * (q_rows @ keys.T)
    qpos = np.arange(row0, row0 + q_rows.shape[0])[:, None]
    kpos = np.arange(keys.shape[0])[None, :]
    return np.where(kpos <= qpos, s, -np.inf)


def _softmax_rows(s):
    """Row-wise softmax and natural-log log-sum-exp of a score matrix whose
    rows each hold at least one finite entry."""
    m = s.max(axis=1, keepdims=True)
    lse = m[:, 0] + np.log(np.exp(s - m).sum(axis=1))
    p = np.exp(s - lse[:, None])
    return p, lse


def _softmax_grad(p, dp):
    """Gradient wrt the scores of a row softmax: dS = P * (dP - rowsum(P * dP))."""
    return p * (dp - (p * dp).sum(axis=1, keepdims=True))


def _paged_positions(table_row, ctx, bs):
    """(physical block, slot) of context positions 0..ctx-1 of one sequence."""
    t = np.arange(ctx)
    return table_row[t // bs], t % bs


def _check_shapes(q, k, v, cu):
    if q.ndim != 3 or k.ndim != 3 or v.ndim != 3:
        raise ValueError("q, k, v must be [T, heads, d]")
    T, h_q, d = q.shape
    if k.shape != v.shape or k.shape[0] != T or k.shape[2] != d:
        raise ValueError("k and v must be [T, H_kv, d] matching q")
    h_kv = k.shape[1]
    if h_kv <= 0 or h_q % h_kv:
        raise ValueError("H_q must be a multiple of H_kv")
    if cu.ndim != 1 or cu[0] != 0 or cu[-1] != T or np.any(np.diff(cu) < 0):
        raise ValueError("cu_seqlens must rise from 0 to T")
    return T, h_q, h_kv, d


def attn_fwd_ref(q, k, v, cu_seqlens, scale):
    """Causal GQA softmax attention forward.

    Returns (o [T, H_q, d] float64, lse [H_q, T] float64). For query i of a
    sequence and its head h (key/value head g = h // G):
    S_ij = scale * <q_i, k_j> for j <= i; LSE_i = log sum_j exp(S_ij);
    O_i = sum_j exp(S_ij - LSE_i) v_j.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    T, h_q, h_kv, d = _check_shapes(q, k, v, cu)
    o = np.zeros((T, h_q, d))
    lse = np.zeros((h_q, T))
    for b in range(len(cu) - 1):
        s0, e0 = int(cu[b]), int(cu[b + 1])
        L = e0 - s0
        for h in range(h_q):
            g = kv_head_of(h, h_q, h_kv)
            Q, K, V = q[s0:e0, h], k[s0:e0, g], v[s0:e0, g]
            for r0 in range(0, L, ROW_CHUNK):
                r1 = min(L, r0 + ROW_CHUNK)
                s = _masked_scores(Q[r0:r1], K[:r1], r0, scale)
                p, lse_rows = _softmax_rows(s)
                o[s0 + r0:s0 + r1, h] = p @ V[:r1]
                lse[h, s0 + r0:s0 + r1] = lse_rows
    return o, lse


def attn_bwd_ref(q, k, v, dout, cu_seqlens, scale):
    """Analytic backward of ``attn_fwd_ref`` for the loss <O, dout>.

    Chain rule through O = P V and P = softmax(S), S = scale * Q K^T:
    dV_j = sum_i P_ij dO_i; dP_ij = <dO_i, v_j>;
    dS_ij = P_ij (dP_ij - sum_l P_il dP_il);
    dQ_i = scale * sum_j dS_ij k_j; dK_j = scale * sum_i dS_ij q_i.
    Gradients of a key/value head sum over the G query heads that read it.
    Returns (dq [T, H_q, d], dk [T, H_kv, d], dv [T, H_kv, d]) in float64.
    """
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    T, h_q, h_kv, d = _check_shapes(q, k, v, cu)
    if dout.shape != q.shape:
        raise ValueError("dout must match q")
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(len(cu) - 1):
        s0, e0 = int(cu[b]), int(cu[b + 1])
        L = e0 - s0
        for h in range(h_q):
            g = kv_head_of(h, h_q, h_kv)
            Q, K, V, dO = q[s0:e0, h], k[s0:e0, g], v[s0:e0, g], dout[s0:e0, h]
            for r0 in range(0, L, ROW_CHUNK):
                r1 = min(L, r0 + ROW_CHUNK)
                s = _masked_scores(Q[r0:r1], K[:r1], r0, scale)
                p, _ = _softmax_rows(s)
                dp = dO[r0:r1] @ V[:r1].T
                ds = _softmax_grad(p, dp)
                dq[s0 + r0:s0 + r1, h] = scale * (ds @ K[:r1])
                dk[s0:s0 + r1, g] += scale * (ds.T @ Q[r0:r1])
                dv[s0:s0 + r1, g] += p.T @ dO[r0:r1]
    return dq, dk, dv


def attn_decode_ref(q, k_pool, v_pool, block_table, ctx_lens, scale):
    """Single-query attention over a paged key/value pool.

    q [n, H_q, d]; k_pool, v_pool [num_blocks, bs, H_kv, d];
    block_table [n, max_blocks] (physical block of each logical block);
    ctx_lens [n]. Position t of sequence b is slot t % bs of physical block
    block_table[b][t // bs]. Only the used entries are gathered, so unused
    slots and table entries never reach the arithmetic. Returns o [n, H_q, d]
    float64; a zero-length context gives a zero row.
    """
    q = _f64(q)
    k_pool = np.asarray(k_pool)
    v_pool = np.asarray(v_pool)
    bt = np.asarray(block_table, dtype=np.int64)
    ctx = np.asarray(ctx_lens, dtype=np.int64)
    n, h_q, d = q.shape
    nb, bs, h_kv, d2 = k_pool.shape
    if d2 != d or v_pool.shape != k_pool.shape or h_q % h_kv:
        raise ValueError("pool / query shapes disagree")
    o = np.zeros((n, h_q, d))
    for b in range(n):
        c = int(ctx[b])
        if c == 0:
            continue
        phys, slot = _paged_positions(bt[b], c, bs)
        if np.any(phys < 0) or np.any(phys >= nb):
            raise ValueError("block_table entry out of range")
        K = _f64(k_pool[phys, slot])  # [c, H_kv, d]
        V = _f64(v_pool[phys, slot])
        for h in range(h_q):
            g = kv_head_of(h, h_q, h_kv)
            s = scale * (K[:, g] @ q[b, h])
            w = np.exp(s - s.max())
            o[b, h] = (w / w.sum()) @ V[:, g]
    return o


# ----------------------------------------------------------------------------- paged prefill
#
# The rollout engine's other attention call (pitchhut "Key Features", item 2:
# continuous batching over a paged key/value cache; mlllm.io "What happened"):
# a chunk of new tokens of each sequence is appended to the cache and attends
# causally to the whole cached context. Readings of points the pages leave
# open: ``ctx_lens[b]`` counts the context INCLUDING the sequence's new tokens,
# which are its last q_len_b = cu_q[b+1] - cu_q[b] positions; new token i of
# sequence b therefore sits at context position ctx_b - q_len_b + i and sees
# positions 0 .. ctx_b - q_len_b + i.


def _chunk_offset(ctx, q_len):
    """Context position of a sequence's first new token (its new tokens are
    the last ``q_len`` of its ``ctx`` positions)."""
    if q_len < 0 or q_len > ctx:
        raise ValueError("a chunk cannot be longer than its context")
    return ctx - q_len


def kv_append_ref(k_pool, v_pool, k_new, v_new, cu_q, block_table, ctx_lens):
    """Write each sequence's new keys and values into the paged pools.

    k_new, v_new [Tq, H_kv, d] packed by ``cu_q``; new token i of sequence b
    goes to context position t = ctx_b - q_len_b + i, i.e. slot t % bs of
    physical block block_table[b][t // bs]. Returns new (k_pool, v_pool)
    arrays (copies, input dtype); every other slot is left as it was.
    """
    kp = np.array(k_pool, copy=True)
    vp = np.array(v_pool, copy=True)
    k_new = np.asarray(k_new)
    v_new = np.asarray(v_new)
    cu = np.asarray(cu_q, dtype=np.int64)
    bt = np.asarray(block_table, dtype=np.int64)
    ctx = np.asarray(ctx_lens, dtype=np.int64)
    bs = kp.shape[1]
    for b in range(len(cu) - 1):
        s0, e0 = int(cu[b]), int(cu[b + 1])
        c = int(ctx[b])
        off = _chunk_offset(c, e0 - s0)
        phys, slot = _paged_positions(bt[b], c, bs)
        phys, slot = phys[off:], slot[off:]
        if np.any(phys < 0) or np.any(phys >= kp.shape[0]):
            raise ValueError("block_table entry out of range")
        kp[phys, slot] = k_new[s0:e0]
        vp[phys, slot] = v_new[s0:e0]
    return kp, vp


def attn_prefill_ref(q, k_pool, v_pool, block_table, ctx_lens, cu_q, scale):
    """Causal GQA attention of new query tokens against a paged context.

    q [Tq, H_q, d] packed by ``cu_q``; pools [num_blocks, bs, H_kv, d];
    ``ctx_lens`` include the new tokens. New token i of sequence b (context
    position p = ctx_b - q_len_b + i) attends to context positions 0..p,
    gathered from the pools; S, LSE and O as in ``attn_fwd_ref``. Returns
    (o [Tq, H_q, d], lse [H_q, Tq]) in float64.
    """
    q = _f64(q)
    k_pool = np.asarray(k_pool)
    v_pool = np.asarray(v_pool)
    cu = np.asarray(cu_q, dtype=np.int64)
    bt = np.asarray(block_table, dtype=np.int64)
    ctx = np.asarray(ctx_lens, dtype=np.int64)
    Tq, h_q, d = q.shape
    nb, bs, h_kv, d2 = k_pool.shape
    if d2 != d or v_pool.shape != k_pool.shape or h_q % h_kv:
        raise ValueError("pool / query shapes disagree")
    if cu.ndim != 1 or cu[0] != 0 or cu[-1] != Tq or np.any(np.diff(cu) < 0):
        raise ValueError("cu_q must rise from 0 to Tq")
    o = np.zeros((Tq, h_q, d))
    lse = np.zeros((h_q, Tq))
    for b in range(len(cu) - 1):
        s0, e0 = int(cu[b]), int(cu[b + 1])
        if e0 == s0:
            continue
        c = int(ctx[b])
        off = _chunk_offset(c, e0 - s0)
        phys, slot = _paged_positions(bt[b], c, bs)
        if np.any(phys < 0) or np.any(phys >= nb):
            raise ValueError("block_table entry out of range")
        K = _f64(k_pool[phys, slot])  # [c, H_kv, d]
        V = _f64(v_pool[phys, slot])
        for h in range(h_q):
            g = kv_head_of(h, h_q, h_kv)
            for r0 in range(0, e0 - s0, ROW_CHUNK):
                r1 = min(e0 - s0, r0 + ROW_CHUNK)
                s = _masked_scores(q[s0 + r0:s0 + r1, h], K[:off + r1, g], off + r0, scale)
                p, lse_rows = _softmax_rows(s)
                o[s0 + r0:s0 + r1, h] = p @ V[:off + r1, g]
                lse[h, s0 + r0:s0 + r1] = lse_rows
    return o, lse
