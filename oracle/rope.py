"""fp64 reference for rotary position embedding (RoPE).

TEST INFRASTRUCTURE ONLY (see the package docstring). Nothing in the HIP
library or its binding may import this module.

Source: the mlllm.io article ("What happened") lists RoPE among the
hand-written kernels of the RL.cu stack, next to FlashAttention-2 and
RMSNorm; the pages print no formula, no pairing and no frequency base.

Readings (the plainest ones the rest of the pages support; the model the
benchmarks run is Qwen3-0.6B, whose RoPE is this one):

* Dimension j < d/2 of a head is paired with dimension j + d/2 ("rotate
  half", the NeoX layout), and the pair is turned by the angle pos * f_j,
  f_j = base ** (-2 j / d):

    y_j         = x_j cos(pos f_j) - x_{j+d/2} sin(pos f_j)
    y_{j+d/2}   = x_{j+d/2} cos(pos f_j) + x_j sin(pos f_j)

* The kernels take the cos / sin values as fp32 tables [max_pos, d/2]
  (``rope_tables_ref`` gives them in fp64; the caller's tables are those
  rounded to fp32). ``rope_ref`` applies whatever tables it is given, in
  fp64.
* The rotation feeds fp16 attention: its output is rounded to fp16 (round
  to nearest even) before attention reads it, as an unfused RoPE kernel
  that stores fp16 would. ``rope_fp16_ref`` is that rounding.
* The backward of y = R(pos) x is dx = R(pos)^T dy, the rotation by
  -pos f_j (``inverse=True``): R is orthogonal.
"""
import numpy as np


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def rope_tables_ref(max_pos, d, base):
    """cos and sin of pos * base ** (-2 j / d) for pos < max_pos, j < d/2,
    in float64, each [max_pos, d/2]."""
    if d % 2:
        raise ValueError("d must be even")
    j = np.arange(d // 2, dtype=np.float64)
    freq = np.power(float(base), -2.0 * j / d)
    ang = np.arange(max_pos, dtype=np.float64)[:, None] * freq[None, :]
    return np.cos(ang), np.sin(ang)


def rope_ref(x, pos, cos, sin, inverse=False):
    """Rotate x [T, H, d] (token t at position pos[t]) with the tables
    cos / sin [max_pos, d/2]. inverse=True applies the transpose (the
    backward). Returns float64 [T, H, d]."""
    x, cos, sin = _f64(x), _f64(cos), _f64(sin)
    pos = np.asarray(pos, dtype=np.int64)
    T, H, d = x.shape
    half = d // 2
    if cos.shape[1] != half or pos.shape != (T,):
        raise ValueError("tables must be [max_pos, d/2] and pos [T]")
    if T and (pos.min() < 0 or pos.max() >= cos.shape[0]):
        raise ValueError("position outside the tables")
    c = cos[pos][:, None, :]
    s = sin[pos][:, None, :]
    if inverse:
        s = -s
    lo, hi = x[..., :half], x[..., half:]
    return np.concatenate([lo * c - hi * s, hi * c + lo * s], axis=-1)


def rope_fp16_ref(x, pos, cos, sin, inverse=False):
    """rope_ref rounded to fp16 (the tensor attention reads)."""
    return rope_ref(x, pos, cos, sin, inverse).astype(np.float16)


def varlen_positions(cu):
    """Position of every packed token within its sequence (0 at its start)."""
    cu = np.asarray(cu, dtype=np.int64)
    return np.concatenate([np.arange(cu[i + 1] - cu[i]) for i in range(len(cu) - 1)]
                          + [np.zeros(0, np.int64)])


def chunk_positions(cu_new, ctx_lens):
    """Context position of each new token of a chunked prefill: the L_b new
    tokens of sequence b are the last L_b of its ctx_lens[b] positions."""
    cu = np.asarray(cu_new, dtype=np.int64)
    out = []
    for b in range(len(cu) - 1):
        L = cu[b + 1] - cu[b]
        out.append(np.arange(int(ctx_lens[b]) - L, int(ctx_lens[b])))
    return np.concatenate(out + [np.zeros(0, np.int64)])
