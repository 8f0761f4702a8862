"""MLA extend (prefill) attention over the paged FP8 latent cache -- oracle
(test infrastructure).

The extend path: "When a Faster Kernel Doesn't Speed Up Serving", *Step 3*
(CastFromFP8): on every extend step the prefill attention reads the
request's whole KV history, and because that kernel takes BF16 only, the
history is cast FP8 -> BF16 first; the direction the page names is an
attention kernel that reads the FP8 cache directly.  "The KV Cache Cast
Bottleneck", *The Message* (its fourth fix): the same direct-FP8 MLA wrapper
serves the paged path of ``forward_extend``.  The attention is the absorbed
MLA form of the decode oracle (``attention``), now with several query tokens
per request:

request b has q_len_b = qo_indptr[b+1] - qo_indptr[b] new query tokens and
kv_len_b = kv_indptr[b+1] - kv_indptr[b] cache tokens, the last q_len_b of
which are the new tokens themselves (the write path stores every step's new
KV before attention, *Step 3*, CastToFP8).  Query token i of request b sees
the first n_i tokens of the request's list:

    causal:      n_i = clamp(kv_len_b - q_len_b + i + 1, 0, kv_len_b)
    not causal:  n_i = kv_len_b

and out[qo_indptr[b] + i, h] is the decode formula over those n_i tokens
(scores over all 576 dims times ``sm_scale``, both operands times ``scale``,
max-subtracted softmax, values = the first 512 dims); n_i = 0 gives a zero
row.  float64 throughout.
"""
import numpy as np

from .attention import KV_WIDTH, V_WIDTH, _request_kv, bf16_bits_to_f64


def visible_tokens(q_len: int, kv_len: int, causal: bool) -> np.ndarray:
    """int64 [q_len]: n_i, the number of leading cache tokens query token i sees."""
    i = np.arange(q_len, dtype=np.int64)
    if not causal:
        return np.full(q_len, kv_len, dtype=np.int64)
    return np.clip(kv_len - q_len + i + 1, 0, kv_len)


def _check(q_bits, pool, qo_indptr, kv_indptr, kv_indices):
    q_bits = np.asarray(q_bits)
    pool = np.asarray(pool)
    qo = np.asarray(qo_indptr).astype(np.int64)
    kv = np.asarray(kv_indptr).astype(np.int64)
    idx = np.asarray(kv_indices).astype(np.int64)
    if q_bits.ndim != 3 or q_bits.shape[2] != KV_WIDTH:
        raise ValueError("q must be [total_q, H, 576] BF16 bits")
    if pool.dtype != np.uint8 or pool.ndim != 2 or pool.shape[1] != KV_WIDTH:
        raise ValueError("pool must be uint8 [num_slots, 576]")
    B = qo.shape[0] - 1
    if B < 1 or kv.shape != (B + 1,):
        raise ValueError("qo_indptr and kv_indptr must both be [B+1]")
    for name, ptr, total in (("qo_indptr", qo, q_bits.shape[0]), ("kv_indptr", kv, idx.shape[0])):
        if ptr[0] != 0 or np.any(np.diff(ptr) < 0) or ptr[-1] > total:
            raise ValueError("%s must start at 0, be non-decreasing and fit its array" % name)
    return q_bits, pool, qo, kv, idx


def mla_extend_ref(q_bits, pool, qo_indptr, kv_indptr, kv_indices, scale, sm_scale,
                   causal=True, rows=None) -> np.ndarray:
    """float64 [total_q, H, 512] (or [len(rows), H, 512] for the query rows
    ``rows``, indices into the total_q axis)."""
    q_bits, pool, qo, kv, idx = _check(q_bits, pool, qo_indptr, kv_indptr, kv_indices)
    total_q, H, _ = q_bits.shape
    want = np.arange(total_q) if rows is None else np.asarray(rows, dtype=np.int64)
    pos = {int(r): k for k, r in enumerate(want)}
    out = np.zeros((len(want), H, V_WIDTH), dtype=np.float64)
    for b in range(qo.shape[0] - 1):
        q0, q1 = int(qo[b]), int(qo[b + 1])
        mine = [r for r in range(q0, q1) if r in pos]
        if not mine:
            continue
        kv_len = int(kv[b + 1] - kv[b])
        n = visible_tokens(q1 - q0, kv_len, causal)
        if kv_len == 0:
            continue
        K = _request_kv(pool, idx, int(kv[b]), int(kv[b + 1]), scale)     # [kv_len, 576]
        for r in mine:
            ni = int(n[r - q0])
            if ni == 0:
                continue
            qd = bf16_bits_to_f64(q_bits[r])                             # [H, 576]
            s = float(sm_scale) * (qd @ K[:ni].T)                         # [H, n_i]
            p = np.exp(s - s.max(axis=1, keepdims=True))
            out[pos[r]] = (p @ K[:ni, :V_WIDTH]) / p.sum(axis=1, keepdims=True)
    return out
