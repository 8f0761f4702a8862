"""Pins for the extend (prefill) attention oracle: reductions to the pinned
decode oracle, a pure-Python brute force with the causal rule stated on token
positions, mask invariance and planted mistakes.  Nothing here comes from the
HIP path."""
import math

import numpy as np
import pytest
import torch

import oracle
import oracle.extend as ext
from oracle.attention import KV_WIDTH, V_WIDTH
from tests.test_oracle_pins import _TORCH_VALUES, _bf16_to_float


def _case(seed, q_lens, kv_lens, H=2, num_slots=40, scale=1.25, q_sigma=1.0):
    rng = np.random.default_rng(seed)
    pool_f = rng.standard_normal((num_slots, KV_WIDTH)).astype(np.float32)
    pool = torch.from_numpy(pool_f).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    total_q = int(sum(q_lens))
    q = (torch.from_numpy(rng.standard_normal((total_q, H, KV_WIDTH)) * q_sigma).to(torch.bfloat16)
         .view(torch.int16).numpy().astype(np.uint16))
    qo = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int64)
    kv = np.concatenate([[0], np.cumsum(kv_lens)]).astype(np.int64)
    idx = rng.integers(0, num_slots, size=int(kv[-1]))
    return q, pool, qo, kv, idx, scale, 1.0 / math.sqrt(192.0)


def brute_force_extend(q, pool, qo, kv, idx, scale, sm, causal):
    """Pure-Python loops, torch's FP8 decode, math.fsum, softmax without max
    subtraction.  The mask is stated on positions: the new tokens are the last
    q_len entries of the request's cache list, so query token i is entry
    kv_len - q_len + i and sees the entries at or before it (every entry when
    not causal)."""
    total_q, H, _ = q.shape
    out = np.zeros((total_q, H, V_WIDTH))
    for b in range(len(qo) - 1):
        q_len, kv_len = int(qo[b + 1] - qo[b]), int(kv[b + 1] - kv[b])
        rows = [[_TORCH_VALUES[int(c)] * scale for c in pool[int(idx[kv[b] + j])]]
                for j in range(kv_len)]
        for i in range(q_len):
            own = kv_len - q_len + i
            seen = [j for j in range(kv_len) if (not causal) or j <= own]
            if not seen:
                continue
            for h in range(H):
                qv = [_bf16_to_float(x) for x in q[qo[b] + i, h]]
                e = [math.exp(sm * math.fsum(qv[d] * rows[j][d] for d in range(KV_WIDTH)))
                     for j in seen]
                den = math.fsum(e)
                for c in range(V_WIDTH):
                    out[qo[b] + i, h, c] = math.fsum(e[t] * rows[j][c] for t, j in enumerate(seen)) / den
    return out


def _rel(a, b):
    return np.max(np.abs(a - b)) / max(1e-300, np.max(np.abs(b)))


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("seed,q_lens,kv_lens", [
    (0, [1], [3]),
    (1, [3], [5]),
    (2, [2, 3], [4, 3]),          # second request: prefill from scratch (kv_len == q_len)
    (3, [3, 1], [2, 4]),          # kv_len < q_len: the first token sees nothing
])
def test_matches_brute_force(seed, q_lens, kv_lens, causal):
    case = _case(seed, q_lens, kv_lens)
    ref = oracle.mla_extend_ref(*case, causal=causal)
    bf = brute_force_extend(*case, causal)
    assert _rel(ref, bf) <= 1e-12
    if seed == 3 and causal:
        assert np.all(ref[0] == 0)                # n_0 = 0: zero row


def test_one_token_per_request_is_decode():
    case = _case(4, [1, 1, 1], [5, 1, 7], H=3)
    q, pool, qo, kv, idx, scale, sm = case
    for causal in (True, False):
        got = oracle.mla_extend_ref(*case, causal=causal)
        dec = oracle.mla_decode_ref(q, pool, kv, idx, scale, sm)
        assert _rel(got, dec) <= 1e-13


def test_last_token_sees_everything_and_non_causal_is_decode_per_token():
    q_lens, kv_lens = [4, 3], [9, 3]
    case = _case(5, q_lens, kv_lens, H=2)
    q, pool, qo, kv, idx, scale, sm = case
    causal = oracle.mla_extend_ref(*case, causal=True)
    full = oracle.mla_extend_ref(*case, causal=False)
    for b in range(2):
        # every token of the request against the whole list, as decode requests
        rows = range(qo[b], qo[b + 1])
        dec = oracle.mla_decode_ref(q[list(rows)], pool,
                                    np.arange(len(rows) + 1) * kv_lens[b],
                                    np.tile(idx[kv[b]:kv[b + 1]], len(rows)), scale, sm)
        assert _rel(full[list(rows)], dec) <= 1e-13
        last = qo[b + 1] - 1
        assert _rel(causal[last], full[last]) <= 1e-13
    # the first token of request 0 sees kv_len - q_len + 1 = 6 tokens
    first = oracle.mla_decode_ref(q[[0]], pool, np.array([0, 6]), idx[0:6], scale, sm)
    assert _rel(causal[0], first[0]) <= 1e-13


def test_mask_invariance():
    """Rewriting cache rows a token must not see leaves its output unchanged."""
    case = _case(6, [5], [12], H=2)
    q, pool, qo, kv, idx, scale, sm = case
    ref = oracle.mla_extend_ref(*case)
    n = oracle.visible_tokens(5, 12, True)
    for i in range(5):
        pool2 = pool.copy()
        hidden = idx[n[i]:]
        keep = set(idx[:n[i]].tolist())
        for s in hidden:
            if s not in keep:
                pool2[s] = ((pool2[s].astype(np.int64) + 17) % 256 & 0x77).astype(np.uint8)  # finite codes
        got = oracle.mla_extend_ref(q, pool2, qo, kv, idx, scale, sm)
        assert np.array_equal(got[i], ref[i])
        if i < 4:   # the rewrite is visible to a token that sees the whole list
            assert not np.array_equal(
                oracle.mla_extend_ref(q, pool2, qo, kv, idx, scale, sm, causal=False)[i],
                oracle.mla_extend_ref(*case, causal=False)[i])


_MUTANTS = {
    "off_by_one": lambda q_len, kv_len, causal: np.clip(
        kv_len - q_len + np.arange(q_len), 0, kv_len) if causal else np.full(q_len, kv_len),
    "top_left": lambda q_len, kv_len, causal: np.clip(
        np.arange(q_len) + 1, 0, kv_len) if causal else np.full(q_len, kv_len),
    "no_mask": lambda q_len, kv_len, causal: np.full(q_len, kv_len),
    "reversed": lambda q_len, kv_len, causal: np.clip(
        kv_len - np.arange(q_len), 0, kv_len) if causal else np.full(q_len, kv_len),
}


@pytest.mark.parametrize("kind", sorted(_MUTANTS))
def test_planted_mask_mistakes_are_caught(kind, monkeypatch):
    case = _case(7, [3, 2], [6, 4], H=2)
    bf = brute_force_extend(*case, True)
    assert _rel(oracle.mla_extend_ref(*case), bf) <= 1e-12
    monkeypatch.setattr(ext, "visible_tokens", _MUTANTS[kind])
    assert _rel(oracle.mla_extend_ref(*case), bf) > 1e-6


def test_rows_subset_and_validation():
    case = _case(8, [3, 2], [5, 4], H=2)
    full = oracle.mla_extend_ref(*case)
    sub = oracle.mla_extend_ref(*case, rows=[4, 0])
    assert np.array_equal(sub, full[[4, 0]])
    q, pool, qo, kv, idx, scale, sm = case
    with pytest.raises(ValueError):
        oracle.mla_extend_ref(q, pool, qo[:-1], kv, idx, scale, sm)
    with pytest.raises(ValueError):
        oracle.mla_extend_ref(q, pool, qo, kv + 1, idx, scale, sm)
