"""Pins for the CPU oracle: values and laws fixed by the format definition,
the pages and mathematics -- never by the oracle itself or by the HIP path."""
import itertools
import math
import os
import struct

import numpy as np
import pytest
import torch

import oracle
from oracle.attention import KV_WIDTH, V_WIDTH

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- E4M3 table

def _golden_pairs(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                a, b = line.split()
                rows.append((a, b))
    return rows


def test_e4m3_ocp_special_values():
    table = oracle.decode_table()
    for code_s, val_s in _golden_pairs("e4m3_ocp_special_values.txt"):
        code = int(code_s, 16)
        if val_s == "nan":
            assert math.isnan(table[code]), hex(code)
        else:
            want = float(val_s)
            assert table[code] == want, (hex(code), table[code], want)
            assert math.copysign(1.0, table[code]) == math.copysign(1.0, want)


def test_e4m3_matches_torch_decode_all_codes():
    # torch's float8_e4m3fn decode is an independent library implementation.
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    table = oracle.decode_table()
    nan_ref = np.isnan(ref)
    assert np.array_equal(nan_ref, np.isnan(table))
    assert np.array_equal(ref[~nan_ref], table[~nan_ref])
    assert np.array_equal(np.signbit(ref[~nan_ref]), np.signbit(table[~nan_ref]))


def test_e4m3_structure():
    t = oracle.decode_table()
    pos = t[:127]
    assert np.all(np.diff(pos) > 0)                      # strictly increasing magnitudes
    assert np.array_equal(t[128:255], -pos)              # sign symmetry
    assert np.isnan(t).sum() == 2 and np.isfinite(t).sum() == 254
    assert np.nanmax(np.abs(t)) == 448.0
    # spacing inside each binade is 2^(e-10); subnormal spacing 2^-9
    for e in range(1, 16):
        codes = [(e << 3) | m for m in range(8) if not (e == 15 and m == 7)]
        assert np.all(np.diff(t[codes]) == 2.0 ** (e - 10))
    assert np.all(np.diff(t[0:9]) == 2.0 ** -9)


def test_e4m3_to_bf16_exact_and_matches_torch():
    table = oracle.decode_table()
    bits = oracle.cast_table_bf16()
    # exactness: decoding the BF16 bits gives back the E4M3 value
    back = oracle.bf16_bits_to_f64(bits)
    fin = np.isfinite(table)
    assert np.array_equal(back[fin], table[fin])
    assert np.array_equal(np.signbit(back[fin]), np.signbit(table[fin]))
    # the pages' cast is torch's .to(); compare all 256 codes bit for bit
    ref = (torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn)
           .to(torch.bfloat16).view(torch.int16).numpy().astype(np.uint16))
    assert np.array_equal(bits, ref)
    assert bits[0x7F] == 0x7FC0 and bits[0xFF] == 0x7FC0 and bits[0x80] == 0x8000


def test_bf16_bits_of_rejects_inexact():
    with pytest.raises(ValueError):
        oracle.bf16_bits_of(1.0 + 2.0 ** -9)
    assert oracle.bf16_bits_of(1.0) == 0x3F80
    assert oracle.bf16_bits_of(-2.0) == 0xC000


# ---------------------------------------------------------------- cast / gather

def test_cast_and_gather_against_torch_rows():
    rng = np.random.default_rng(5)
    pool = rng.integers(0, 256, size=(37, KV_WIDTH), dtype=np.uint8)
    torch_cast = (torch.from_numpy(pool).view(torch.float8_e4m3fn).to(torch.bfloat16)
                  .view(torch.int16).numpy().astype(np.uint16))
    assert np.array_equal(oracle.cast_ref(pool), torch_cast)
    idx = rng.integers(0, 37, size=11)
    assert np.array_equal(oracle.gather_ref(pool, idx), torch_cast[idx])
    assert oracle.gather_ref(pool, np.zeros(0, dtype=np.int64)).shape == (0, KV_WIDTH)
    with pytest.raises(IndexError):
        oracle.gather_ref(pool, np.array([37]))


def test_cast_accounting_matches_pages():
    vals = dict(_golden_pairs("pages_cast_accounting.txt"))
    slots, width, layers = int(vals["pool_slots"]), int(vals["kv_width"]), int(vals["layers"])
    small = np.zeros((4, width), dtype=np.uint8)
    out = oracle.cast_ref(small)
    bytes_per_elem = small.itemsize + out.itemsize           # read FP8 + write BF16
    per_layer = slots * width * bytes_per_elem
    assert per_layer == 856_313_856
    assert round(per_layer * layers / 1e9, 1) == float(vals["printed_GB_per_step"])


# ---------------------------------------------------------------- attention: brute force

_TORCH_VALUES = (torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn)
                 .to(torch.float64).tolist())


def _bf16_to_float(bits):
    return struct.unpack("<f", struct.pack("<I", (int(bits) & 0xFFFF) << 16))[0]


def brute_force(q_bits, pool, indptr, indices, scale, sm_scale):
    """Pure-Python triple loop: torch's FP8 decode, math.fsum, softmax WITHOUT
    max subtraction.  Independent of the oracle's code and table."""
    B, H, _ = q_bits.shape
    out = [[[0.0] * V_WIDTH for _ in range(H)] for _ in range(B)]
    for b in range(B):
        rows = []
        for t in range(int(indptr[b]), int(indptr[b + 1])):
            slot = int(indices[t])
            rows.append([_TORCH_VALUES[int(c)] * scale for c in pool[slot]])
        if not rows:
            continue
        for h in range(H):
            qv = [_bf16_to_float(x) for x in q_bits[b, h]]
            e = [math.exp(sm_scale * math.fsum(qv[d] * r[d] for d in range(KV_WIDTH)))
                 for r in rows]
            den = math.fsum(e)
            for c in range(V_WIDTH):
                out[b][h][c] = math.fsum(e[t] * rows[t][c] for t in range(len(rows))) / den
    return np.array(out)


def _tiny_case(seed, B, H, lens, num_slots=23, q_sigma=1.0, scale=1.0):
    rng = np.random.default_rng(seed)
    pool_f = rng.standard_normal((num_slots, KV_WIDTH)).astype(np.float32)
    pool = torch.from_numpy(pool_f).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    q = (torch.from_numpy(rng.standard_normal((B, H, KV_WIDTH)) * q_sigma).to(torch.bfloat16)
         .view(torch.int16).numpy().astype(np.uint16))
    indptr = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    indices = rng.integers(0, num_slots, size=int(indptr[-1]))
    return q, pool, indptr, indices, scale, 1.0 / math.sqrt(192.0)


def _rel_err(a, b):
    return np.max(np.abs(a - b)) / max(1e-300, np.max(np.abs(b)))


@pytest.mark.parametrize("seed,B,H,lens,scale", [
    (0, 1, 1, [1], 1.0),
    (1, 1, 2, [2], 0.75),
    (2, 2, 2, [5, 3], 1.5),
    (3, 2, 1, [4, 0], 2.0),
])
def test_oracle_matches_brute_force(seed, B, H, lens, scale):
    case = _tiny_case(seed, B, H, lens, scale=scale)
    ref = oracle.mla_decode_ref(*case)
    bf = brute_force(*case)
    assert _rel_err(ref, bf) <= 1e-12


def test_max_subtraction_needed_for_large_scores():
    q, pool, indptr, indices, _, sm = _tiny_case(9, 1, 1, [4], q_sigma=16.0)
    scale = 64.0
    with pytest.raises(OverflowError):
        brute_force(q, pool, indptr, indices, scale, sm)
    ref = oracle.mla_decode_ref(q, pool, indptr, indices, scale, sm)
    assert np.all(np.isfinite(ref))
    # the softmax is then (nearly) one-hot: the output is one of the rows
    vals = np.array(_TORCH_VALUES)[pool[indices]] * scale
    best = np.min(np.max(np.abs(vals[:, :V_WIDTH] - ref[0, 0]), axis=1))
    assert best <= 1e-6 * np.max(np.abs(vals))


# ---------------------------------------------------------------- attention: closed forms

def _decoded_rows(pool, slots, scale):
    return np.array([[_TORCH_VALUES[int(c)] for c in pool[s]] for s in slots]) * scale


def test_zero_query_gives_mean_of_values():
    q, pool, indptr, indices, scale, sm = _tiny_case(11, 1, 3, [7], scale=1.25)
    q[:] = 0
    ref = oracle.mla_decode_ref(q, pool, indptr, indices, scale, sm)
    rows = _decoded_rows(pool, indices, scale)
    mean = np.array([math.fsum(rows[:, c]) / 7 for c in range(V_WIDTH)])
    for h in range(3):
        assert np.max(np.abs(ref[0, h] - mean)) <= 1e-12 * np.max(np.abs(mean))


def test_single_token_returns_its_value_row():
    q, pool, indptr, indices, scale, sm = _tiny_case(12, 2, 4, [1, 1], scale=0.5)
    ref = oracle.mla_decode_ref(q, pool, indptr, indices, scale, sm)
    rows = _decoded_rows(pool, indices, scale)
    for b in range(2):
        for h in range(4):
            assert np.array_equal(ref[b, h], rows[b, :V_WIDTH])


def test_two_tokens_sigmoid_form():
    q, pool, indptr, indices, scale, sm = _tiny_case(13, 1, 2, [2], scale=1.0)
    ref = oracle.mla_decode_ref(q, pool, indptr, indices, scale, sm)
    rows = _decoded_rows(pool, indices, scale)
    for h in range(2):
        qv = [_bf16_to_float(x) for x in q[0, h]]
        s1 = sm * math.fsum(qv[d] * rows[0][d] for d in range(KV_WIDTH))
        s2 = sm * math.fsum(qv[d] * rows[1][d] for d in range(KV_WIDTH))
        w1 = 1.0 / (1.0 + math.exp(s2 - s1))
        w2 = 1.0 / (1.0 + math.exp(s1 - s2))
        want = w1 * rows[0, :V_WIDTH] + w2 * rows[1, :V_WIDTH]
        assert np.max(np.abs(ref[0, h] - want)) <= 1e-12 * np.max(np.abs(want))


def test_empty_request_is_zero():
    q, pool, indptr, indices, scale, sm = _tiny_case(14, 3, 2, [3, 0, 2])
    ref = oracle.mla_decode_ref(q, pool, indptr, indices, scale, sm)
    assert np.all(ref[1] == 0.0) and np.any(ref[0] != 0.0)


# ---------------------------------------------------------------- attention: invariants

def test_invariant_token_permutation():
    q, pool, indptr, indices, scale, sm = _tiny_case(15, 2, 4, [9, 6], num_slots=40)
    ref = oracle.mla_decode_ref(q, pool, indptr, indices, scale, sm)
    rng = np.random.default_rng(0)
    perm_idx = indices.copy()
    perm_idx[0:9] = indices[0:9][rng.permutation(9)]
    perm_idx[9:15] = indices[9:15][rng.permutation(6)]
    got = oracle.mla_decode_ref(q, pool, indptr, perm_idx, scale, sm)
    assert _rel_err(got, ref) <= 1e-12


def test_invariant_slot_relocation():
    q, pool, indptr, indices, scale, sm = _tiny_case(16, 2, 2, [5, 4], num_slots=20)
    ref = oracle.mla_decode_ref(q, pool, indptr, indices, scale, sm)
    rng = np.random.default_rng(1)
    perm = rng.permutation(20)             # slot s moves to perm[s]
    moved = np.empty_like(pool)
    moved[perm] = pool
    got = oracle.mla_decode_ref(q, moved, indptr, perm[indices], scale, sm)
    assert _rel_err(got, ref) <= 1e-12


def test_invariant_head_independence():
    q, pool, indptr, indices, scale, sm = _tiny_case(17, 1, 5, [8])
    ref = oracle.mla_decode_ref(q, pool, indptr, indices, scale, sm)
    q2 = q.copy()
    q2[0, 2] = q[0, 4][::-1]
    got = oracle.mla_decode_ref(q2, pool, indptr, indices, scale, sm)
    keep = [0, 1, 3, 4]
    assert np.array_equal(got[0, keep], ref[0, keep])
    assert not np.array_equal(got[0, 2], ref[0, 2])


def test_invariant_query_and_softmax_scale_trade():
    q, pool, indptr, indices, scale, sm = _tiny_case(18, 2, 3, [6, 7])
    ref = oracle.mla_decode_ref(q, pool, indptr, indices, scale, sm)
    # doubling a BF16 value adds one to its exponent field (exact)
    q2 = (q.astype(np.uint32) + (1 << 7)).astype(np.uint16)
    assert np.array_equal(oracle.bf16_bits_to_f64(q2), 2.0 * oracle.bf16_bits_to_f64(q))
    got = oracle.mla_decode_ref(q2, pool, indptr, indices, scale, sm / 2.0)
    assert _rel_err(got, ref) <= 1e-12


@pytest.mark.parametrize("cuts", [[3], [1, 5], [2, 4, 7], [0, 8]])
def test_split_combine_identity(cuts):
    q, pool, indptr, indices, scale, sm = _tiny_case(19, 1, 4, [9], scale=1.5)
    ref = oracle.mla_decode_ref(q, pool, indptr, indices, scale, sm)[0]
    bounds = [0] + list(cuts) + [9]
    parts = [oracle.mla_decode_partial_ref(q, pool, indptr, indices, scale, sm, 0, lo, hi)
             for lo, hi in zip(bounds[:-1], bounds[1:])]
    got = oracle.combine_partials_ref(parts)
    assert np.max(np.abs(got - ref)) <= 1e-12 * np.max(np.abs(ref))


# ---------------------------------------------------------------- planted mistakes

def _mutant_outputs(case, kind):
    q, pool, indptr, indices, scale, sm = case
    table = oracle.decode_table()
    if kind == "fnuz_bias":            # exponent bias 8 instead of 7
        table = table / 2.0
    B, H, _ = q.shape
    out = np.zeros((B, H, V_WIDTH))
    for b in range(B):
        slots = indices[indptr[b]:indptr[b + 1]]
        if len(slots) == 0:
            continue
        K = table[pool[slots]] * scale
        qd = oracle.bf16_bits_to_f64(q[b])
        if kind == "scores_latent_only":
            s = sm * qd[:, :V_WIDTH] @ K[:, :V_WIDTH].T
        elif kind == "sign_flip":
            s = -sm * qd @ K.T
        else:
            s = sm * qd @ K.T
        p = np.exp(s - s.max(axis=1, keepdims=True))
        V = K[:, KV_WIDTH - V_WIDTH:] if kind == "values_from_tail" else K[:, :V_WIDTH]
        if kind == "unscaled_values":
            V = V / scale
        o = p @ V
        if kind != "no_normalise":
            o = o / p.sum(axis=1, keepdims=True)
        if kind == "heads_transposed":
            o = o[::-1]
        out[b] = o
    return out


@pytest.mark.parametrize("kind", ["fnuz_bias", "scores_latent_only", "sign_flip",
                                  "values_from_tail", "unscaled_values", "no_normalise",
                                  "heads_transposed"])
def test_planted_mistakes_are_caught_by_brute_force(kind):
    case = _tiny_case(21, 2, 3, [4, 3], scale=1.5)
    bf = brute_force(*case)
    assert _rel_err(oracle.mla_decode_ref(*case), bf) <= 1e-12
    assert _rel_err(_mutant_outputs(case, kind), bf) > 1e-6
