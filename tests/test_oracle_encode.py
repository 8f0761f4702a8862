"""Pins for the oracle's BF16 -> E4M3FN write path (``oracle.encode``): the
OCP format's rounding boundaries, torch's own float -> Float8_e4m3fn copy (the
``aten::copy_`` of the pages' CastToFP8 step), round trips, brute-force nearest
search and planted mistakes.  Nothing here comes from the HIP path."""
import os
import types

import numpy as np
import pytest
import torch

import oracle
import oracle.encode as enc_mod

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
F8 = torch.float8_e4m3fn


def _bf16_bits(text):
    if text == "nan":
        return 0x7FC0
    if text == "-nan":
        return 0xFFC0
    f = np.float32(float(text))
    bits = int(f.view(np.uint32))
    assert bits & 0xFFFF == 0, f"{text} is not a BF16 value"
    return bits >> 16


def _golden_cases(name="e4m3_encode_rounding.txt"):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                v, c = line.split()
                rows.append((v, _bf16_bits(v), int(c, 16)))
    return rows


def _golden_mismatches(encode, name="e4m3_encode_rounding.txt", **kw):
    bad = []
    for text, bits, code in _golden_cases(name):
        got = int(encode(oracle.encode.bf16_bits_to_f32(np.uint16(bits)), **kw))
        if got != code:
            bad.append((text, hex(code), hex(got)))
    return bad


def test_golden_rounding_boundaries():
    assert len(_golden_cases()) >= 25
    assert _golden_mismatches(oracle.encode_e4m3fn) == []


def test_golden_saturating_mode():
    assert len(_golden_cases("e4m3_encode_saturate.txt")) >= 12
    assert _golden_mismatches(oracle.encode_e4m3fn, "e4m3_encode_saturate.txt", saturate=True) == []


def _torch_codes_of_bf16(bits_u16):
    t = torch.from_numpy(bits_u16.astype(np.int32)).to(torch.int16).view(torch.bfloat16)
    return t.to(F8).view(torch.uint8).numpy()


def test_all_bf16_patterns_match_torch_copy():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ours = oracle.encode_e4m3fn(oracle.encode.bf16_bits_to_f32(bits))
    ref = _torch_codes_of_bf16(bits)
    assert np.array_equal(ours, ref), np.nonzero(ours != ref)[0][:10]


def test_all_bf16_patterns_saturating_match_torch_clamp_then_copy():
    """Saturating mode = clamp to [-448, 448] (NaN passes through), then copy."""
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ours = oracle.encode_e4m3fn(oracle.encode.bf16_bits_to_f32(bits), saturate=True)
    t = torch.from_numpy(bits.astype(np.int32)).to(torch.int16).view(torch.bfloat16).float()
    ref = t.clamp(-448.0, 448.0).to(F8).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref), np.nonzero(ours != ref)[0][:10]


@pytest.mark.parametrize("inv_scale", [1.0, 0.5, 1.0 / 3.0, 7.25, 1e-3, 300.0])
def test_scaled_float32_values_match_torch(inv_scale):
    rng = np.random.default_rng(11)
    bits = rng.integers(0, 1 << 16, size=200_000).astype(np.uint16)
    x = oracle.encode.bf16_bits_to_f32(bits)
    with np.errstate(invalid="ignore", over="ignore"):
        y = (x * np.float32(inv_scale)).astype(np.float32)
    ours = oracle.encode_e4m3fn(y)
    ref = torch.from_numpy(y).to(F8).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_round_trip_every_finite_code():
    table = oracle.decode_table()
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    assert np.array_equal(oracle.encode_e4m3fn(table[codes]), codes)


def test_nearest_code_by_brute_force():
    """Each finite input within range goes to a code at minimum distance; of
    two at equal distance, to the one with an even last bit."""
    table = oracle.decode_table()
    finite = np.array([c for c in range(128) if c != 0x7F])
    rng = np.random.default_rng(5)
    mags = np.concatenate([
        rng.uniform(0, 464, 4000),
        np.exp2(rng.uniform(-12, 8.85, 4000)),
        (table[0:126] + table[1:127]) / 2,     # every midpoint between finite codes
        [464.0],
    ]).astype(np.float32)
    mags = mags[mags <= 464]
    codes = oracle.encode_e4m3fn(mags)
    d = np.abs(table[finite][None, :] - mags[:, None].astype(np.float64))
    best = d.min(axis=1)
    got = np.abs(table[codes] - mags)
    assert np.array_equal(got, best)
    ties = (d == best[:, None]).sum(axis=1) == 2
    assert ties.sum() > 100
    assert np.all(codes[ties] % 2 == 0)


def test_monotone_and_odd_symmetric():
    rng = np.random.default_rng(9)
    x = np.sort(rng.normal(0, 60, 50_000).astype(np.float32))
    x = x[np.abs(x) <= 464]
    v = oracle.decode_table()[oracle.encode_e4m3fn(x)]
    assert np.all(np.diff(v) >= 0)
    assert np.array_equal(oracle.encode_e4m3fn(-x), oracle.encode_e4m3fn(x) ^ 0x80)


def test_scatter_writes_only_named_slots():
    rng = np.random.default_rng(3)
    pool = rng.integers(0, 256, size=(40, 576), dtype=np.uint8)
    src = rng.integers(0, 1 << 16, size=(6, 576)).astype(np.uint16)
    slots = np.array([7, 0, 39, -1, 40, 12])      # -1 and 40 are outside the pool
    out = oracle.scatter_ref(pool, src, slots, 0.5)
    sat = oracle.scatter_ref(pool, src, slots, 0.5, saturate=True)
    with np.errstate(invalid="ignore"):
        big = np.abs(oracle.encode.bf16_bits_to_f32(src[[0, 1, 2, 5]])) * np.float32(0.5) > 464
    assert big.sum() > 100
    assert np.all(sat[[7, 0, 39, 12]][big] & 0x7F == 0x7E)
    assert np.array_equal(sat[[7, 0, 39, 12]][~big], out[[7, 0, 39, 12]][~big])
    with np.errstate(invalid="ignore"):
        y = (oracle.encode.bf16_bits_to_f32(src) * np.float32(0.5)).astype(np.float32)
    for r, s in enumerate(slots):
        if 0 <= s < 40:
            assert np.array_equal(out[s], torch.from_numpy(y[r]).to(F8).view(torch.uint8).numpy())
    untouched = [s for s in range(40) if s not in (7, 0, 39, 12)]
    assert np.array_equal(out[untouched], pool[untouched])
    assert not np.shares_memory(out, pool)


# ---------------------------------------------------------------- planted mistakes

_SRC = open(enc_mod.__file__).read()

_MUTANTS = {
    "ties_away_from_zero": [("((d_hi == d_lo) & (lo % 2 == 1))", "(d_hi == d_lo)")],
    "ties_to_odd": [("(lo % 2 == 1)", "(lo % 2 == 0)")],
    "truncate": [("take_hi = (d_hi < d_lo)", "take_hi = (d_hi < -1.0)")],
    "saturate_overflow": [("v[0x7F] = 480.0", "v[0x7F] = 1e30"),
                          ("np.where(m > 480.0, np.uint8(0x7F), code)", "np.where(m > 448.0, np.uint8(0x7E), code)")],
    "inf_saturates": [("np.where(m > 480.0, np.uint8(0x7F), code)",
                       "np.where(np.isinf(m), np.uint8(0x7E), np.where(m > 480.0, np.uint8(0x7F), code))")],
    "sign_dropped": [("return (code | sign)", "return (code)")],
    "neighbour_off_by_one": [("lo = hi - 1", "lo = np.maximum(hi - 2, 0)")],
    "flush_subnormals": [("m = np.where(nan, 0.0, np.abs(y))", "m = np.where(nan | (np.abs(y) < 2.0**-6), 0.0, np.abs(y))")],
    "saturate_ignored": [("        m = np.minimum(m, 448.0)", "        pass")],
    "saturate_clamps_nan": [("code = np.where(nan, np.uint8(0x7F), code)", "code = np.where(nan, np.uint8(0x7F if not saturate else 0x7E), code)")],
}

_SATURATE_MUTANTS = {"saturate_ignored", "saturate_clamps_nan"}


def _mutant_encoder(name):
    src = _SRC
    for old, new in _MUTANTS[name]:
        assert src.count(old) == 1, (name, old)
        src = src.replace(old, new)
    mod = types.ModuleType(f"encode_mutant_{name}")
    mod.__dict__["decode_table"] = oracle.decode_table
    code = compile(src.replace("from .e4m3 import decode_table\n", ""), f"<{name}>", "exec")
    exec(code, mod.__dict__)
    return mod.encode_e4m3fn


@pytest.mark.parametrize("name", sorted(_MUTANTS))
def test_planted_mistakes_fail_the_golden_pins(name):
    if name in _SATURATE_MUTANTS:
        bad = _golden_mismatches(_mutant_encoder(name), "e4m3_encode_saturate.txt", saturate=True)
    else:
        bad = _golden_mismatches(_mutant_encoder(name))
    assert bad != []
