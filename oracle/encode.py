"""BF16 -> E4M3FN write path (CastToFP8) -- oracle (test infrastructure).

"When a Faster Kernel Doesn't Speed Up Serving", *Step 3* (the CastToFP8
section): every decode or extend step produces new KV rows in BF16 and
``set_kv_buffer`` stores them into the FP8 KV cache through an
``aten::copy_`` from the BF16 tensor into the FP8 one, i.e. torch's
float -> ``Float8_e4m3fn`` conversion.  The pages name that conversion only;
its rule, read off the format (OCP E4M3FN, see ``e4m3``) and checked against
torch's own conversion in the tests, is:

* round to the nearest E4M3FN value, ties to the code with an even last
  mantissa bit;
* magnitudes past the largest finite value are measured against the next
  code up, 480 (the NaN pattern 0x7F): up to 464 (the midpoint, a tie that
  goes to the even code of 448) they give 448, beyond it NaN;
* NaN and infinities give NaN; the sign bit is kept in every case (so
  -0 -> 0x80 and negative overflow -> 0xFF).

``saturate=True`` is the other common writer convention for an FP8 KV cache:
magnitudes are first clamped to 448, so overflow and infinities give +-448
(0x7E / 0xFE) instead of NaN, while NaN stays NaN; below 448 the two modes
agree.  The pages' ``copy_`` is the default, ``saturate=False``.

``scatter_ref`` applies it row by row: pool row ``slots[r]`` receives the
encoded BF16 row ``r`` times ``inv_scale``; the product is taken in float32
(round to nearest even), as the kernel does, so that both sides decide each
code from the same float32 value.  ``inv_scale = 1`` is the pages' unscaled
copy.  Slots outside ``[0, num_slots)`` are skipped; the pool is otherwise
unchanged.
"""
import numpy as np

from .e4m3 import decode_table

_POS = None


def _positive_values() -> np.ndarray:
    """float64[128]: value of codes 0x00..0x7F with 0x7F read as 480 (the
    rounding bound above 448), ascending."""
    global _POS
    if _POS is None:
        v = decode_table()[:128].copy()
        v[0x7F] = 480.0
        assert np.all(np.diff(v) > 0)
        _POS = v
    return _POS


def encode_e4m3fn(y, saturate: bool = False) -> np.ndarray:
    """uint8 E4M3FN codes of float values (any shape), by the rule above."""
    with np.errstate(invalid="ignore"):    # signalling NaN inputs are expected
        y = np.asarray(y, dtype=np.float64)
    table = _positive_values()
    sign = np.signbit(y).astype(np.uint8) << 7
    nan = np.isnan(y)
    m = np.where(nan, 0.0, np.abs(y))
    if saturate:
        m = np.minimum(m, 448.0)                       # also clamps +-inf
    # neighbours table[lo] <= m < table[lo + 1], for m below 480
    with np.errstate(invalid="ignore"):
        hi = np.clip(np.searchsorted(table, m, side="right"), 1, 127)
        lo = hi - 1
        d_lo = m - table[lo]
        d_hi = table[hi] - m
        take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (lo % 2 == 1))
    code = np.where(take_hi, hi, lo).astype(np.uint8)
    code = np.where(m > 480.0, np.uint8(0x7F), code)  # beyond the table, inf: NaN
    code = np.where(nan, np.uint8(0x7F), code)
    return (code | sign).astype(np.uint8)


def bf16_bits_to_f32(bits) -> np.ndarray:
    """float32 values of BF16 bit patterns (exact: BF16 is a float32 prefix)."""
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32)


def scatter_ref(pool: np.ndarray, src_bits: np.ndarray, slots: np.ndarray,
                inv_scale: float, saturate: bool = False) -> np.ndarray:
    """Copy of ``pool`` (uint8 [num_slots, W]) with row ``slots[r]`` replaced
    by the E4M3FN encoding of float32(src[r, :]) * float32(inv_scale)."""
    pool = np.array(pool, dtype=np.uint8, copy=True)
    src = bf16_bits_to_f32(src_bits)
    with np.errstate(invalid="ignore", over="ignore"):   # NaN / overflow inputs are expected
        y = (src * np.float32(inv_scale)).astype(np.float32)
    codes = encode_e4m3fn(y, saturate)
    for r, s in enumerate(np.asarray(slots, dtype=np.int64)):
        if 0 <= s < pool.shape[0]:
            pool[s] = codes[r]
    return pool
