"""Appending new positions to the paged latent cache, with FP8 quantisation.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source pages: "Kimi K3 on AMD Instinct MI355X: vLLM serving ... on AgentX" (AMD blog
post).  Section 1 "Cache": every MLA layer keeps, for each cached position, one
compressed latent of 576 values, stored in FP8 (the payload estimate counts 576 bytes
per position and layer); the history grows by the new tokens of every step.  Section 4
table notes: attention itself runs in BF16, so the model hands the new latents over in
BF16 and the cache stores them quantised.

Readings where the pages are silent: FP8 is OCP E4M3FN with one fp32 scale per layer
pool (value = code * scale); a latent x is stored as the code nearest to the fp32
quotient fp32(x) / scale, ties to the even code, magnitudes past the largest finite
code (448) saturating to it.  The T new tokens of request r are its last T positions
L_r - T .. L_r - 1, L_r = seq_lens[r] counting them (the convention of the decode).
"""

import numpy as np

from .numerics import e4m3fn_codes_to_f64

_E4M3FN_MAX = 448.0
# the 127 non-negative finite codes 0x00 .. 0x7E and their values, ascending
_POS_CODES = np.arange(0x7F, dtype=np.uint8)
_POS_VALUES = e4m3fn_codes_to_f64(_POS_CODES)


def quantize_e4m3fn(x32):
    """fp32 values -> E4M3FN codes (uint8): the nearest code, ties to the even code.

    |x| > 448 saturates to +-448; the sign of zero is kept; NaN gives 0x7F (with the
    sign bit of the input).  Written from the definition: the non-negative finite codes
    are listed with their values in ascending order (the code order is the value
    order), |x| is placed between two neighbours, the nearer one is taken, and on a tie
    the one with an even code (even mantissa) wins.
    """
    x = np.asarray(x32, dtype=np.float32).astype(np.float64)
    neg = np.signbit(x)
    a = np.abs(x)
    nan = np.isnan(a)
    a = np.where(nan, 0.0, np.minimum(a, _E4M3FN_MAX))
    hi = np.searchsorted(_POS_VALUES, a, side="left")   # first value >= a
    hi = np.minimum(hi, len(_POS_VALUES) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _POS_VALUES[lo]
    d_hi = _POS_VALUES[hi] - a
    exact = d_hi == 0
    take_hi = exact | (d_hi < d_lo) | ((d_hi == d_lo) & (_POS_CODES[hi] % 2 == 0))
    code = np.where(take_hi, _POS_CODES[hi], _POS_CODES[lo]).astype(np.uint8)
    code = np.where(nan, np.uint8(0x7F), code)
    return (code | np.where(neg, np.uint8(0x80), np.uint8(0))).astype(np.uint8)


def bf16_bits_to_f32(bits):
    """bfloat16 bit patterns -> fp32 values (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def stored_row(latent_bits, kv_format, kv_scale):
    """One new latent row (bf16 bit patterns, 576 values) as the cache stores it."""
    if kv_format == "bf16":
        assert float(kv_scale) == 1.0
        return np.asarray(latent_bits, dtype=np.uint16).copy()
    if kv_format == "fp8_e4m3fn":
        x = bf16_bits_to_f32(latent_bits)
        q = x / np.float32(kv_scale)   # fp32 division, rounded to nearest even
        return quantize_e4m3fn(q.astype(np.float32))
    raise ValueError(f"unknown kv_format {kv_format!r}")


def kv_append(pool, block_table, seq_lens, latent_bits, q_len, kv_format, kv_scale, page_size):
    """A copy of ``pool`` with the q_len new latents of every request written in.

    pool: [num_pages][page_size][576] (uint16 bf16 patterns or uint8 codes);
    block_table: int [B][max_pages]; seq_lens: [B], counting the new tokens;
    latent_bits: uint16 bf16 patterns [B][q_len][576].  Token t of request r goes to
    position L_r - q_len + t, i.e. page block_table[r][j // page_size], slot
    j % page_size.  Nothing else changes.
    """
    out = np.array(pool, copy=True)
    B = len(seq_lens)
    for r in range(B):
        L = int(seq_lens[r])
        for t in range(q_len):
            j = L - q_len + t
            assert j >= 0
            page = int(block_table[r][j // page_size])
            out[page, j % page_size, :] = stored_row(latent_bits[r, t], kv_format, kv_scale)
    return out
