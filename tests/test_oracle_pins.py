"""Pins of the fp64 oracle to things other than itself (CPU only).

* exact decimal brute force (50 significant digits) on tiny inputs;
* closed forms (one and two positions, zero query, tied keys, a spike key);
* independent library routines (scipy's logsumexp / softmax, torch's E4M3FN);
* invariants the pages fix (Kimi K3 on MI355X, section 4 "MLA": heads are
  independent, so padding heads changes no real head, and splitting the history
  into partitions then combining changes nothing; section 1 "Cache", DCP8
  paragraph: shard partials merged with their normalisation equal the unsharded
  answer, and 8x heads over 1/8 of the history keeps the arithmetic unchanged);
* the pages' own worked numbers (the DCP8 payload estimate, tests/golden).

Each pin is a function taking the oracle routine(s) it checks, so that the
mutation tests at the end can plant a mistake in a copy of the oracle and show
that some pin fails.
"""

import decimal
import json
import math
import os

import numpy as np
import pytest

import oracle
from mla_split_kv_decode_amd import workloads as wk

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
TAU = float(np.float32(1.0 / math.sqrt(192.0)))


def torch_bf16_to_f64(bits):
    """bf16 bit patterns -> fp64 through torch's own bfloat16 type (independent of the
    oracle's decoder)."""
    import torch

    b = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16))
    return torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()


def torch_e4m3fn_to_f64(codes):
    """E4M3FN codes -> fp64 through torch's float8_e4m3fn type."""
    import torch

    c = np.ascontiguousarray(np.asarray(codes, dtype=np.uint8))
    return torch.from_numpy(c).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def bf16_values(rng, shape, scale=1.0):
    """Random values exactly representable in bf16 (via the generator's cast)."""
    bits = wk.to_bf16_bits(rng.standard_normal(shape).astype(np.float32) * scale)
    return torch_bf16_to_f64(bits)


# ------------------------------------------------------------------ P1 decimal

def decimal_attention(q_rows, x, tau, prec=50):
    """Softmax attention in exact decimal arithmetic (prec significant digits)."""
    ctx = decimal.Context(prec=prec)
    D = decimal.Decimal
    tau_d = D(tau)
    # rows of x may be given as Decimals already (exact products such as code x scale)
    xs = [[v if isinstance(v, D) else D(float(v)) for v in row] for row in x]
    outs, lses = [], []
    for q in q_rows:
        qd = [D(float(v)) for v in q]
        s = [ctx.multiply(tau_d, sum((a * b for a, b in zip(qd, row)), D(0))) for row in xs]
        m = max(s)
        w = [ctx.exp(si - m) for si in s]
        l = sum(w, D(0))
        o = []
        for e in range(oracle.D_V):
            acc = sum((wj * row[e] for wj, row in zip(w, xs)), D(0))
            o.append(float(ctx.divide(acc, l)))
        outs.append(o)
        lses.append(float(m + ctx.ln(l)))
    return np.array(outs), np.array(lses)


def pin_decimal(attention_fn, cases=((1, 1), (2, 2), (3, 3), (1, 5), (2, 8))):
    rng = np.random.default_rng(11)
    worst = 0.0
    for n_rows, n in cases:
        q = bf16_values(rng, (n_rows, oracle.D_LATENT))
        x = bf16_values(rng, (n, oracle.D_LATENT))
        o, lse = attention_fn(q, x, TAU)
        od, lsed = decimal_attention(q, x, TAU)
        worst = max(worst, float(np.abs(o - od).max()), float(np.abs(lse - lsed).max()))
    return worst


def test_decimal_brute_force():
    assert pin_decimal(oracle.attention) <= 1e-12


def decimal_decode_paged(wl, r, t, h):
    """One output row of a paged workload, with the causal reading written out
    independently of the oracle (token t of T sees the first L - T + t + 1
    positions), every position gathered one by one, and the stored values decoded by
    torch's bfloat16 / float8_e4m3fn types.  An FP8 value is its code's value times the
    per-tensor scale, formed here in exact decimal arithmetic (Kimi K3 on MI355X,
    section 1 "Cache": the latents are stored in FP8)."""
    L = int(wl.seq_lens[r])
    n = L - wl.q_len + t + 1
    rows = []
    for j in range(n):
        page = int(wl.block_table[r][j // wl.page_size])
        raw = wl.pool[page, j % wl.page_size]
        if wl.kv_format == "bf16":
            rows.append([decimal.Decimal(float(v)) for v in torch_bf16_to_f64(raw)])
        else:
            sigma = decimal.Decimal(float(np.float32(wl.kv_scale)))
            rows.append([decimal.Decimal(float(v)) * sigma for v in torch_e4m3fn_to_f64(raw)])
    q = torch_bf16_to_f64(wl.q_bits[r, t, h])[None]
    return decimal_attention(q, rows, float(wl.softmax_scale), prec=40)


def pin_decimal_paged(decode_paged_fn, kv_format, seed=5):
    """Largest difference between decode_paged_fn and the decimal brute force on a small
    shuffled paged workload with a causal two-token verify."""
    wl = wk.make_workload(None, seed=seed, batch=2, q_len=2, num_heads=3, seq_lens=[70, 5],
                          kv_format=kv_format, shuffled=True)
    o, lse = decode_paged_fn(wl.q_bits, wl.pool, kv_format, wl.kv_scale, wl.block_table,
                             wl.seq_lens, wl.page_size, wl.softmax_scale, causal=True)
    worst = 0.0
    for r, t, h in [(0, 0, 0), (0, 1, 2), (1, 0, 1), (1, 1, 0)]:
        od, lsed = decimal_decode_paged(wl, r, t, h)
        worst = max(worst, float(np.abs(o[r, t, h] - od[0]).max()), abs(float(lse[r, t, h] - lsed[0])))
    return worst


def test_decimal_paged_decode():
    assert pin_decimal_paged(oracle.decode_paged, "bf16") <= 1e-12


def test_decimal_paged_decode_fp8():
    """FP8 pool: the oracle's codes x scale against decimal codes x scale, the codes
    decoded by torch's float8_e4m3fn (the scale of this workload is about 1/100, so a
    division in place of the product, or a dropped scale, is far off)."""
    wl = wk.make_workload(None, seed=5, batch=1, q_len=1, num_heads=1, seq_lens=[3],
                          kv_format="fp8_e4m3fn")
    assert 1e-3 < float(wl.kv_scale) < 0.1
    assert pin_decimal_paged(oracle.decode_paged, "fp8_e4m3fn") <= 1e-12


def test_fp8_scale_mutants_fail(monkeypatch):
    """Planted in the oracle: the FP8 rows divided by the scale, or the scale dropped."""
    import importlib

    att = importlib.import_module("oracle.attention")  # the module (the package re-exports a function of that name)
    good = att.decode_latent_rows
    for mutant in (lambda raw, fmt, sc: good(raw, fmt, 1.0) / float(np.float32(sc)) if fmt != "bf16"
                   else good(raw, fmt, sc),
                   lambda raw, fmt, sc: good(raw, fmt, 1.0) if fmt != "bf16" else good(raw, fmt, sc)):
        monkeypatch.setattr(att, "decode_latent_rows", mutant)
        assert pin_decimal_paged(att.decode_paged, "fp8_e4m3fn") > 1e-3
        assert pin_decimal_paged(att.decode_paged, "bf16") <= 1e-12
    monkeypatch.setattr(att, "decode_latent_rows", good)
    assert pin_decimal_paged(att.decode_paged, "fp8_e4m3fn") <= 1e-12


def pin_bf16_decoder(decode_fn):
    """Number of the 65,536 bf16 bit patterns that decode_fn gets wrong against torch's
    bfloat16 -> float64 conversion (NaN patterns must give NaN; the sign of zero counts)."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    mine = np.asarray(decode_fn(bits), dtype=np.float64)
    ref = torch_bf16_to_f64(bits)
    nan_ok = np.isnan(mine) == np.isnan(ref)
    val_ok = np.isnan(ref) | ((mine == ref) & (np.signbit(mine) == np.signbit(ref)))
    return int(np.sum(~(nan_ok & val_ok)))


def test_bf16_decoder_all_patterns():
    assert pin_bf16_decoder(oracle.bf16_bits_to_f64) == 0
    # a few values written out from the format: sign, 8 exponent bits (bias 127), 7 mantissa bits
    v = oracle.bf16_bits_to_f64(np.array([0x3F80, 0xC000, 0x0001, 0x7F7F, 0x8000, 0x7F80],
                                         dtype=np.uint16))
    assert list(v[:4]) == [1.0, -2.0, 2.0 ** -133, (2 - 2.0 ** -7) * 2.0 ** 127]
    assert v[4] == 0.0 and np.signbit(v[4]) and v[5] == np.inf


def test_bf16_decoder_mutants_fail():
    def shift15(bits):
        return (np.asarray(bits, np.uint16).astype(np.uint32) << np.uint32(15)).view(np.float32).astype(np.float64)

    def as_fp16(bits):
        return np.asarray(bits, np.uint16).view(np.float16).astype(np.float64)

    def byte_swapped(bits):
        return oracle.bf16_bits_to_f64(np.asarray(bits, np.uint16).byteswap())

    for fn in (shift15, as_fp16, byte_swapped):
        assert pin_bf16_decoder(fn) > 1000


# ------------------------------------------------------------- P2 closed forms

def pin_closed_forms(attention_fn):
    """Return a list of (name, error) for the closed-form cases."""
    rng = np.random.default_rng(12)
    out = []
    q = bf16_values(rng, (2, oracle.D_LATENT))
    x = bf16_values(rng, (2, oracle.D_LATENT))
    # one position: O is that position's value row, LSE its score
    o, lse = attention_fn(q, x[:1], TAU)
    s0 = TAU * np.array([math.fsum(q[i] * x[0]) for i in range(2)])
    out.append(("n1_value", float(np.abs(o - x[0, :oracle.D_V][None]).max())))
    out.append(("n1_lse", float(np.abs(lse - s0).max())))
    # two positions: logistic weights, LSE = logaddexp
    o, lse = attention_fn(q, x, TAU)
    s = TAU * np.array([[math.fsum(q[i] * x[j]) for j in range(2)] for i in range(2)])
    w0 = 1.0 / (1.0 + np.exp(s[:, 1] - s[:, 0]))
    ref = w0[:, None] * x[0, :oracle.D_V] + (1 - w0)[:, None] * x[1, :oracle.D_V]
    out.append(("n2_value", float(np.abs(o - ref).max())))
    out.append(("n2_lse", float(np.abs(lse - np.logaddexp(s[:, 0], s[:, 1])).max())))
    # zero query (a zero-padded head): O = mean of V, LSE = ln n
    xn = bf16_values(rng, (37, oracle.D_LATENT))
    o, lse = attention_fn(np.zeros((1, oracle.D_LATENT)), xn, TAU)
    out.append(("zero_q_value", float(np.abs(o[0] - xn[:, :oracle.D_V].mean(axis=0)).max())))
    out.append(("zero_q_lse", abs(float(lse[0]) - math.log(37))))
    # query only on the 64 trailing (rotary) columns, keys tied there: every
    # score equals s, so O = mean of the first 512 columns and LSE = s + ln n.
    qr = np.zeros((1, oracle.D_LATENT))
    qr[0, oracle.D_V:] = bf16_values(rng, (64,))
    xt = bf16_values(rng, (9, oracle.D_LATENT))
    xt[:, oracle.D_V:] = xt[0, oracle.D_V:]
    o, lse = attention_fn(qr, xt, TAU)
    st = TAU * math.fsum(qr[0, oracle.D_V:] * xt[0, oracle.D_V:])
    out.append(("tied_value", float(np.abs(o[0] - xt[:, :oracle.D_V].mean(axis=0)).max())))
    out.append(("tied_lse", abs(float(lse[0]) - (st + math.log(9)))))
    # spike: one key along q with a huge score takes all the weight
    xs = bf16_values(rng, (16, oracle.D_LATENT))
    qs = bf16_values(rng, (1, oracle.D_LATENT))
    xs[5] = 64.0 * np.sign(qs[0])
    o, _ = attention_fn(qs, xs, TAU)
    out.append(("spike_value", float(np.abs(o[0] - xs[5, :oracle.D_V]).max())))
    return out


def test_closed_forms():
    errs = dict(pin_closed_forms(oracle.attention))
    assert errs["n1_value"] == 0.0
    for name, err in errs.items():
        assert err <= 1e-12, (name, err)


def pin_library(attention_fn):
    """scipy's logsumexp and softmax on independently computed scores."""
    from scipy.special import logsumexp, softmax

    rng = np.random.default_rng(13)
    q = bf16_values(rng, (5, oracle.D_LATENT))
    x = bf16_values(rng, (300, oracle.D_LATENT))
    s = TAU * np.einsum("rd,nd->rn", q, x)
    o, lse = attention_fn(q, x, TAU)
    e_lse = float(np.abs(lse - logsumexp(s, axis=1)).max())
    e_o = float(np.abs(o - softmax(s, axis=1) @ x[:, :oracle.D_V]).max())
    return max(e_lse, e_o)


def test_library_routines():
    assert pin_library(oracle.attention) <= 1e-12


# --------------------------------------------------------------- P3 invariants

def pin_split_merge(attention_fn, merge_fn, seed=14):
    """Random covers of the history (empty pieces included, any order):
    merging the pieces' (O, LSE) equals attending over the whole history."""
    rng = np.random.default_rng(seed)
    q = bf16_values(rng, (4, oracle.D_LATENT))
    x = bf16_values(rng, (1000, oracle.D_LATENT))
    o_ref, lse_ref = attention_fn(q, x, TAU)
    worst = 0.0
    for parts in (1, 2, 4, 16, 33):
        cuts = np.sort(rng.integers(0, 1001, size=parts - 1))
        bounds = np.concatenate([[0], cuts, [1000]])
        pieces = [attention_fn(q, x[a:b], TAU) for a, b in zip(bounds[:-1], bounds[1:])]
        order = rng.permutation(len(pieces))
        o, lse = merge_fn(np.stack([pieces[i][0] for i in order]),
                          np.stack([pieces[i][1] for i in order]))
        worst = max(worst, float(np.abs(o - o_ref).max()), float(np.abs(lse - lse_ref).max()))
    return worst


def test_split_merge_equals_unsplit():
    assert pin_split_merge(oracle.attention, oracle.merge) <= 1e-13


def test_merge_all_empty():
    o, lse = oracle.merge(np.zeros((3, 2, oracle.D_V)), np.full((3, 2), -np.inf))
    assert np.all(o == 0) and np.all(np.isneginf(lse))
    # one live part among empties passes through unchanged
    o_live = np.arange(2 * oracle.D_V, dtype=np.float64).reshape(2, oracle.D_V)
    lse_parts = np.array([[-np.inf, -np.inf], [1.5, -2.0], [-np.inf, -np.inf]])
    o_parts = np.zeros((3, 2, oracle.D_V))
    o_parts[1] = o_live
    o, lse = oracle.merge(o_parts, lse_parts)
    assert np.array_equal(o, o_live) and np.array_equal(lse, [1.5, -2.0])


def test_head_padding_leaves_real_heads():
    """12 real heads padded to 16 with zero rows or with copies of real heads."""
    rng = np.random.default_rng(15)
    q = bf16_values(rng, (1, 1, 12, oracle.D_LATENT))
    x = [bf16_values(rng, (777, oracle.D_LATENT))]
    o12, l12 = oracle.decode(q, x, TAU)
    for pad in ("zero", "copy"):
        q16 = np.zeros((1, 1, 16, oracle.D_LATENT))
        q16[:, :, :12] = q
        if pad == "copy":
            q16[:, :, 12:] = q[:, :, :4]
        o16, l16 = oracle.decode(q16, x, TAU)
        assert np.abs(o16[:, :, :12] - o12).max() <= 1e-15
        assert np.abs(l16[:, :, :12] - l12).max() <= 1e-15
        if pad == "zero":  # a zero pad head weighs every position alike
            assert np.abs(l16[0, 0, 12:] - math.log(777)).max() <= 1e-12
            assert np.abs(o16[0, 0, 12:] - x[0][:, :oracle.D_V].mean(axis=0)).max() <= 1e-12


def test_page_permutation_invariance():
    """The same logical history under two different physical page layouts."""
    wl = wk.make_workload(None, seed=16, batch=3, q_len=1, num_heads=4,
                          seq_lens=[200, 64, 129], shuffled=True)
    rng = np.random.default_rng(17)
    perm = rng.permutation(wl.num_pages)
    pool2 = np.empty_like(wl.pool)
    pool2[perm] = wl.pool  # physical page p moves to perm[p]
    table2 = np.where(wl.block_table >= 0, perm[np.maximum(wl.block_table, 0)], -1)
    a = oracle.decode_paged(wl.q_bits, wl.pool, "bf16", 1.0, wl.block_table, wl.seq_lens,
                            64, wl.softmax_scale)
    b = oracle.decode_paged(wl.q_bits, pool2, "bf16", 1.0, table2, wl.seq_lens, 64,
                            wl.softmax_scale)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def pin_causal_drafts(decode_fn):
    """Causal masking among T drafts (the last T cached positions).

    Returns a list of failures.  Token t must not depend on the latents of
    later drafts, must depend on its own latent, and must equal a one-token
    decode over the first L - T + t + 1 positions.
    """
    rng = np.random.default_rng(18)
    T, L, H = 4, 70, 3
    q = bf16_values(rng, (1, T, H, oracle.D_LATENT))
    x = bf16_values(rng, (L, oracle.D_LATENT))
    o, lse = decode_fn(q, [x], TAU)
    bad = []
    for t in range(T):
        o1, lse1 = decode_fn(q[:, t:t + 1], [x[:L - T + t + 1]], TAU)
        if not (np.abs(o1[0, 0] - o[0, t]).max() <= 1e-14 and
                np.abs(lse1[0, 0] - lse[0, t]).max() <= 1e-14):
            bad.append(("single_token", t))
    # spike the latent of draft d (position L - T + d) towards every query
    for d in range(T):
        xs = x.copy()
        xs[L - T + d] = 40.0 * np.sign(q[0, 0, 0])
        os_, _ = decode_fn(q, [xs], TAU)
        for t in range(T):
            changed = np.abs(os_[0, t] - o[0, t]).max() > 1e-6
            if changed != (d <= t):
                bad.append(("spike", d, t))
    return bad


def test_causal_among_drafts():
    assert pin_causal_drafts(oracle.decode) == []


def pin_dcp(decode_fn, merge_fn, layout):
    """DCP8 emulation: each shard decodes its local positions; merging the
    shards' (O, LSE) equals the unsharded decode."""
    rng = np.random.default_rng(19)
    B, H, L, ways = 2, 6, 8 * 150, 8
    q = bf16_values(rng, (B, 1, H, oracle.D_LATENT))
    xs = [bf16_values(rng, (L, oracle.D_LATENT)) for _ in range(B)]
    o_ref, lse_ref = decode_fn(q, xs, TAU)
    pos = np.arange(L)
    if layout == "contiguous":
        owner = pos // (L // ways)
    else:  # round-robin by 64-position page
        owner = (pos // 64) % ways
    parts = [decode_fn(q, [x[owner == s] for x in xs], TAU) for s in range(ways)]
    o, lse = merge_fn(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]))
    return max(float(np.abs(o - o_ref).max()), float(np.abs(lse - lse_ref).max()))


@pytest.mark.parametrize("layout", ["contiguous", "round_robin_pages"])
def test_dcp_shard_merge(layout):
    assert pin_dcp(oracle.decode, oracle.merge, layout) <= 1e-13


# --------------------------------------------------------- P4 / P6 counters

def test_work_conservation_dcp8():
    """8x the heads over 1/8 of the history: the same attention arithmetic."""
    g = json.load(open(os.path.join(GOLDEN, "payload_k3.json")))
    n = g["positions"]
    heads_tp = g["tp_heads_total"] // g["tp_ways"]
    assert heads_tp == g["printed_heads_per_gpu_tp8"]
    a = wk.attention_flops([n // g["dcp_ways"]], 1, g["tp_heads_total"])
    b = wk.attention_flops([n], 1, heads_tp)
    assert a == b


def test_payload_bytes_match_page():
    g = json.load(open(os.path.join(GOLDEN, "payload_k3.json")))
    per_layer = wk.kv_bytes([g["positions"]], "fp8_e4m3fn")
    total = g["mla_layers"] * per_layer
    assert total == 1_963_008_000
    assert round(total / 1e9, 2) == g["printed_payload_gb_per_gpu"]
    assert round(total / g["dcp_ways"] / 1e6) == g["printed_dcp8_payload_mb_per_gpu"]


# -------------------------------------------------------------- P5 FP8 codec

def test_e4m3fn_codec_all_codes():
    import torch

    codes = np.arange(256, dtype=np.uint8)
    mine = oracle.e4m3fn_codes_to_f64(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    both_nan = np.isnan(mine) & np.isnan(ref)
    assert np.array_equal(np.isnan(mine), np.isnan(ref))
    assert np.all(both_nan | (mine == ref))
    assert set(np.flatnonzero(np.isnan(mine))) == {0x7F, 0xFF}
    assert mine[0x7E] == 448.0 and mine[0x01] == 2.0 ** -9 and mine[0x08] == 2.0 ** -6


def test_e4m3fn_quantiser():
    vals = np.array([1.0625, 1.1875, 448.0, -448.0, 2.0 ** -10, 3 * 2.0 ** -11, 0.0],
                    dtype=np.float32)
    codes = wk.to_e4m3fn_codes(vals)
    dec = oracle.e4m3fn_codes_to_f64(codes)
    # ties to even: 1.0625 -> 1.0, 1.1875 -> 1.25; 2^-10 ties to 0, 3*2^-11 -> 2^-9
    assert list(dec) == [1.0, 1.25, 448.0, -448.0, 0.0, 2.0 ** -9, 0.0]
    wl = wk.make_workload(None, seed=20, batch=2, q_len=1, num_heads=2, seq_lens=[100, 30],
                          kv_format="fp8_e4m3fn")
    valid = np.concatenate([oracle.gather_latents(wl.pool, wl.block_table[r], int(L), 64)
                            for r, L in enumerate(wl.seq_lens)])
    assert not np.any((valid & 0x7F) == 0x7F)  # no NaN in valid data
    assert np.max(np.abs(oracle.e4m3fn_codes_to_f64(valid))) == 448.0


def test_generator_pins():
    wl = wk.make_workload("ragged")
    assert list(wl.seq_lens[:5]) == [26785, 3742, 6720, 8541, 6781]
    assert int(wl.seq_lens.sum()) == 1_002_597
    assert wl.num_pages - wk.SPARE_PAGES == 15_698
    assert wk.kv_bytes(wl.seq_lens, "bf16") == 1_154_991_744


def test_generator_poison():
    wl = wk.make_workload(None, seed=21, batch=2, q_len=1, num_heads=2, seq_lens=[65, 3])
    # the tail slots of each request's last page and the spare pages are NaN
    assert np.all(wl.pool[wl.block_table[0, 1], 1:] == wk.BF16_NAN)
    assert np.all(wl.pool[wl.block_table[1, 0], 3:] == wk.BF16_NAN)
    assert np.all(wl.pool[wl.extra["spare_pages"]] == wk.BF16_NAN)
    assert not np.any(np.isnan(oracle.decode_paged(
        wl.q_bits, wl.pool, "bf16", 1.0, wl.block_table, wl.seq_lens, 64,
        wl.softmax_scale)[0]))


# --------------------------------------------- mutations planted in the oracle

def _attention_mutant(kind):
    def fn(q_rows, x, softmax_scale):
        q_rows = np.asarray(q_rows, dtype=np.float64)
        x = np.asarray(x, dtype=np.float64)
        tau = float(softmax_scale)
        if x.shape[0] == 0:
            return np.zeros((q_rows.shape[0], oracle.D_V)), np.full(q_rows.shape[0], -np.inf)
        if kind == "k_512_only":
            s = tau * (x[:, :oracle.D_V] @ q_rows[:, :oracle.D_V].T)
        elif kind == "no_scale":
            s = x @ q_rows.T
        else:
            s = tau * (x @ q_rows.T)
        m = s.max(axis=0)
        w = np.exp(s - m)
        l = w.sum(axis=0)
        v = x[:, 64:] if kind == "v_last_512" else x[:, :oracle.D_V]
        o = (w.T @ v) / l[:, None]
        lse = m + np.log(l) if kind != "lse_log2" else m + np.log2(l)
        return o, lse
    return fn


@pytest.mark.parametrize("kind", ["k_512_only", "no_scale", "v_last_512", "lse_log2"])
def test_mutants_fail_a_pin(kind):
    fn = _attention_mutant(kind)
    errs = [pin_decimal(fn, cases=((2, 3),)), max(e for _, e in pin_closed_forms(fn))]
    assert max(errs) > 1e-6


def test_merge_mutant_fails():
    def plain_average(o_parts, lse_parts):
        return np.mean(o_parts, axis=0), np.max(lse_parts, axis=0)
    assert pin_split_merge(oracle.attention, plain_average) > 1e-3


def test_causal_mutants_fail():
    def shifted(delta):
        def decode_fn(q, latents, softmax_scale):
            T = q.shape[1]
            outs = []
            for r, x in enumerate(latents):
                L = x.shape[0]
                rows = [oracle.attention(q[r, t], x[:max(0, min(L, L - T + t + 1 + delta))],
                                         softmax_scale) for t in range(T)]
                outs.append(rows)
            o = np.array([[row[0] for row in req] for req in outs])
            lse = np.array([[row[1] for row in req] for req in outs])
            return o, lse
        return decode_fn
    assert pin_causal_drafts(shifted(0)) == []
    assert pin_causal_drafts(shifted(-1)) != []
    assert pin_causal_drafts(shifted(+1)) != []


# --------------------------------------------------- P7 cache append, FP8 quantiser
#
# Kimi K3 on MI355X, section 1 "Cache": the latent cache is stored in FP8 and grows by
# the new positions of every step.  The quantiser (nearest E4M3FN code, ties to even,
# saturating at 448) is pinned to the format's own codes, to torch's independent E4M3FN
# cast, and to worked ties; the append to positions and pages.

def _finite_codes():
    return np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)


def pin_quantiser_roundtrip(quantise):
    """Every finite code decodes to a value that encodes back to the same code."""
    codes = _finite_codes()
    vals = oracle.e4m3fn_codes_to_f64(codes).astype(np.float32)
    return np.flatnonzero(quantise(vals) != codes).tolist()


def pin_quantiser_library(quantise, n=200_000):
    """Against torch's float8_e4m3fn cast (round to nearest even) inside [-448, 448]:
    random magnitudes over the whole range, every code, and every midpoint between
    neighbouring codes (the ties)."""
    import torch

    rng = np.random.default_rng(71)
    mags = np.exp2(rng.uniform(-12.0, np.log2(448.0), n))
    signs = np.where(rng.random(n) < 0.5, -1.0, 1.0)
    pos = oracle.e4m3fn_codes_to_f64(np.arange(0x7F, dtype=np.uint8))
    mids = (pos[1:] + pos[:-1]) / 2
    vals = np.concatenate([mags * signs, pos, -pos, mids, -mids]).astype(np.float32)
    ref = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return int(np.count_nonzero(quantise(vals) != ref))


QUANTISER_WORKED = [  # (fp32 value, code): ties go to the even code; past 448 saturates
    # (near the top the codes are 384 0x7C, 416 0x7D, 448 0x7E: 400 and 432 are ties)
    (1.0625, 0x38), (1.1875, 0x3A), (-1.0625, 0xB8), (432.0, 0x7E), (400.0, 0x7C),
    (447.0, 0x7E), (464.0, 0x7E), (1e6, 0x7E), (-1e6, 0xFE), (np.inf, 0x7E),
    (-np.inf, 0xFE), (2.0 ** -10, 0x00), (3 * 2.0 ** -10, 0x02), (2.0 ** -9, 0x01),
    (0.0, 0x00), (-0.0, 0x80), (2.0 ** -6, 0x08), (15 * 2.0 ** -10, 0x08),
]


def pin_quantiser_worked(quantise):
    vals = np.array([v for v, _ in QUANTISER_WORKED], dtype=np.float32)
    want = np.array([c for _, c in QUANTISER_WORKED], dtype=np.uint8)
    return np.flatnonzero(quantise(vals) != want).tolist()


def test_quantiser_roundtrip_all_codes():
    assert pin_quantiser_roundtrip(oracle.quantize_e4m3fn) == []


def test_quantiser_matches_library_cast():
    assert pin_quantiser_library(oracle.quantize_e4m3fn) == 0


def test_quantiser_worked_ties_and_saturation():
    assert pin_quantiser_worked(oracle.quantize_e4m3fn) == []


def _append_case(kv_format, seed=81):
    wl = wk.make_workload(None, seed=seed, batch=3, q_len=3, num_heads=2, seq_lens=[3, 64, 130],
                          kv_format=kv_format, shuffled=True)
    rng = np.random.default_rng(seed + 1)
    lat = wk.to_bf16_bits(rng.standard_normal((3, 3, oracle.D_LATENT)).astype(np.float32) * 4)
    return wl, lat


def pin_kv_append(append_fn):
    """The new rows land at positions L - T .. L - 1 through the block table, stored as
    the cache format stores them (bf16 bits, or the library cast of x / scale), and no
    other byte of the pool changes.  Returns the failures."""
    import torch

    fails = []
    for kv_format in ("bf16", "fp8_e4m3fn"):
        wl, lat = _append_case(kv_format)
        scale = wl.kv_scale
        new = append_fn(wl.pool, wl.block_table, wl.seq_lens, lat, 3, kv_format, scale, 64)
        touched = np.zeros(wl.pool.shape[:2], dtype=bool)
        for r, L in enumerate(wl.seq_lens):
            for t in range(3):
                j = int(L) - 3 + t
                page, slot = int(wl.block_table[r][j // 64]), j % 64
                touched[page, slot] = True
                if kv_format == "bf16":
                    want = lat[r, t]
                else:
                    x = (lat[r, t].astype(np.uint32) << 16).view(np.float32) / np.float32(scale)
                    want = torch.from_numpy(np.clip(x, -448, 448).astype(np.float32)).to(
                        torch.float8_e4m3fn).view(torch.uint8).numpy()
                if not np.array_equal(new[page, slot], want):
                    fails.append((kv_format, r, t))
        if not np.array_equal(new[~touched], wl.pool[~touched]):
            fails.append((kv_format, "untouched rows changed"))
    return fails


def test_kv_append_positions_and_storage():
    assert pin_kv_append(oracle.kv_append) == []


def test_kv_append_then_decode_sees_the_new_rows():
    """Decoding after the append equals decoding a history built with the new rows."""
    wl, lat = _append_case("fp8_e4m3fn", seed=91)
    new = oracle.kv_append(wl.pool, wl.block_table, wl.seq_lens, lat, 3, "fp8_e4m3fn",
                           wl.kv_scale, 64)
    o1, l1 = oracle.decode_paged(wl.q_bits, new, "fp8_e4m3fn", wl.kv_scale, wl.block_table,
                                 wl.seq_lens, 64, wl.softmax_scale)
    for r, L in enumerate(wl.seq_lens):
        rows = oracle.gather_latents(new, wl.block_table[r], int(L), 64)
        want = np.stack([oracle.stored_row(lat[r, t], "fp8_e4m3fn", wl.kv_scale) for t in range(3)])
        assert np.array_equal(rows[-3:], want)
    assert np.isfinite(o1).all() and np.isfinite(l1).all()


def test_quantiser_mutants_fail_a_pin():
    def truncating(x32):   # toward zero instead of nearest
        x = np.asarray(x32, dtype=np.float32).astype(np.float64)
        pos = oracle.e4m3fn_codes_to_f64(np.arange(0x7F, dtype=np.uint8))
        a = np.minimum(np.abs(x), 448.0)
        code = (np.searchsorted(pos, a, side="right") - 1).astype(np.uint8)
        return code | np.where(np.signbit(x), np.uint8(0x80), np.uint8(0))

    def ties_away(x32):    # ties away from zero instead of to even
        x = np.asarray(x32, dtype=np.float32).astype(np.float64)
        pos = oracle.e4m3fn_codes_to_f64(np.arange(0x7F, dtype=np.uint8))
        a = np.minimum(np.abs(x), 448.0)
        hi = np.minimum(np.searchsorted(pos, a, side="left"), 126)
        lo = np.maximum(hi - 1, 0)
        code = np.where(pos[hi] - a <= a - pos[lo], hi, lo).astype(np.uint8)
        return code | np.where(np.signbit(x), np.uint8(0x80), np.uint8(0))

    def no_saturation(x32):  # past 448 becomes the NaN code
        x = np.asarray(x32, dtype=np.float32)
        c = oracle.quantize_e4m3fn(x)
        return np.where(np.abs(x) > 448, c | np.uint8(0x7F), c).astype(np.uint8)

    for mutant in (truncating, ties_away, no_saturation):
        assert (pin_quantiser_roundtrip(mutant) or pin_quantiser_library(mutant, n=20_000)
                or pin_quantiser_worked(mutant)), mutant.__name__


def test_kv_append_mutant_fails():
    def shifted(pool, block_table, seq_lens, lat, q_len, kv_format, scale, page_size):
        # one position too far
        return oracle.kv_append(pool, block_table, np.asarray(seq_lens) + 1, lat, q_len,
                                kv_format, scale, page_size)
    assert pin_kv_append(shifted) != []
