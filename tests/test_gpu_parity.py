"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Gates (element by element, real heads only): max |O_gpu - O_oracle| <= 1e-2 with
bf16 KV and <= 3e-2 with FP8 KV, max |LSE_gpu - LSE_oracle| <= 1e-3.  Exact
(bitwise) equalities where the method fixes them: repeated runs, page
permutation, padded heads.  The full-size workloads are compared on every request,
token and real head.
"""

import numpy as np
import pytest

import oracle
from mla_split_kv_decode_amd import binding as mb
from mla_split_kv_decode_amd import workloads as wk

pytestmark = pytest.mark.gpu

TOL_O = {"bf16": 1e-2, "fp8_e4m3fn": 3e-2}
TOL_LSE = 1e-3


@pytest.fixture(scope="module", autouse=True)
def _device():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mb.load(build_if_missing=False)


def kv_dtype_of(wl):
    return mb.MLA_BF16 if wl.kv_format == "bf16" else mb.MLA_FP8_E4M3FN


def run_gpu(wl, num_splits=None, dev=None, out_dtype="bf16", want_lse=True, heads=None,
            block_table=None, pool=None, canary=False, fp8_qk=False, hidden=None):
    """Decode a workload on the GPU; returns (O fp64 [B][T][H][512], LSE fp64 [B][T][H])."""
    import torch

    dev = dev or wk.to_device(wl, pool=pool)
    if block_table is not None:
        dev = dict(dev, block_table=torch.from_numpy(np.ascontiguousarray(block_table)).cuda())
    splits = wl.num_splits if num_splits is None else num_splits
    plan = mb.Plan(wl.batch, wl.q_len, wl.num_heads, wl.seq_lens, wl.softmax_scale,
                   causal=wl.causal, num_splits=splits, kv_dtype=kv_dtype_of(wl), fp8_qk=fp8_qk)
    hid = None
    if hidden is not None:
        hid = torch.from_numpy(np.ascontiguousarray(hidden, dtype=np.int32)).cuda()
    ws = mb.workspace(plan)
    B, T, H = wl.batch, wl.q_len, wl.num_heads
    tdt = torch.bfloat16 if out_dtype == "bf16" else torch.float32
    pad = 4096 if canary else 0
    out_buf = torch.full((B * T * H * 512 + 2 * pad,), 7.0, dtype=tdt, device="cuda")
    lse_buf = torch.full((B * T * H + 2 * pad,), 7.0, dtype=torch.float32, device="cuda")
    out = out_buf[pad:pad + B * T * H * 512].view(B, T, H, 512)
    lse = lse_buf[pad:pad + B * T * H].view(B, T, H) if want_lse else None
    kv = mb.paged_kv(dev["pool"], dev["block_table"], dev["seq_lens"], kv_dtype_of(wl),
                     dev["kv_scale"])
    mb.decode_splitkv(plan, dev["q"], kv, ws, out=out,
                      out_dtype=mb.MLA_BF16 if out_dtype == "bf16" else mb.MLA_FP32, out_lse=lse,
                      hidden=hid)
    torch.cuda.synchronize()
    if canary:
        assert torch.all(out_buf[:pad] == 7.0) and torch.all(out_buf[-pad:] == 7.0)
        assert torch.all(lse_buf[:pad] == 7.0) and torch.all(lse_buf[-pad:] == 7.0)
    o = out.float().cpu().numpy().astype(np.float64)
    l = lse.cpu().numpy().astype(np.float64) if want_lse else None
    return o, l


def run_oracle(wl, requests=None, heads=None, pool=None, block_table=None):
    return oracle.decode_paged(wl.q_bits, wl.pool if pool is None else pool, wl.kv_format,
                               wl.kv_scale, wl.block_table if block_table is None else block_table,
                               wl.seq_lens, wl.page_size, wl.softmax_scale, causal=wl.causal,
                               requests=requests, heads=heads)


def compare(wl, o_gpu, lse_gpu, o_ref, lse_ref, what=""):
    eo = float(np.abs(o_gpu - o_ref).max())
    el = float(np.abs(lse_gpu - lse_ref).max()) if lse_gpu is not None else 0.0
    rms = float(np.sqrt(np.mean(o_ref ** 2)))
    print(f"[parity] {wl.name} {what}: max|dO|={eo:.3e} (rel rms {eo / rms:.3e}) "
          f"max|dLSE|={el:.3e}", flush=True)
    assert np.isfinite(o_gpu).all() and (lse_gpu is None or np.isfinite(lse_gpu).all())
    assert eo <= TOL_O[wl.kv_format], (what, eo)
    assert el <= TOL_LSE, (what, el)
    return eo, el


def check_full(wl, num_splits=None, **kw):
    o, l = run_gpu(wl, num_splits=num_splits, **kw)
    o_ref, l_ref = run_oracle(wl)
    return compare(wl, o, l, o_ref, l_ref, f"splits={wl.num_splits if num_splits is None else num_splits}")


# ------------------------------------------------------------ small shapes

SMALL = [
    # batch, q_len, heads, seq_lens, splits, kv
    (1, 1, 16, [1000], 0, "bf16"),
    (1, 1, 16, [1000], 4, "bf16"),
    (2, 1, 12, [65, 130], 0, "bf16"),
    (3, 1, 16, [1, 64, 129], 2, "bf16"),
    (3, 1, 16, [1, 64, 129], 16, "bf16"),
    (2, 4, 16, [4, 70], 0, "bf16"),
    (2, 4, 12, [68, 200], 3, "bf16"),
    (2, 2, 16, [70, 200], 0, "bf16"),
    (1, 1, 96, [300], 0, "bf16"),
    (2, 1, 7, [500, 33], 0, "bf16"),
    (1, 8, 16, [100], 0, "bf16"),
    (1, 3, 32, [150], 0, "bf16"),
    (5, 1, 16, [3000, 5, 700, 64, 1], 0, "bf16"),
    (1, 1, 16, [1000], 0, "fp8_e4m3fn"),
    (2, 1, 96, [300, 77], 0, "fp8_e4m3fn"),
    (2, 4, 16, [4, 70], 0, "fp8_e4m3fn"),
    (3, 1, 12, [1, 64, 129], 5, "fp8_e4m3fn"),
    (1, 2, 48, [200], 0, "fp8_e4m3fn"),
    # odd row-block counts (one row block per workgroup), more than eight row blocks,
    # and several row groups under fixed splits
    (1, 3, 16, [150], 0, "bf16"),
    (2, 5, 16, [300, 70], 0, "bf16"),
    (2, 7, 16, [64, 500], 2, "bf16"),
    (1, 3, 48, [200], 0, "fp8_e4m3fn"),
    (2, 2, 96, [300, 100], 0, "bf16"),
    (2, 2, 96, [300, 100], 3, "fp8_e4m3fn"),
    (1, 4, 256, [130], 0, "bf16"),
    # more than 32 parts a row: the column-chunk merge
    (1, 1, 16, [4000], 0, "fp8_e4m3fn"),
    (2, 1, 12, [4000, 2500], 0, "bf16"),
    # parts of at least 4 MiB and an eighth of the KV: stored non-temporal (one row block
    # FP8, column-chunk merge; two row blocks bf16, row-wise merge)
    (1, 1, 16, [10000], 0, "fp8_e4m3fn"),
    (1, 1, 96, [4000], 0, "bf16"),
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: f"B{c[0]}T{c[1]}H{c[2]}L{'-'.join(map(str, c[3]))}s{c[4]}{c[5]}")
def test_small_shapes(case):
    B, T, H, seq_lens, splits, kv = case
    wl = wk.make_workload(None, seed=101 + len(seq_lens) * 7 + T, batch=B, q_len=T, num_heads=H,
                          seq_lens=seq_lens, kv_format=kv, shuffled=True, num_splits=splits)
    check_full(wl, canary=True)


def test_fp32_output_and_no_lse():
    wl = wk.make_workload(None, seed=102, batch=2, q_len=1, num_heads=16, seq_lens=[333, 900])
    o, l = run_gpu(wl, out_dtype="fp32")
    o_ref, l_ref = run_oracle(wl)
    eo, _ = compare(wl, o, l, o_ref, l_ref, "fp32 out")
    assert eo <= 2e-3  # no bf16 rounding anywhere but P
    o2, _ = run_gpu(wl, want_lse=False)
    assert np.abs(o2 - o_ref).max() <= TOL_O["bf16"]


def test_non_causal_multi_token():
    wl = wk.make_workload(None, seed=103, batch=2, q_len=3, num_heads=16, seq_lens=[50, 300],
                          causal=False)
    check_full(wl)


# ------------------------------------------------------------ named workloads

def test_tiny():
    wl = wk.make_workload("tiny")
    check_full(wl)           # 4 partitions
    check_full(wl, num_splits=0)


@pytest.fixture(scope="module")
def long32k():
    return wk.make_workload("long32k")


@pytest.mark.parametrize("splits", [16, 0, 1])
def test_long32k(long32k, splits):
    check_full(long32k, num_splits=splits)


def test_long32k_seeds():
    for seed in (201, 202):
        check_full(wk.make_workload("long32k", seed=seed), num_splits=0)


@pytest.fixture(scope="module")
def ragged():
    wl = wk.make_workload("ragged")
    return wl, run_oracle(wl)


def test_ragged_full(ragged):
    """All 64 requests (1,002,597 positions), every head, at auto splits."""
    wl, (o_ref, l_ref) = ragged
    o, l = run_gpu(wl, num_splits=0)
    compare(wl, o, l, o_ref, l_ref, "auto, all 64 requests")


@pytest.fixture(scope="module")
def dcp_fp8():
    wl = wk.make_workload("dcp_fp8")
    return wl, run_oracle(wl)


def test_dcp_fp8_shard_full(dcp_fp8):
    """All 8 requests and all 96 heads (six row blocks, three row groups of two) of the
    17,750-position FP8 shard."""
    wl, (o_ref, l_ref) = dcp_fp8
    o, l = run_gpu(wl)
    compare(wl, o, l, o_ref, l_ref, "shard, every request and head")


# ------------------------------------------------------------ FP8 matrix-core q.k (opt-in)
#
# The pool's E4M3FN codes enter the FP8 matrix cores as they are, each query row as
# hi + lo E4M3FN after a power-of-two row scale.  Same gates as the default path; and
# since hi + lo reproduces the bf16 query elements (all but the smallest exactly), the
# two paths agree far inside the gates.

F8QK_CASES = [c for c in SMALL if c[5] == "fp8_e4m3fn" and c[1] * -(-c[2] // 16) >= 2]


@pytest.mark.parametrize("case", F8QK_CASES,
                         ids=lambda c: f"B{c[0]}T{c[1]}H{c[2]}L{'-'.join(map(str, c[3]))}s{c[4]}")
def test_fp8_qk_small_shapes(case):
    B, T, H, seq_lens, splits, kv = case
    wl = wk.make_workload(None, seed=101 + len(seq_lens) * 7 + T, batch=B, q_len=T, num_heads=H,
                          seq_lens=seq_lens, kv_format=kv, shuffled=True, num_splits=splits)
    check_full(wl, canary=True, fp8_qk=True)


def test_fp8_qk_dcp_shard_full(dcp_fp8):
    wl, (o_ref, l_ref) = dcp_fp8
    o, l = run_gpu(wl, fp8_qk=True)
    compare(wl, o, l, o_ref, l_ref, "shard, FP8 q.k, every request and head")


def test_fp8_qk_agrees_with_bf16_qk():
    # The scores of the two paths differ only by the order of fp32 additions and the
    # error of the smallest query elements (below 2^-17 of their row's largest
    # magnitude): the LSE, computed from the scores alone, agrees to ~1e-5.  O goes
    # through the bf16 weights P, and a score that moves a little can flip the rounding
    # of its weight by one bf16 place (at most 2^-7 of the weight: eight significant
    # bits); the weights sum to the denominator, so O moves by at most 2^-7 max|V|.
    wl = wk.make_workload(None, seed=77, batch=2, q_len=2, num_heads=96, seq_lens=[3000, 1200],
                          kv_format="fp8_e4m3fn", shuffled=True)
    o0, l0 = run_gpu(wl, out_dtype="fp32")
    o1, l1 = run_gpu(wl, out_dtype="fp32", fp8_qk=True)
    do, dl = float(np.abs(o1 - o0).max()), float(np.abs(l1 - l0).max())
    vmax = 448.0 * float(wl.kv_scale)
    print(f"[parity] FP8 vs bf16 q.k: max|dO|={do:.3e} (bound {vmax / 128:.3e}) max|dLSE|={dl:.3e}",
          flush=True)
    assert dl <= 1e-4, dl
    assert do <= vmax / 128, (do, vmax)


@pytest.mark.parametrize("fp8_qk", [False, True], ids=["bf16qk", "fp8qk"])
def test_query_dynamic_range(fp8_qk):
    # rows whose largest magnitude is far from one (the FP8 q.k path's power-of-two row
    # scale) and a row of zeros (scale 1, uniform weights).  The FP8 matrix cores' dot
    # products hold about 17 significant bits of the score (measured: a row times 64,
    # LSE 359, came out 2.4e-3 off, where exact sums of the same hi + lo give 5e-5), so
    # the FP8 case stops at a row times 8 (LSE about 45)
    import dataclasses

    wl = wk.make_workload(None, seed=78, batch=1, q_len=1, num_heads=48, seq_lens=[700],
                          kv_format="fp8_e4m3fn", shuffled=True)
    q = wl.q_bits.copy()
    f = (q.astype(np.uint32) << 16).view(np.float32)
    for h, k in ((0, -20), (1, 3 if fp8_qk else 6), (2, -126), (17, 2 if fp8_qk else 3), (40, -3)):
        f[:, :, h] *= np.float32(2.0 ** k) if k > -126 else np.float32(0.0)
    q = (f.view(np.uint32) >> 16).astype(np.uint16)  # exact: powers of two, no subnormals
    wl = dataclasses.replace(wl, q_bits=q)
    check_full(wl, fp8_qk=fp8_qk)


# ------------------------------------------------------------ seeded random shapes

def _random_cases(n, seed=11):
    """Shapes drawn from a seeded generator: head counts with and without padding, one
    to four query tokens (causal or not), lengths from one page's worth to a few dozen
    pages, every split policy, both pool formats and the FP8 q.k option on FP8 multi-row
    shapes."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        kv = ["bf16", "fp8_e4m3fn"][rng.integers(2)]
        T = int(rng.choice([1, 1, 2, 3, 4]))
        H = int(rng.choice([7, 12, 16, 32, 48, 96, 128]))
        while T * -(-H // 16) > 64:
            H //= 2
        B = int(rng.integers(1, 5))
        seq = [int(rng.integers(T, 2500)) for _ in range(B)]
        splits = int(rng.choice([0, 0, 1, 3, 16]))
        causal = bool(rng.integers(2))
        f8qk = kv == "fp8_e4m3fn" and T * -(-H // 16) >= 2 and bool(rng.integers(2))
        if rng.integers(4) == 0:
            rng.integers(2)  # (a draw kept so that the seeded shapes stay the same)
        cases.append((i, B, T, H, seq, splits, kv, causal, f8qk))
    return cases


@pytest.mark.parametrize("case", _random_cases(16), ids=lambda c: f"r{c[0]}")
def test_random_shapes(case):
    i, B, T, H, seq, splits, kv, causal, f8qk = case
    wl = wk.make_workload(None, seed=1000 + i, batch=B, q_len=T, num_heads=H, seq_lens=seq,
                          kv_format=kv, shuffled=True, num_splits=splits, causal=causal)
    o, l = run_gpu(wl, canary=True, fp8_qk=f8qk)
    o_ref, l_ref = run_oracle(wl)
    compare(wl, o, l, o_ref, l_ref, f"B{B} T{T} H{H} s{splits} causal={causal} fp8qk={f8qk}")


def _wide_cases(n, seed=777):
    """A wider seeded draw: up to eight query tokens, 1 to 128 heads (odd head counts
    and head groups included), up to six requests, fixed splits beyond a request's page
    count, fp32 outputs on about a quarter of the cases."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        kv = ["bf16", "fp8_e4m3fn"][rng.integers(2)]
        T = int(rng.choice([1, 1, 2, 3, 4, 5, 6, 8]))
        H = int(rng.choice([1, 5, 12, 16, 17, 32, 48, 64, 96, 128]))
        while T * -(-H // 16) > 64:
            H //= 2
        B = int(rng.integers(1, 7))
        seq = [int(rng.integers(T, 3000)) for _ in range(B)]
        splits = int(rng.choice([0, 0, 0, 1, 2, 5, 16, 40]))
        causal = bool(rng.integers(2))
        f8qk = kv == "fp8_e4m3fn" and T * -(-H // 16) >= 2 and bool(rng.integers(3) == 0)
        out_dtype = "fp32" if rng.integers(4) == 0 else "bf16"
        cases.append((i, B, T, H, seq, splits, kv, causal, f8qk, out_dtype))
    return cases


@pytest.mark.parametrize("case", _wide_cases(120), ids=lambda c: f"w{c[0]}")
def test_random_shapes_wide(case):
    i, B, T, H, seq, splits, kv, causal, f8qk, out_dtype = case
    wl = wk.make_workload(None, seed=50777 + i, batch=B, q_len=T, num_heads=H, seq_lens=seq,
                          kv_format=kv, shuffled=True, num_splits=splits, causal=causal)
    o, l = run_gpu(wl, canary=True, fp8_qk=f8qk, out_dtype=out_dtype)
    o_ref, l_ref = run_oracle(wl)
    compare(wl, o, l, o_ref, l_ref, f"B{B} T{T} H{H} s{splits} causal={causal} fp8qk={f8qk} out={out_dtype}")


def test_spec_verify_full():
    """All 8 requests, 4 causal draft tokens each, 16 heads, 131,076 positions, at the
    16 partitions of the pages' policy and at auto splits."""
    wl = wk.make_workload("spec_verify")
    o_ref, l_ref = run_oracle(wl)
    o16, l16 = run_gpu(wl, num_splits=16)
    compare(wl, o16, l16, o_ref, l_ref, "16 splits, all requests")
    o0, l0 = run_gpu(wl, num_splits=0)
    compare(wl, o0, l0, o_ref, l_ref, "auto, all requests")


# ------------------------------------------------------------ DCP shards

def test_dcp_shard_merge():
    """8 position shards of one history: shard partials (bf16 O + LSE) merged on the
    host (oracle merge) and on the device (mla_merge_lse) equal the unsharded oracle."""
    import torch

    B, H, ways, per = 2, 96, 8, 520
    rng = np.random.default_rng(301)
    x32 = rng.standard_normal((B, ways * per, 576), dtype=np.float32)
    sigma = wk.e4m3fn_scale(np.abs(x32).max())
    codes = wk.to_e4m3fn_codes(x32 / sigma)
    q_bits = wk.to_bf16_bits(rng.standard_normal((B, 1, H, 576), dtype=np.float32))
    o_parts, l_parts = [], []
    for s in range(ways):
        seq = np.full(B, per, dtype=np.int32)
        pages = -(-per // 64)
        table = np.arange(B * pages, dtype=np.int32).reshape(B, pages)
        pool = np.full((B * pages, 64, 576), wk.E4M3FN_NAN, dtype=np.uint8)
        for r in range(B):
            rows = codes[r, s * per:(s + 1) * per]
            j = np.arange(per)
            pool[table[r, j // 64], j % 64] = rows
        wl = wk.Workload("dcp_shard", 301, B, 1, H, seq, "fp8_e4m3fn", sigma, table, pool, q_bits)
        o, l = run_gpu(wl)
        o_parts.append(o)
        l_parts.append(l)
    lat = [oracle.e4m3fn_codes_to_f64(codes[r]) * float(sigma) for r in range(B)]
    o_ref, l_ref = oracle.decode(oracle.bf16_bits_to_f64(q_bits), lat, wk.SOFTMAX_SCALE)
    o_host, l_host = oracle.merge(np.stack(o_parts), np.stack(l_parts))
    wl.name = "dcp_8_shards"
    compare(wl, o_host, l_host, o_ref, l_ref, "host merge of 8 shards")
    po = torch.from_numpy(np.stack(o_parts).astype(np.float32)).to(torch.bfloat16).cuda()
    pl = torch.from_numpy(np.stack(l_parts).astype(np.float32)).cuda()
    out = torch.empty((B * H, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B * H,), dtype=torch.float32, device="cuda")
    mb.merge_lse(po.view(ways, B * H, 512), pl.view(ways, B * H), out=out, out_lse=lse)
    torch.cuda.synchronize()
    compare(wl, out.float().cpu().numpy().reshape(B, 1, H, 512).astype(np.float64),
            lse.cpu().numpy().reshape(B, 1, H).astype(np.float64), o_ref, l_ref,
            "device merge of 8 shards")


@pytest.mark.parametrize("kv,split", [("fp8_e4m3fn", "contiguous"), ("bf16", "contiguous"),
                                      ("fp8_e4m3fn", "pages"), ("bf16", "pages")])
def test_dcp_multi_token_verification(kv, split):
    """DCP with T > 1 (several draft tokens verified under decode context parallelism):
    each request's history split into 8 position shards, contiguous ranges or pages dealt
    round robin.  The T drafts are the last T positions; with these lengths they lie in
    one page, so in one shard (the last range, or the owner of the last page), where they
    are that shard's last T positions: it is a causal call on its local history.  Every
    position of the other shards precedes the drafts and is visible to every token (a
    non-causal call).  The 8 shard answers, merged on the host and with mla_merge_lse,
    equal the unsharded causal oracle.  (Drafts that straddle two shards would need
    per-token visible counts, which the shard call does not take.)"""
    import dataclasses
    import torch

    B, T, H, ways = 2, 4, 48, 8
    # 65 and 41 pages: both last pages go to shard 0 under the round robin (one causal
    # flag serves a whole call, so the requests' drafts must share a shard)
    glob_lens = [65 * 64, 40 * 64 + 5]
    for L in glob_lens:
        assert (L - T) // 64 == (L - 1) // 64  # the drafts share a page
    rng = np.random.default_rng(302)
    xs = [rng.standard_normal((L, 576), dtype=np.float32) for L in glob_lens]
    if kv == "fp8_e4m3fn":
        sigma = wk.e4m3fn_scale(max(float(np.abs(x).max()) for x in xs))
        enc = [wk.to_e4m3fn_codes(x / sigma) for x in xs]
        empty, dec = wk.E4M3FN_NAN, (lambda c: oracle.e4m3fn_codes_to_f64(c) * float(sigma))
    else:
        sigma = np.float32(1.0)
        enc = [wk.to_bf16_bits(x) for x in xs]
        empty, dec = wk.BF16_NAN, oracle.bf16_bits_to_f64
    q_bits = wk.to_bf16_bits(rng.standard_normal((B, T, H, 576), dtype=np.float32))
    o_parts, l_parts = [], []
    def shard_positions(r, s):  # global positions held by shard s, in local order
        L = glob_lens[r]
        if split == "contiguous":
            return np.arange((L // ways) * s, (L // ways) * (s + 1) if s < ways - 1 else L)
        pos = np.arange(L)
        return pos[(pos // 64) % ways == s]

    for s in range(ways):
        held = [shard_positions(r, s) for r in range(B)]
        seq = np.array([len(h) for h in held], dtype=np.int32)
        has_drafts = [len(h) > 0 and h[-1] == glob_lens[r] - 1 for r, h in enumerate(held)]
        assert all(has_drafts) or not any(has_drafts)  # same shard for both requests here
        pages = [max(1, -(-int(n) // 64)) for n in seq]
        table = np.full((B, max(pages)), -1, dtype=np.int32)
        pool = np.full((sum(pages), 64, 576), empty, dtype=enc[0].dtype)
        nxt = 0
        for r in range(B):
            table[r, :pages[r]] = np.arange(nxt, nxt + pages[r])
            nxt += pages[r]
            j = np.arange(seq[r])
            pool[table[r, j // 64], j % 64] = enc[r][held[r]]
        wl = wk.Workload("dcp_shard_T4", 302, B, T, H, seq, kv, sigma, table, pool, q_bits,
                         causal=any(has_drafts))
        o, l = run_gpu(wl)
        o_parts.append(o)
        l_parts.append(l)
    lat = [dec(e) for e in enc]
    o_ref, l_ref = oracle.decode(oracle.bf16_bits_to_f64(q_bits), lat, wk.SOFTMAX_SCALE, causal=True)
    o_host, l_host = oracle.merge(np.stack(o_parts), np.stack(l_parts))
    wl = dataclasses.replace(wl, name="dcp_8_shards_T4")
    compare(wl, o_host, l_host, o_ref, l_ref, f"host merge of 8 {split} shards, T = 4")
    rows = B * T * H
    po = torch.from_numpy(np.stack(o_parts).astype(np.float32)).to(torch.bfloat16).cuda()
    pl = torch.from_numpy(np.stack(l_parts).astype(np.float32)).cuda()
    out = torch.empty((rows, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((rows,), dtype=torch.float32, device="cuda")
    mb.merge_lse(po.view(ways, rows, 512), pl.view(ways, rows), out=out, out_lse=lse)
    torch.cuda.synchronize()
    compare(wl, out.float().cpu().numpy().reshape(B, T, H, 512).astype(np.float64),
            lse.cpu().numpy().reshape(B, T, H).astype(np.float64), o_ref, l_ref,
            f"device merge of 8 {split} shards, T = 4")


@pytest.mark.parametrize("kv,split", [("bf16", "pages"), ("fp8_e4m3fn", "pages"),
                                      ("bf16", "ragged"), ("fp8_e4m3fn", "ragged")])
def test_dcp_straddling_drafts_with_hidden_tails(kv, split):
    """DCP with T > 1 where the drafts straddle two shards and lie in different shards per
    request.  Each shard call is non-causal with per-(request, token) hidden tails: token
    t (global position L - T + t) does not see the held positions after it, which are the
    last ones of the shard's local history.  A shard whose every held position is hidden
    from a token returns an empty part (LSE = -inf) for it.  The 8 merged shard answers
    equal the unsharded causal oracle."""
    import dataclasses
    import torch

    B, T, H, ways = 2, 4, 48, 8
    if split == "pages":  # drafts over pages 64|65 (shards 0, 1) and 39|40 (shards 7, 0)
        glob_lens = [65 * 64 + 2, 40 * 64 + 1]
    else:  # uneven contiguous ranges; the last shard holds only the last 2 positions
        glob_lens = [3000, 1537]
    rng = np.random.default_rng(305)
    xs = [rng.standard_normal((L, 576), dtype=np.float32) for L in glob_lens]
    if kv == "fp8_e4m3fn":
        sigma = wk.e4m3fn_scale(max(float(np.abs(x).max()) for x in xs))
        enc = [wk.to_e4m3fn_codes(x / sigma) for x in xs]
        empty, dec = wk.E4M3FN_NAN, (lambda c: oracle.e4m3fn_codes_to_f64(c) * float(sigma))
    else:
        sigma = np.float32(1.0)
        enc = [wk.to_bf16_bits(x) for x in xs]
        empty, dec = wk.BF16_NAN, oracle.bf16_bits_to_f64
    q_bits = wk.to_bf16_bits(rng.standard_normal((B, T, H, 576), dtype=np.float32))

    def shard_positions(r, s):
        L = glob_lens[r]
        pos = np.arange(L)
        if split == "pages":
            return pos[(pos // 64) % ways == s]
        cuts = np.concatenate([[0], np.sort(rng_cuts[r]), [L - 2, L]])
        return pos[cuts[s]:cuts[s + 1]]

    rng_cuts = [np.random.default_rng(306 + r).choice(np.arange(64, L - 64), ways - 2,
                                                      replace=False) for r, L in enumerate(glob_lens)]
    o_parts, l_parts, straddle = [], [], 0
    for s in range(ways):
        held = [shard_positions(r, s) for r in range(B)]
        seq = np.array([len(h) for h in held], dtype=np.int32)
        # token t of request r is at global position L - T + t and sees what precedes it
        hidden = np.array([[int(np.sum(held[r] > glob_lens[r] - T + t)) for t in range(T)]
                           for r in range(B)], dtype=np.int32)
        straddle += int(np.any((hidden > 0) & (hidden < seq[:, None])))
        pages = [max(1, -(-int(n) // 64)) for n in seq]
        table = np.full((B, max(pages)), -1, dtype=np.int32)
        pool = np.full((sum(pages), 64, 576), empty, dtype=enc[0].dtype)
        nxt = 0
        for r in range(B):
            table[r, :pages[r]] = np.arange(nxt, nxt + pages[r])
            nxt += pages[r]
            j = np.arange(seq[r])
            pool[table[r, j // 64], j % 64] = enc[r][held[r]]
        wl = wk.Workload("dcp_shard_T4_hidden", 305, B, T, H, seq, kv, sigma, table, pool,
                         q_bits, causal=False)
        o, l = run_gpu(wl, hidden=hidden)
        o_parts.append(o)
        l_parts.append(l)
    assert straddle >= 2  # more than one shard holds drafts
    lat = [dec(e) for e in enc]
    o_ref, l_ref = oracle.decode(oracle.bf16_bits_to_f64(q_bits), lat, wk.SOFTMAX_SCALE, causal=True)
    o_host, l_host = oracle.merge(np.stack(o_parts), np.stack(l_parts))
    wl = dataclasses.replace(wl, name="dcp_8_shards_T4_hidden")
    compare(wl, o_host, l_host, o_ref, l_ref, f"host merge of 8 {split} shards, straddling drafts")
    rows = B * T * H
    po = torch.from_numpy(np.stack(o_parts).astype(np.float32)).to(torch.bfloat16).cuda()
    pl = torch.from_numpy(np.stack(l_parts).astype(np.float32)).cuda()
    out = torch.empty((rows, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((rows,), dtype=torch.float32, device="cuda")
    mb.merge_lse(po.view(ways, rows, 512), pl.view(ways, rows), out=out, out_lse=lse)
    torch.cuda.synchronize()
    compare(wl, out.float().cpu().numpy().reshape(B, T, H, 512).astype(np.float64),
            lse.cpu().numpy().reshape(B, T, H).astype(np.float64), o_ref, l_ref,
            f"device merge of 8 {split} shards, straddling drafts")


@pytest.mark.parametrize("B,T,H,kv,f8qk", [(2, 4, 16, "bf16", False), (2, 3, 48, "fp8_e4m3fn", False),
                                           (3, 2, 96, "fp8_e4m3fn", False), (1, 4, 7, "bf16", False),
                                           (2, 3, 48, "fp8_e4m3fn", True)])
def test_hidden_tails_reproduce_causal_and_full(B, T, H, kv, f8qk):
    """Hidden tails q_len - 1 - t on a non-causal plan are the causal pattern, and zero
    tails on a causal plan show every position: both bitwise equal to the plain calls
    (also with QK^T on the FP8 matrix cores)."""
    wl = wk.make_workload(None, seed=303, batch=B, q_len=T, num_heads=H,
                          seq_lens=[700 + 97 * r for r in range(B)], kv_format=kv)
    causal_tail = np.tile(np.arange(T - 1, -1, -1, dtype=np.int32), (B, 1))
    o_c, l_c = run_gpu(dataclasses_replace(wl, causal=True), fp8_qk=f8qk)
    o_h, l_h = run_gpu(dataclasses_replace(wl, causal=False), hidden=causal_tail, fp8_qk=f8qk)
    assert np.array_equal(o_c, o_h) and np.array_equal(l_c, l_h)
    o_n, l_n = run_gpu(dataclasses_replace(wl, causal=False), fp8_qk=f8qk)
    o_z, l_z = run_gpu(dataclasses_replace(wl, causal=True), hidden=np.zeros((B, T), np.int32),
                       fp8_qk=f8qk)
    assert np.array_equal(o_n, o_z) and np.array_equal(l_n, l_z)
    assert not np.array_equal(l_c, l_n)  # the two patterns do differ


@pytest.mark.parametrize("kv,T,H,lens,causal", [
    ("bf16", 2, 16, [5000, 3001], True),
    ("bf16", 2, 12, [4100, 4100], False),
    ("fp8_e4m3fn", 1, 32, [9000, 6001], False),
    ("fp8_e4m3fn", 2, 16, [8000, 7100], True),
    # KV over eight times the partial answers: ordinary part stores (the kernel that two
    # draft tokens over a long history run)
    ("bf16", 2, 16, [61000, 60000], True),
], ids=["bf16_T2_causal", "bf16_T2_H12", "fp8_H32", "fp8_T2_causal", "bf16_T2_long"])
def test_streamed_two_row_blocks(kv, T, H, lens, causal):
    """Two row blocks in one row group over more than 8 MB of KV: the kernels whose page
    copies carry the non-temporal hint, every request and head, also with hidden tails
    (bitwise equal to the causal plan when the tails are the causal pattern)."""
    wl = wk.make_workload(None, seed=320 + T + H, batch=len(lens), q_len=T, num_heads=H,
                          seq_lens=lens, kv_format=kv, shuffled=True, causal=causal)
    assert wk.kv_bytes(wl.seq_lens, wl.kv_format) > 8 << 20
    plan = mb.Plan(wl.batch, T, H, wl.seq_lens, wl.softmax_scale, causal=causal,
                   kv_dtype=kv_dtype_of(wl))
    assert plan.row_groups == 1
    o, l = run_gpu(wl, canary=True)
    o_ref, l_ref = run_oracle(wl)
    compare(wl, o, l, o_ref, l_ref, "streamed two row blocks")
    if causal:
        tails = np.tile(np.arange(T - 1, -1, -1, dtype=np.int32), (wl.batch, 1))
        o_h, l_h = run_gpu(dataclasses_replace(wl, causal=False), hidden=tails)
        assert np.array_equal(o, o_h) and np.array_equal(l, l_h)


@pytest.mark.parametrize("splits", [0, 3])
def test_hidden_tails_one_row_block(splits):
    """One token and 12 heads (one row block): hidden tails on pieces of one page (auto
    splits here) and of several pages equal the oracle over the histories shortened by the
    tails."""
    lens = np.array([700, 130, 64, 65, 1000], dtype=np.int32)
    hid = np.array([[5], [64], [0], [1], [999]], dtype=np.int32)
    wl = wk.make_workload(None, seed=310, batch=5, q_len=1, num_heads=12, seq_lens=list(lens))
    o, l = run_gpu(wl, num_splits=splits, hidden=hid)
    o_ref, l_ref = run_oracle(dataclasses_replace(wl, seq_lens=lens - hid[:, 0]))
    compare(wl, o, l, o_ref, l_ref, f"hidden tails, one row block, splits={splits}")


def test_hidden_tail_covering_the_history_gives_empty_rows():
    wl = wk.make_workload(None, seed=304, batch=2, q_len=2, num_heads=16, seq_lens=[300, 500])
    hidden = np.array([[0, 300], [-5, 499]], dtype=np.int32)  # (1, 1): everything hidden
    o, l = run_gpu(wl, out_dtype="fp32", hidden=hidden)
    assert np.all(np.isneginf(l[0, 1])) and np.all(o[0, 1] == 0)
    o_ref, l_ref = run_oracle(dataclasses_replace(wl, causal=False))
    compare(wl, o[0, 0], l[0, 0], o_ref[0, 0], l_ref[0, 0], "hidden 0")
    compare(wl, o[1, 0], l[1, 0], o_ref[1, 0], l_ref[1, 0], "negative hidden counts as 0")
    # hiding 499 of 500 leaves position 0 alone: O is its value row, LSE its scaled score
    one = dataclasses_replace(wl, seq_lens=np.array([300, 1], dtype=np.int32), causal=False)
    o1, l1 = run_oracle(one, requests=[1])
    compare(wl, o[1:2, 1:2], l[1:2, 1:2], o1[:, 1:2], l1[:, 1:2], "one visible position")


def dataclasses_replace(wl, **kw):
    import dataclasses

    return dataclasses.replace(wl, **kw)


@pytest.mark.parametrize("P", [7, 32, 33, 300])
def test_merge_lse_api(P):
    """Both merge shapes: up to 32 parts a row runs row-wise, more by column chunks."""
    import torch

    rng = np.random.default_rng(302 + P)
    R = 40
    o = rng.standard_normal((P, R, 512))
    l = rng.standard_normal((P, R)) * 3
    l[2, :5] = -np.inf
    l[:, 7] = -np.inf  # all parts empty
    o[2, :5] = 0.0
    o[:, 7] = 0.0
    for pdt in (torch.float32, torch.bfloat16):
        po = torch.from_numpy(o.astype(np.float32)).to(pdt).cuda()
        o_in = po.float().cpu().numpy().astype(np.float64)
        pl = torch.from_numpy(l.astype(np.float32)).cuda()
        out = torch.empty((R, 512), dtype=torch.float32, device="cuda")
        lse = torch.empty((R,), dtype=torch.float32, device="cuda")
        mb.merge_lse(po, pl, out=out, out_lse=lse)
        torch.cuda.synchronize()
        o_ref, l_ref = oracle.merge(o_in, l.astype(np.float32).astype(np.float64))
        got_o = out.cpu().numpy()
        got_l = lse.cpu().numpy()
        assert np.all(got_o[7] == 0) and np.isneginf(got_l[7])
        fin = np.isfinite(l_ref)
        assert np.abs(got_o - o_ref).max() <= 1e-5
        assert np.abs(got_l[fin] - l_ref[fin]).max() <= 1e-5


# ------------------------------------------------------------ exact properties

def test_bitwise_determinism():
    wl = wk.make_workload(None, seed=401, batch=3, q_len=2, num_heads=12, seq_lens=[900, 64, 2000])
    a = run_gpu(wl)
    b = run_gpu(wl)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_page_permutation_bitwise():
    """Identity and shuffled tables over the same logical history give identical bits."""
    wl = wk.make_workload(None, seed=402, batch=2, q_len=1, num_heads=16, seq_lens=[1500, 700],
                          shuffled=True)
    rng = np.random.default_rng(403)
    perm = rng.permutation(wl.num_pages)
    pool2 = np.empty_like(wl.pool)
    pool2[perm] = wl.pool
    table2 = np.where(wl.block_table >= 0, perm[np.maximum(wl.block_table, 0)], -1).astype(np.int32)
    for splits in (0, 4):
        a = run_gpu(wl, num_splits=splits)
        b = run_gpu(wl, num_splits=splits, pool=pool2, block_table=table2)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_head_padding_bitwise():
    """12 real heads: padding rows inside the kernel or on the host (zero rows or copies of
    real heads, outputs discarded) leaves the 12 real heads bit-identical."""
    wl = wk.make_workload(None, seed=404, batch=2, q_len=1, num_heads=12, seq_lens=[3000, 100])
    o12, l12 = run_gpu(wl)
    for pad in ("zero", "copy"):
        q16 = np.zeros((2, 1, 16, 576), dtype=np.uint16)
        q16[:, :, :12] = wl.q_bits
        if pad == "copy":
            q16[:, :, 12:] = wl.q_bits[:, :, :4]
        wl16 = wk.Workload(wl.name, wl.seed, 2, 1, 16, wl.seq_lens, "bf16", wl.kv_scale,
                           wl.block_table, wl.pool, q16)
        o16, l16 = run_gpu(wl16)
        assert np.array_equal(o16[:, :, :12], o12) and np.array_equal(l16[:, :, :12], l12)


def test_split_count_invariance():
    wl = wk.make_workload(None, seed=405, batch=2, q_len=1, num_heads=16, seq_lens=[4096, 1000])
    ref = run_oracle(wl)
    outs = {s: run_gpu(wl, num_splits=s) for s in (1, 2, 7, 16, 64, 0)}
    for s, (o, l) in outs.items():
        compare(wl, o, l, ref[0], ref[1], f"splits={s}")
    # the partition is a scheduling choice: results agree to rounding
    for s, (o, l) in outs.items():
        assert np.abs(o - outs[1][0]).max() <= 4e-3 and np.abs(l - outs[1][1]).max() <= 1e-4


def test_pool_is_read_only():
    import torch

    wl = wk.make_workload(None, seed=406, batch=2, q_len=1, num_heads=16, seq_lens=[700, 70])
    dev = wk.to_device(wl)
    before = dev["pool"].clone()
    run_gpu(wl, dev=dev)
    assert torch.equal(before.view(torch.int16), dev["pool"].view(torch.int16))


# ------------------------------------------------------------ masks and tails

@pytest.mark.parametrize("prefix", [0, 1, 60, 63, 64, 65, 300, 1020])
def test_causal_short_context(prefix):
    T = 4
    wl = wk.make_workload(None, seed=500 + prefix, batch=2, q_len=T, num_heads=16,
                          seq_lens=[prefix + T, prefix + T + 9], kv_format="bf16")
    check_full(wl)


def test_spike_at_draft_positions():
    """A key at draft d aligned with every query dominates tokens t >= d only."""
    T = 4
    wl = wk.make_workload(None, seed=510, batch=1, q_len=T, num_heads=16, seq_lens=[200 + T])
    L = int(wl.seq_lens[0])
    base = run_gpu(wl)
    for d in range(T):
        pool = wl.pool.copy()
        j = L - T + d
        q = oracle.bf16_bits_to_f64(wl.q_bits[0, d])
        # |values| = 2 keeps |O| <= 2, where bf16 output rounding stays under 4e-3
        spike = wk.to_bf16_bits((2.0 * np.sign(q.sum(axis=0))).astype(np.float32))
        pool[wl.block_table[0, j // 64], j % 64] = spike
        o, l = run_gpu(wl, pool=pool)
        o_ref, l_ref = run_oracle(wl, pool=pool)
        compare(wl, o, l, o_ref, l_ref, f"spike at draft {d}")
        for t in range(T):
            changed = np.abs(l[0, t] - base[1][0, t]).max() > 1e-3
            assert changed == (t >= d), (d, t)


def test_table_swap_is_caught():
    """Replacing one page of a request by another request's page moves the result past
    the gates (the parity gates can see a single-page error at this length)."""
    wl = wk.make_workload(None, seed=520, batch=2, q_len=1, num_heads=16, seq_lens=[256, 256])
    bad = wl.block_table.copy()
    bad[0, 1] = wl.block_table[1, 2]
    o, l = run_gpu(wl, block_table=bad)
    o_ref, l_ref = run_oracle(wl)
    assert (np.abs(o - o_ref).max() > TOL_O["bf16"] or np.abs(l - l_ref).max() > TOL_LSE)
    o_bad, l_bad = run_oracle(wl, block_table=bad)
    assert np.abs(o - o_bad).max() <= TOL_O["bf16"] and np.abs(l - l_bad).max() <= TOL_LSE


@pytest.mark.parametrize("splits", [2, 0])
@pytest.mark.parametrize("which", ["past_pool", "negative", "int32_max"])
def test_out_of_range_page_gives_nan_not_fault(splits, which):
    """A page id outside the pool (past its end, negative, or the largest int32) is never
    dereferenced; that request's rows are NaN.  The entry is a piece's first page (two
    splits: pieces of two and three pages; auto splits: pieces of one page), whose id the
    one-row-block kernel fetches ahead of its query copies."""
    wl = wk.make_workload(None, seed=530, batch=3, q_len=1, num_heads=16, seq_lens=[300, 300, 300])
    bad = wl.block_table.copy()
    bad[1, 2] = {"past_pool": wl.num_pages + 1000, "negative": -3, "int32_max": 2**31 - 1}[which]
    o, l = run_gpu(wl, num_splits=splits, block_table=bad)
    assert np.isnan(l[1]).all() and np.isnan(o[1]).all()
    o_ref, l_ref = run_oracle(wl, requests=[0, 2])
    compare(wl, o[[0, 2]], l[[0, 2]], o_ref, l_ref, "other requests")


@pytest.mark.parametrize("kv,T,H", [("bf16", 1, 16), ("bf16", 4, 16), ("fp8_e4m3fn", 1, 16),
                                    ("fp8_e4m3fn", 1, 96)],
                         ids=["bf16-1block", "bf16-2blocks", "fp8-1block", "fp8-2blocks"])
def test_out_of_range_page_inside_the_page_loop(kv, T, H):
    """The same with the bad id on page 10 of a 16-page piece: its copy is issued from
    inside the page loop (in parts, for the kernels that split their copies)."""
    wl = wk.make_workload(None, seed=531, batch=3, q_len=T, num_heads=H, seq_lens=[1000, 1000, 1000],
                          kv_format=kv)
    bad = wl.block_table.copy()
    bad[1, 10] = -7
    o, l = run_gpu(wl, num_splits=1, block_table=bad)
    assert np.isnan(l[1]).all() and np.isnan(o[1]).all()
    o_ref, l_ref = run_oracle(wl, requests=[0, 2])
    compare(wl, o[[0, 2]], l[[0, 2]], o_ref, l_ref, "other requests")


# ------------------------------------------------------------ workspace layout

def test_partial_only_layout():
    """With no outputs only the partial stage runs; the workspace then holds fp32 O as
    [rows][16][parts][32] and LSE as [rows][parts], and merging each request's parts
    (its slots from the work list) with the oracle's merge gives the oracle's answer."""
    import torch

    wl = wk.make_workload(None, seed=610, batch=3, q_len=2, num_heads=12, seq_lens=[900, 70, 2500])
    dev = wk.to_device(wl)
    plan = mb.Plan(wl.batch, wl.q_len, wl.num_heads, wl.seq_lens, wl.softmax_scale, num_splits=0,
                   num_cus=24)
    ws = mb.workspace(plan)
    kv = mb.paged_kv(dev["pool"], dev["block_table"], dev["seq_lens"], mb.MLA_BF16)
    mb.decode_splitkv(plan, dev["q"], kv, ws, out=None, out_lse=None)
    torch.cuda.synchronize()
    S, rows = plan.num_parts, wl.q_len * wl.num_heads
    o_bytes = -(-S * rows * 512 * 4 // 256) * 256
    o = ws[:S * rows * 512 * 4].view(torch.float32)
    o = o.view(rows, 16, S, 32).permute(2, 0, 1, 3).reshape(S, rows, 512).cpu().numpy()
    lse = ws[o_bytes:o_bytes + S * rows * 4].view(torch.float32).view(rows, S).T.cpu().numpy()
    work = plan.work()
    o_ref, l_ref = run_oracle(wl)
    for r in range(wl.batch):
        slots = work[work[:, 1] == r][:, 4]
        om, lm = oracle.merge(o[slots].astype(np.float64), lse[slots].astype(np.float64))
        compare(wl, om.reshape(1, wl.q_len, wl.num_heads, 512), lm.reshape(1, wl.q_len, wl.num_heads),
                o_ref[r:r + 1], l_ref[r:r + 1], f"request {r} from {len(slots)} workspace parts")


@pytest.mark.parametrize("splits", [0, 3])
def test_device_lengths_disagreeing_with_plan_give_nan(splits):
    """Up to 64 requests the kernels take the plan's lengths from their arguments and
    compare each request's device length with it: a differing request is NaN, the
    others are unaffected."""
    import torch

    wl = wk.make_workload(None, seed=603, batch=2, q_len=1, num_heads=16, seq_lens=[700, 700])
    dev = wk.to_device(wl)
    plan = mb.Plan(2, 1, 16, [700, 500], wl.softmax_scale, num_splits=splits)  # request 1 differs
    ws = mb.workspace(plan)
    out = torch.empty((2, 1, 16, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((2, 1, 16), dtype=torch.float32, device="cuda")
    kv = mb.paged_kv(dev["pool"], dev["block_table"], dev["seq_lens"], mb.MLA_BF16)
    mb.decode_splitkv(plan, dev["q"], kv, ws, out=out, out_lse=lse)
    torch.cuda.synchronize()
    assert torch.isnan(lse[1]).all() and torch.isnan(out[1].float()).all()
    o_ref, l_ref = run_oracle(wl, requests=[0])
    compare(wl, out[:1].float().cpu().numpy().astype(np.float64),
            lse[:1].cpu().numpy().astype(np.float64), o_ref, l_ref, "consistent request")


def test_large_batch_device_lengths_path():
    """Past 64 requests the lengths come from the device (no plan copy in the kernel
    arguments): results match the oracle, and a total page count that differs from the
    plan's gives NaN everywhere."""
    import torch

    B = 70
    rng = np.random.default_rng(604)
    lens = rng.integers(1, 300, size=B)
    wl = wk.make_workload(None, seed=604, batch=B, q_len=1, num_heads=16, seq_lens=list(lens),
                          shuffled=True)
    o, l = run_gpu(wl, num_splits=0)
    req = [0, 33, 64, 65, 69]
    o_ref, l_ref = run_oracle(wl, requests=req)
    compare(wl, o[req], l[req], o_ref, l_ref, "70 requests, device lengths")
    dev = wk.to_device(wl)
    bad = list(lens)
    bad[5] = bad[5] + 64  # one more page on the host side
    plan = mb.Plan(B, 1, 16, bad, wl.softmax_scale)
    ws = mb.workspace(plan)
    out = torch.empty((B, 1, 16, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, 1, 16), dtype=torch.float32, device="cuda")
    table = np.zeros((B, wl.block_table.shape[1] + 1), dtype=np.int32)
    table[:, :-1] = np.maximum(wl.block_table, 0)
    kv = mb.paged_kv(dev["pool"], torch.from_numpy(table).cuda(), dev["seq_lens"], mb.MLA_BF16)
    mb.decode_splitkv(plan, dev["q"], kv, ws, out=out, out_lse=lse)
    torch.cuda.synchronize()
    assert torch.isnan(lse).all()


LARGE_BATCH = [
    # batch, q_len, heads, kv, splits, lengths
    (300, 1, 16, "bf16", 0, "short"),       # one request per scan thread, row-wise merge
    (600, 1, 16, "bf16", 0, "tiny"),        # two requests per scan thread
    (90, 1, 7, "bf16", 0, "short"),         # odd row count per request
    (80, 1, 16, "bf16", 0, "one_long"),     # > 32 parts for one request: column-chunk merge
    (100, 2, 16, "fp8_e4m3fn", 0, "short"),
    (130, 1, 48, "bf16", 0, "short"),       # several row groups
    (100, 1, 16, "bf16", 3, "short"),       # fixed splits
]


@pytest.mark.parametrize("case", LARGE_BATCH, ids=lambda c: f"B{c[0]}T{c[1]}H{c[2]}{c[3]}s{c[4]}{c[5]}")
def test_large_batch_device_lengths_full(case):
    """Past 64 requests every workgroup finds its pages and slots from the device lengths
    by a workgroup scan: every request of the batch matches the oracle, including the
    shortest requests the plan accepts, requests whose pages span several units and
    head counts that are not a multiple of 16."""
    B, T, H, kv, splits, mix = case
    rng = np.random.default_rng(605 + B + H)
    lens = rng.integers(T, 130 if mix == "tiny" else 400, size=B)
    lens[1], lens[2], lens[-1] = T, 65, 64
    if mix == "one_long":
        lens[B // 3] = 6000
    wl = wk.make_workload(None, seed=605 + B, batch=B, q_len=T, num_heads=H, seq_lens=list(lens),
                          kv_format=kv, shuffled=True)
    # Requests of a few positions give outputs of magnitude above 4, where one bf16 rounding
    # alone can reach 2^-6: the bar applies to the fp32 result, and the bf16 output must be
    # that result rounded to nearest even.
    o, l = run_gpu(wl, num_splits=splits, out_dtype="fp32")
    o_ref, l_ref = run_oracle(wl)
    compare(wl, o, l, o_ref, l_ref, f"{B} requests, device lengths")
    o16, l16 = run_gpu(wl, num_splits=splits)
    import torch
    rne = torch.from_numpy(o.astype(np.float32)).bfloat16().double().numpy()
    assert np.array_equal(o16, rne) and np.array_equal(l16, l)


@pytest.mark.parametrize("reserve", [65536, 131072])
def test_lds_reserve_leaves_results_unchanged(monkeypatch, reserve):
    """The residency experiment's knob only reserves unused LDS in the merge workgroups:
    the outputs are bitwise those of a plan made without it (row-wise and column-chunk
    merges)."""
    for lens in ([700, 70, 1300], [6000]):
        wl = wk.make_workload(None, seed=606, batch=len(lens), q_len=1, num_heads=16, seq_lens=lens)
        o0, l0 = run_gpu(wl, num_splits=0)
        monkeypatch.setenv("MLA_LDS_RESERVE", str(reserve))
        o1, l1 = run_gpu(wl, num_splits=0)
        monkeypatch.delenv("MLA_LDS_RESERVE")
        assert np.array_equal(o0, o1) and np.array_equal(l0, l1)


# ------------------------------------------------------------ cache append

def _append_inputs(kv_format, seed, batch, q_len, seq_lens, special=False):
    import torch

    wl = wk.make_workload(None, seed=seed, batch=batch, q_len=q_len, num_heads=16,
                          seq_lens=seq_lens, kv_format=kv_format, shuffled=True)
    rng = np.random.default_rng(seed + 1)
    x = rng.standard_normal((batch, q_len, oracle.D_LATENT)).astype(np.float32) * 3
    scale = float(wl.kv_scale)
    if special:  # ties, saturation, signed zeros and subnormal codes after x / scale
        if kv_format != "bf16":  # a power of two keeps x * scale and x / scale exact
            scale = float(2.0 ** np.round(np.log2(scale)))
        s = scale
        vals = np.array([1.0625, 1.1875, -1.0625, 432.0, 400.0, 447.0, 464.0, 1e6, -1e6, 2.0 ** -10,
                         3 * 2.0 ** -10, 2.0 ** -9, 0.0, -0.0, 2.0 ** -6, 15 * 2.0 ** -10, np.inf, -np.inf],
                        dtype=np.float64)
        x[0, 0, :len(vals)] = (vals * s).astype(np.float32)
    lat = wk.to_bf16_bits(x)
    dev = wk.to_device(wl)
    lat_dev = torch.from_numpy(lat.view(np.int16)).cuda().view(torch.bfloat16)
    return wl, lat, dev, lat_dev, scale


def _pool_bytes(pool_tensor):
    import torch

    t = pool_tensor.contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy().view(np.uint8)


@pytest.mark.parametrize("kv_format", ["bf16", "fp8_e4m3fn"])
@pytest.mark.parametrize("q_len", [1, 4])
def test_kv_append_bit_exact(kv_format, q_len):
    """Every byte of the pool after the append equals the oracle's (new rows written,
    nothing else touched), including ties, saturation and signed zeros."""
    import torch

    wl, lat, dev, lat_dev, scale = _append_inputs(kv_format, 501 + q_len, 3, q_len,
                                                  [q_len, 64 + q_len, 300], special=True)
    kvd = kv_dtype_of(wl)
    mb.kv_append(dev["pool"], dev["block_table"], dev["seq_lens"], lat_dev, kvd, scale)
    torch.cuda.synchronize()
    got = _pool_bytes(dev["pool"]).reshape(wl.pool.shape)
    want = oracle.kv_append(wl.pool, wl.block_table, wl.seq_lens, lat, q_len, kv_format,
                            scale, wl.page_size)
    bad = np.argwhere(got != want)
    print(f"[append] {kv_format} T={q_len}: {len(bad)} differing bytes of {got.size}", flush=True)
    assert len(bad) == 0, bad[:8]


def test_kv_append_skips_invalid_positions():
    """A device length below q_len, and a page id outside the pool, write nothing."""
    import torch

    wl, lat, dev, lat_dev, _ = _append_inputs("fp8_e4m3fn", 601, 3, 2, [100, 200, 50])
    sl = dev["seq_lens"].clone()
    sl[0] = 1  # below q_len: request 0 has no valid new positions 0 - 1 .. 0
    bt = dev["block_table"].clone()
    bt[2, (50 - 2) // 64] = 10 ** 6  # request 2's new rows point outside the pool
    mb.kv_append(dev["pool"], bt, sl, lat_dev, mb.MLA_FP8_E4M3FN, dev["kv_scale"])
    torch.cuda.synchronize()
    got = _pool_bytes(dev["pool"]).reshape(wl.pool.shape)
    # only request 1 is written; position -1 of request 0 is skipped, position 0 written
    want = oracle.kv_append(wl.pool, wl.block_table[1:2], wl.seq_lens[1:2], lat[1:2], 2,
                            "fp8_e4m3fn", wl.kv_scale, 64)
    p0 = int(wl.block_table[0][0])
    want[p0, 0] = oracle.stored_row(lat[0, 1], "fp8_e4m3fn", wl.kv_scale)
    assert np.array_equal(got, want)


def test_append_then_decode():
    """Append the new tokens of a verification step, then decode: matches the oracle on
    the appended pool (the path a serving step takes: write the drafts, verify them)."""
    import torch

    wl, lat, dev, lat_dev, _ = _append_inputs("fp8_e4m3fn", 701, 2, 3, [500, 130])
    mb.kv_append(dev["pool"], dev["block_table"], dev["seq_lens"], lat_dev, mb.MLA_FP8_E4M3FN,
                 dev["kv_scale"])
    new_pool = oracle.kv_append(wl.pool, wl.block_table, wl.seq_lens, lat, 3, "fp8_e4m3fn",
                                wl.kv_scale, 64)
    o, l = run_gpu(wl, num_splits=0, dev=dev)
    o_ref, l_ref = run_oracle(wl, pool=new_pool)
    compare(wl, o, l, o_ref, l_ref, "after append")
