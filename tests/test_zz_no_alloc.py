"""The decode entry point that allocates nothing (mla_decode_splitkv_noalloc), through
the C ABI: its partial answers live in the library's per-GPU scratch array instead of
a caller's workspace.  Its outputs must equal mla_decode_splitkv's bit for bit (same
kernels, same plan) and meet the oracle's bars, on two calls in a row, the second with
a smaller input (the scratch keeps the first call's contents), and it refuses a plan
whose partial answers do not fit the scratch.
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


def _run(wl, noalloc, splits=0):
    import torch

    dev = wk.to_device(wl)
    kv_dtype = mb.MLA_BF16 if wl.kv_format == "bf16" else mb.MLA_FP8_E4M3FN
    plan = mb.Plan(wl.batch, wl.q_len, wl.num_heads, wl.seq_lens, wl.softmax_scale,
                   causal=wl.causal, num_splits=splits, kv_dtype=kv_dtype)
    B, T, H = wl.batch, wl.q_len, wl.num_heads
    out = torch.full((B, T, H, 512), 7.0, dtype=torch.bfloat16, device="cuda")
    lse = torch.full((B, T, H), 7.0, dtype=torch.float32, device="cuda")
    kv = mb.paged_kv(dev["pool"], dev["block_table"], dev["seq_lens"], kv_dtype, dev["kv_scale"])
    if noalloc:
        assert plan.workspace_bytes <= mb.NOALLOC_SCRATCH_BYTES
        mb.decode_splitkv_noalloc(plan, dev["q"], kv, out=out, out_lse=lse)
    else:
        mb.decode_splitkv(plan, dev["q"], kv, mb.workspace(plan), out=out, out_lse=lse)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def _check(wl, o, l):
    o_ref, l_ref = oracle.decode_paged(wl.q_bits, wl.pool, wl.kv_format, wl.kv_scale, wl.block_table,
                                       wl.seq_lens, wl.page_size, wl.softmax_scale, causal=wl.causal)
    eo, el = float(np.abs(o - o_ref).max()), float(np.abs(l - l_ref).max())
    print(f"[no-alloc] {wl.name}: max|dO|={eo:.3e} max|dLSE|={el:.3e}", flush=True)
    assert eo <= TOL_O[wl.kv_format] and el <= TOL_LSE, (eo, el)


def test_noalloc_matches_workspace_entry_point_twice():
    # first a larger problem (14 MB of partial answers), then a smaller one on the same scratch
    big = wk.make_workload(None, seed=901, batch=3, q_len=2, num_heads=48, seq_lens=[9000, 4100, 700],
                           kv_format="bf16", shuffled=True)
    small = wk.make_workload(None, seed=902, batch=1, q_len=1, num_heads=12, seq_lens=[1500],
                             kv_format="fp8_e4m3fn", shuffled=True)
    for wl in (big, small):
        o_ws, l_ws = _run(wl, noalloc=False)
        o_na, l_na = _run(wl, noalloc=True)
        assert np.array_equal(o_na, o_ws) and np.array_equal(l_na, l_ws)
        _check(wl, o_na, l_na)


def test_noalloc_refuses_a_plan_beyond_the_scratch():
    import torch

    # 64 row blocks (4 tokens x 256 heads) of 16 requests: 46 MiB of partial answers
    B, T, H, L = 16, 4, 256, 20000
    plan = mb.Plan(B, T, H, [L] * B, float(wk.SOFTMAX_SCALE))
    assert plan.workspace_bytes > mb.NOALLOC_SCRATCH_BYTES
    pool = torch.zeros((8, 64, 576), dtype=torch.bfloat16, device="cuda")
    bt = torch.zeros((B, -(-L // 64)), dtype=torch.int32, device="cuda")
    sl = torch.full((B,), L, dtype=torch.int32, device="cuda")
    kv = mb.paged_kv(pool, bt, sl, mb.MLA_BF16)
    q = torch.zeros((B, T, H, 576), dtype=torch.bfloat16, device="cuda")
    out = torch.zeros((B, T, H, 512), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(mb.MlaError) as err:
        mb.decode_splitkv_noalloc(plan, q, kv, out=out)
    assert err.value.status == mb.MLA_ERR_UNSUPPORTED
    # out and out_lse both missing: nothing to return, refused
    small = mb.Plan(1, 1, 16, [100], float(wk.SOFTMAX_SCALE))
    q1 = torch.zeros((1, 1, 16, 576), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(mb.MlaError) as err:
        mb.decode_splitkv_noalloc(small, q1, mb.paged_kv(pool, bt[:1], sl[:1], mb.MLA_BF16))
    assert err.value.status == mb.MLA_ERR_INVALID_ARGUMENT
    torch.cuda.synchronize()
