"""Host-side tests of the C-ABI library (no GPU needed).

* the library loads and exports every function include/mla_decode.h declares;
* argument checking: every bad argument is refused on the host, before any work
  is enqueued (no device is touched, so these run here);
* the partition planner: exact coverage of every request's pages, no overlap,
  page alignment, one slot per piece, contiguous slots per request, balance, and
  the workgroup counts of the named workloads.
"""

import ctypes
import os
import re

import numpy as np
import pytest

from mla_split_kv_decode_amd import binding as mb
from mla_split_kv_decode_amd import workloads as wk

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include",
                      "mla_decode.h")
TAU = float(wk.SOFTMAX_SCALE)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_[a-z_0-9]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert len(names) >= 12
    assert set(names) == set(mb.exported_symbols())
    for n in names:
        assert hasattr(lib, n), n


def test_timeline_build_exports_its_header(lib):
    """The stamping variant (include/mla_timeline.h) exports what its header declares, on
    top of the library's own symbols; the ordinary library exports none of it."""
    from mla_split_kv_decode_amd import build as mbuild

    tl_header = os.path.join(os.path.dirname(HEADER), "mla_timeline.h")
    text = re.sub(r"/\*.*?\*/", "", open(tl_header).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(mla_[a-z_0-9]+)\s*\(", text)))
    assert names == ["mla_timeline_clear", "mla_timeline_read"]
    for n in names:
        assert not hasattr(lib, n), n
    if not os.path.exists(mbuild.LIB_TIMELINE):
        pytest.skip("timeline build not present (build() makes it)")
    tl = ctypes.CDLL(mbuild.LIB_TIMELINE)
    for n in names + declared_functions():
        assert hasattr(tl, n), n


def test_version_and_status_strings(lib):
    assert "gfx950" in mb.version()
    assert mb.status_str(mb.MLA_OK) == "ok"
    assert mb.status_str(mb.MLA_ERR_WORKSPACE_TOO_SMALL) == "workspace too small"
    assert lib.mla_page_bytes(64, mb.MLA_BF16) == 64 * 576 * 2
    assert lib.mla_page_bytes(64, mb.MLA_FP8_E4M3FN) == 64 * 576
    assert lib.mla_page_bytes(64, 7) == 0


def test_block_table_check(lib):
    wl = wk.make_workload(None, seed=1, batch=3, q_len=1, num_heads=2, seq_lens=[65, 1, 200])
    assert mb.block_table_check(wl.block_table, wl.seq_lens, 64, wl.num_pages) == mb.MLA_OK
    bad = wl.block_table.copy()
    bad[2, 3] = wl.num_pages  # last page of request 2 out of range
    assert mb.block_table_check(bad, wl.seq_lens, 64, wl.num_pages) == mb.MLA_ERR_INVALID_ARGUMENT
    assert "block_table[2][3]" in lib.mla_last_error().decode()
    bad = wl.block_table.copy()
    bad[1, 0] = -5
    assert mb.block_table_check(bad, wl.seq_lens, 64, wl.num_pages) == mb.MLA_ERR_INVALID_ARGUMENT
    # entries past a request's pages are never read, so -1 there is fine
    assert wl.block_table[1, 1] == -1
    long = np.array([65, 1, 64 * wl.block_table.shape[1] + 1], dtype=np.int32)
    assert mb.block_table_check(wl.block_table, long, 64, wl.num_pages) == mb.MLA_ERR_INVALID_ARGUMENT


def plan_status(batch=1, q_len=1, heads=16, seq_lens=(1024,), scale=TAU, causal=1, splits=0,
                page=64, dtype=mb.MLA_BF16, cus=256):
    lib = mb.load()
    shape = mb.MlaDecodeShape(batch, q_len, heads, scale, causal, splits)
    sl = np.asarray(seq_lens, dtype=np.int32)
    h = ctypes.c_void_p()
    ws = ctypes.c_size_t()
    st = lib.mla_plan_create(ctypes.byref(shape), sl.ctypes.data, page, dtype, cus,
                             ctypes.byref(h), ctypes.byref(ws))
    if st == mb.MLA_OK:
        lib.mla_plan_destroy(h)
    else:
        assert not h.value
    return st


def test_plan_argument_checks():
    assert plan_status() == mb.MLA_OK
    E, U = mb.MLA_ERR_INVALID_ARGUMENT, mb.MLA_ERR_UNSUPPORTED
    assert plan_status(batch=0, seq_lens=()) == E
    assert plan_status(q_len=0) == E
    assert plan_status(heads=0) == E
    assert plan_status(scale=0.0) == E
    assert plan_status(scale=float("nan")) == E
    assert plan_status(causal=2) == E
    assert plan_status(splits=-1) == E
    assert plan_status(page=32) == U
    assert plan_status(dtype=mb.MLA_FP32) == U
    assert plan_status(q_len=4, seq_lens=(3,)) == E  # causal: seq_len < q_len
    assert plan_status(q_len=4, seq_lens=(3,), causal=0) == mb.MLA_OK  # a shard's history
    assert plan_status(q_len=4, seq_lens=(0,), causal=0) == E
    assert plan_status(heads=129) == mb.MLA_OK  # 9 row blocks
    assert plan_status(q_len=3, heads=48, seq_lens=(100,)) == mb.MLA_OK  # 9 row blocks
    assert plan_status(q_len=8, heads=16, seq_lens=(100,)) == mb.MLA_OK
    assert plan_status(q_len=4, heads=256, seq_lens=(100,)) == mb.MLA_OK  # 64 row blocks
    assert plan_status(heads=1025) == U  # 65 row blocks
    assert plan_status(q_len=5, heads=208, seq_lens=(100,)) == U  # 65 row blocks
    assert plan_status(cus=-1) == E


def _fake(addr=1 << 20):
    return ctypes.c_void_p(addr)


@pytest.mark.parametrize("dtype,q_len,heads,want", [
    (mb.MLA_FP8_E4M3FN, 1, 96, mb.MLA_OK),    # six row blocks: the FP8 row split
    (mb.MLA_FP8_E4M3FN, 4, 16, mb.MLA_OK),    # four row blocks
    (mb.MLA_FP8_E4M3FN, 1, 32, mb.MLA_OK),    # two
    (mb.MLA_FP8_E4M3FN, 1, 16, mb.MLA_ERR_UNSUPPORTED),  # one row block: no row split
    (mb.MLA_FP8_E4M3FN, 1, 12, mb.MLA_ERR_UNSUPPORTED),
    (mb.MLA_BF16, 1, 96, mb.MLA_ERR_UNSUPPORTED),        # no FP8 codes to feed
])
def test_fp8_qk_option_rules(dtype, q_len, heads, want):
    lib = mb.load()
    plan = mb.Plan(1, q_len, heads, [1000], TAU, kv_dtype=dtype, num_cus=256)
    assert lib.mla_plan_set_fp8_qk(plan.handle, 1) == want
    assert lib.mla_plan_set_fp8_qk(plan.handle, 0) == mb.MLA_OK  # off is always allowed
    assert lib.mla_plan_set_fp8_qk(plan.handle, 2) == mb.MLA_ERR_INVALID_ARGUMENT
    assert lib.mla_plan_set_fp8_qk(None, 0) == mb.MLA_ERR_INVALID_ARGUMENT
    if want != mb.MLA_OK:
        with pytest.raises(mb.MlaError):
            mb.Plan(1, q_len, heads, [1000], TAU, kv_dtype=dtype, num_cus=256, fp8_qk=True)


def test_binding_refuses_bad_tensors(monkeypatch):
    """The binding checks every tensor before the library sees it (the library takes any
    address as a device pointer).  CPU tensors stand in for device tensors here (the GPU
    check is patched out), so each refusal below is the shape / dtype / contiguity check
    it names; nothing reaches the library."""
    import torch

    with pytest.raises(ValueError, match="on a GPU"):
        mb.paged_kv(torch.zeros(2, 64, 576, dtype=torch.bfloat16), torch.zeros(1, 2, dtype=torch.int32),
                    torch.zeros(1, dtype=torch.int32), mb.MLA_BF16)
    monkeypatch.setattr(mb, "_on_gpu", lambda x: True)
    i32 = torch.int32
    pool = torch.zeros(4, 64, 576, dtype=torch.bfloat16)
    bt = torch.zeros(2, 3, dtype=i32)
    sl = torch.tensor([100, 5], dtype=i32)

    def refused(fn, match):
        with pytest.raises(ValueError, match=match):
            fn()

    refused(lambda: mb.paged_kv(np.zeros((4, 64, 576), np.uint16), bt, sl, mb.MLA_BF16), "torch")
    refused(lambda: mb.paged_kv(pool.view(torch.uint8), bt, sl, mb.MLA_BF16), "dtype")
    refused(lambda: mb.paged_kv(pool, bt, sl, mb.MLA_FP8_E4M3FN), "dtype")
    mb.paged_kv(pool.view(torch.uint8).view(8, 64, 576), bt, sl, mb.MLA_FP8_E4M3FN, 0.5)  # valid
    refused(lambda: mb.paged_kv(pool.view(2, 128, 576), bt, sl, mb.MLA_BF16), "pool must be")
    refused(lambda: mb.paged_kv(pool.view(4, 64 * 576), bt, sl, mb.MLA_BF16), "pool must be")
    refused(lambda: mb.paged_kv(pool, bt.to(torch.int64), sl, mb.MLA_BF16), "dtype")
    refused(lambda: mb.paged_kv(pool, bt.t(), sl, mb.MLA_BF16), "shape|contiguous")
    refused(lambda: mb.paged_kv(pool, bt, sl[:1], mb.MLA_BF16), "shape")
    refused(lambda: mb.paged_kv(pool, bt, sl, 7), "kv_dtype")
    kv = mb.paged_kv(pool, bt, sl, mb.MLA_BF16)
    plan = mb.Plan(2, 1, 12, [100, 5], TAU, num_cus=256)
    q = torch.zeros(2, 1, 12, 576, dtype=torch.bfloat16)
    ws = torch.zeros(plan.workspace_bytes, dtype=torch.uint8)
    out = torch.zeros(2, 1, 12, 512, dtype=torch.bfloat16)
    lse = torch.zeros(2, 1, 12, dtype=torch.float32)

    def dec(**kw):
        args = dict(q=q, kv=kv, ws=ws, out=out, out_lse=lse)
        args.update(kw)
        return lambda: mb.decode_splitkv(plan, args["q"], args["kv"], args["ws"], out=args["out"],
                                         out_lse=args["out_lse"], hidden=args.get("hidden"),
                                         out_dtype=args.get("out_dtype", mb.MLA_BF16))

    refused(dec(q=np.zeros((2, 1, 12, 576), np.uint16)), "torch")
    refused(dec(q=q.float()), "dtype")
    refused(dec(q=torch.zeros(2, 1, 16, 576, dtype=torch.bfloat16)), "shape")
    refused(dec(q=torch.zeros(2, 1, 12, 1152, dtype=torch.bfloat16)[..., :576]), "contiguous")
    refused(dec(ws=ws[:-1]), "workspace")
    refused(dec(out=out.float()), "dtype")
    refused(dec(out=out, out_dtype=mb.MLA_FP32), "dtype")
    refused(dec(out=torch.zeros(2, 1, 12, 576, dtype=torch.bfloat16)), "shape")
    refused(dec(out_lse=lse.double()), "dtype")
    refused(dec(out_lse=torch.zeros(2, 12, dtype=torch.float32)), "shape")
    refused(dec(hidden=torch.zeros(2, 1, dtype=torch.int64)), "dtype")
    refused(dec(hidden=torch.zeros(1, 2, dtype=i32)), "shape")
    refused(dec(kv=mb.paged_kv(pool, bt[:1], sl[:1], mb.MLA_BF16)), "requests")
    refused(dec(kv=mb.MlaPagedKV()), "paged_kv")
    lat = torch.zeros(2, 1, 576, dtype=torch.bfloat16)
    refused(lambda: mb.kv_append(pool, bt, sl, lat.float(), mb.MLA_BF16), "dtype")
    refused(lambda: mb.kv_append(pool, bt, sl, torch.zeros(3, 1, 576, dtype=torch.bfloat16), mb.MLA_BF16),
            "latents")
    refused(lambda: mb.kv_append(pool[:, :32].contiguous(), bt, sl, lat, mb.MLA_BF16), "pool must be")
    po = torch.zeros(3, 4, 512, dtype=torch.float32)
    pl = torch.zeros(3, 4, dtype=torch.float32)
    refused(lambda: mb.merge_lse(po.double(), pl), "dtype")
    refused(lambda: mb.merge_lse(po[..., :256], pl), "contiguous|part_o")
    refused(lambda: mb.merge_lse(po, pl[:, :3]), "part_lse")
    refused(lambda: mb.merge_lse(po, pl, out=torch.zeros(3, 512)), "out must")
    refused(lambda: mb.merge_lse(po, pl, out_lse=torch.zeros(5)), "out_lse")


def test_decode_refuses_misaligned_hidden():
    """hidden is a per-call device argument; its alignment is checked on the host."""
    lib = mb.load()
    plan = mb.Plan(2, 4, 16, [1000, 700], TAU, num_cus=256)
    kv = mb.MlaPagedKV(1 << 22, 32, 64, mb.MLA_BF16, 1.0, 1 << 21, 16, 1 << 23)
    st = lib.mla_decode_splitkv(plan.handle, _fake(), ctypes.byref(kv), _fake(1 << 24),
                                plan.workspace_bytes, _fake(1 << 25), mb.MLA_BF16, None,
                                _fake((1 << 26) + 2), None)
    assert st == mb.MLA_ERR_INVALID_ARGUMENT
    assert "hidden" in lib.mla_last_error().decode()


def test_kv_append_argument_checks_enqueue_nothing():
    """Every failing check of mla_kv_append returns before any device call."""
    lib = mb.load()
    E, U = mb.MLA_ERR_INVALID_ARGUMENT, mb.MLA_ERR_UNSUPPORTED

    def call(pool=_fake(1 << 22), npages=16, page=64, dt=mb.MLA_FP8_E4M3FN, scale=0.5,
             bt=_fake(1 << 21), maxp=16, sl=_fake(1 << 23), lat=_fake(1 << 24), batch=2, q_len=1):
        return lib.mla_kv_append(pool, npages, page, dt, scale, bt, maxp, sl, lat, batch, q_len, None)

    assert call(pool=None) == E
    assert call(bt=None) == E
    assert call(sl=None) == E
    assert call(lat=None) == E
    assert call(batch=0) == E
    assert call(q_len=0) == E
    assert call(npages=0) == E
    assert call(maxp=0) == E
    assert call(page=32) == U
    assert call(dt=mb.MLA_FP32) == U
    assert call(scale=0.0) == E
    assert call(scale=float("inf")) == E
    assert call(dt=mb.MLA_BF16, scale=0.5) == E
    assert call(pool=_fake((1 << 22) + 8)) == E
    assert call(lat=_fake((1 << 24) + 4)) == E
    assert call(sl=_fake((1 << 23) + 2)) == E
    assert call(batch=1 << 20, q_len=1 << 12) == U


def test_decode_argument_checks_enqueue_nothing():
    """Every failing check returns before any device call (so this runs on a CPU)."""
    lib = mb.load()
    plan = mb.Plan(1, 1, 16, [1024], TAU, kv_dtype=mb.MLA_BF16, num_cus=256)
    bt = _fake(1 << 21)
    kv = mb.MlaPagedKV(1 << 22, 16, 64, mb.MLA_BF16, 1.0, 1 << 21, 16, 1 << 23)
    ws = plan.workspace_bytes

    def call(q=_fake(), kvd=kv, wsp=_fake(1 << 24), wsb=ws, out=_fake(1 << 25), od=mb.MLA_BF16,
             lse=None):
        return lib.mla_decode_splitkv(plan.handle, q, ctypes.byref(kvd), wsp, wsb, out, od, lse,
                                      None, None)

    E = mb.MLA_ERR_INVALID_ARGUMENT
    assert call(q=None) == E
    assert call(wsp=None) == E
    assert call(wsb=ws - 1) == mb.MLA_ERR_WORKSPACE_TOO_SMALL
    assert call(wsp=_fake((1 << 24) + 16)) == E  # workspace not 256-aligned
    assert call(q=_fake((1 << 20) + 2)) == E  # q not 16-byte aligned
    assert call(od=mb.MLA_FP8_E4M3FN) == mb.MLA_ERR_UNSUPPORTED
    bad = mb.MlaPagedKV(1 << 22, 16, 64, mb.MLA_FP8_E4M3FN, 1.0, 1 << 21, 16, 1 << 23)
    assert call(kvd=bad) == E  # dtype differs from the plan
    bad = mb.MlaPagedKV(1 << 22, 16, 64, mb.MLA_BF16, 0.5, 1 << 21, 16, 1 << 23)
    assert call(kvd=bad) == E  # bf16 needs kv_scale 1
    bad = mb.MlaPagedKV(None, 16, 64, mb.MLA_BF16, 1.0, 1 << 21, 16, 1 << 23)
    assert call(kvd=bad) == E
    bad = mb.MlaPagedKV(1 << 22, 16, 32, mb.MLA_BF16, 1.0, 1 << 21, 16, 1 << 23)
    assert call(kvd=bad) == E
    bad = mb.MlaPagedKV(1 << 22, 16, 64, mb.MLA_BF16, 1.0, 1 << 21, 15, 1 << 23)
    assert call(kvd=bad) == E  # 1024 positions need 16 pages per table row
    fplan = mb.Plan(1, 1, 16, [1024], TAU, kv_dtype=mb.MLA_FP8_E4M3FN, num_cus=256)
    for s in (0.0, -1.0, float("inf")):
        bad = mb.MlaPagedKV(1 << 22, 16, 64, mb.MLA_FP8_E4M3FN, s, 1 << 21, 16, 1 << 23)
        assert lib.mla_decode_splitkv(fplan.handle, _fake(), ctypes.byref(bad), _fake(1 << 24),
                                      fplan.workspace_bytes, _fake(1 << 25), mb.MLA_BF16, None,
                                      None, None) == E
    # merge checks
    assert lib.mla_merge_lse(None, mb.MLA_FP32, _fake(), 2, 4, _fake(), mb.MLA_BF16, None, None) == E
    assert lib.mla_merge_lse(_fake(), mb.MLA_FP32, _fake(), 0, 4, _fake(), mb.MLA_BF16, None, None) == E
    assert lib.mla_merge_lse(_fake(), 1, _fake(), 2, 4, _fake(), mb.MLA_BF16, None, None) == mb.MLA_ERR_UNSUPPORTED
    assert lib.mla_merge_lse(_fake(), mb.MLA_FP32, _fake(), 2, 4, _fake(3), mb.MLA_BF16, None, None) == E


# ----------------------------------------------------------------- planner

def check_plan(seq_lens, q_len=1, heads=16, splits=0, cus=256, dtype=mb.MLA_BF16):
    plan = mb.Plan(len(seq_lens), q_len, heads, seq_lens, TAU, num_splits=splits, kv_dtype=dtype,
                   num_cus=cus)
    work = plan.work()
    pages = [-(-int(L) // 64) for L in seq_lens]
    W, S = plan.num_units, plan.num_parts
    # every request's pages covered exactly once, by page-aligned pieces
    for r, n in enumerate(pages):
        mine = work[work[:, 1] == r]
        cover = np.zeros(n, dtype=np.int32)
        for _, _, pb, pe, _ in mine:
            assert 0 <= pb <= pe <= n
            cover[pb:pe] += 1
        assert np.all(cover == 1), (r, cover)
        nonempty = mine[mine[:, 3] > mine[:, 2]]
        slots = np.sort(nonempty[:, 4])
        if splits == 0:  # contiguous slot range, one per non-empty piece
            assert np.array_equal(slots, np.arange(slots[0], slots[0] + len(slots)))
    # slots unique and inside the workspace
    assert len(set(work[:, 4])) == len(work)
    assert work[:, 4].min() >= 0 and work[:, 4].max() < S
    assert set(work[:, 0]) <= set(range(W))
    rb = q_len * -(-heads // 16)
    G = 1 if rb == 1 else -(-rb // 2)  # row blocks go two to a workgroup (odd: one padding)
    assert plan.row_groups == G
    if splits == 0:
        P = sum(pages)
        # every compute unit busy when possible; with several row groups, whole units per
        # XCD (eight XCDs)
        target = cus if G == 1 else (8 * (cus // 8 // G) if cus // 8 >= G else cus // G)
        assert W == min(P, max(1, target))
        per_wg = np.zeros(W, dtype=np.int64)
        for w, _, pb, pe, _ in work:
            per_wg[w] += pe - pb
        assert per_wg.sum() == P
        assert per_wg.max() - per_wg.min() <= 1  # balanced to one page
        assert per_wg.min() >= 1
        assert S == W + len(seq_lens) - 1
    else:
        assert W == len(seq_lens) * splits and S == W
        sizes = work[:, 3] - work[:, 2]
        for r in range(len(seq_lens)):
            s = sizes[work[:, 1] == r]
            assert s.max() - s.min() <= 1
    return plan, work


@pytest.mark.parametrize("name", list(wk.CONFIGS))
def test_planner_named_workloads(name):
    spec = wk.CONFIGS[name]
    rng = np.random.default_rng(list(wk.CONFIGS).index(name) + 1)
    if "seq_len_range" in spec:
        lo, hi = spec["seq_len_range"]
        seq_lens = rng.integers(lo, hi + 1, size=spec["batch"])
    else:
        seq_lens = [spec["seq_len"]] * spec["batch"]
    dtype = mb.MLA_BF16 if spec["kv_format"] == "bf16" else mb.MLA_FP8_E4M3FN
    for splits in {0, spec["num_splits"]}:
        plan, _ = check_plan(list(seq_lens), spec["q_len"], spec["num_heads"], splits, dtype=dtype)
        if splits == 0:
            P = sum(-(-int(L) // 64) for L in seq_lens)
            G = plan.row_groups
            assert plan.num_units == min(P, 256 if G == 1 else 8 * (32 // G))
            assert plan.num_units * G <= 256
    # the named counts the pages give: 16 partitions per request, 4 for the tiny case
    if spec["num_splits"]:
        plan = mb.Plan(spec["batch"], spec["q_len"], spec["num_heads"], list(seq_lens), TAU,
                       num_splits=spec["num_splits"], kv_dtype=dtype, num_cus=256)
        assert plan.num_units == spec["batch"] * spec["num_splits"]


def test_planner_long32k_auto_fills_all_cus():
    plan, work = check_plan([32768], heads=12)
    assert plan.num_units == 256  # 512 pages -> 2 pages per workgroup
    assert np.all(work[:, 3] - work[:, 2] == 2)


@pytest.mark.parametrize("seq_lens", [[1], [64], [65], [1, 1, 1], [5000, 1, 64, 130, 7],
                                      list(range(1, 300, 7)), [100000] * 3])
@pytest.mark.parametrize("cus", [1, 7, 256])
def test_planner_invariants(seq_lens, cus):
    check_plan(seq_lens, cus=cus)
    check_plan(seq_lens, splits=3, cus=cus)
    check_plan(seq_lens, splits=16, cus=cus)


@pytest.mark.parametrize("q_len,heads", [(4, 16), (1, 96), (3, 16), (2, 96), (4, 256)])
@pytest.mark.parametrize("cus", [1, 7, 100, 256])
def test_planner_row_groups(q_len, heads, cus):
    seq_lens = [max(q_len, L) for L in (17750, 3, 700, 64)]
    check_plan(seq_lens, q_len=q_len, heads=heads, cus=cus)
    check_plan(seq_lens, q_len=q_len, heads=heads, splits=5, cus=cus)


def test_workspace_size():
    plan = mb.Plan(2, 4, 16, [500, 1000], TAU, num_cus=256)
    rows = 4 * 16
    o_bytes = -(-plan.num_parts * rows * 512 * 4 // 256) * 256
    assert plan.workspace_bytes == o_bytes + -(-plan.num_parts * rows * 4 // 256) * 256
