"""Seeded synthetic inputs for MLA split-KV decode, plus the measurement counters.

This module holds no step of the attention method: it draws random numbers,
encodes them in the storage formats (bf16, FP8 E4M3FN with a per-tensor
scale), lays them out in a paged pool, and counts algorithmic bytes and flops.
Both the HIP path (through the binding) and the fp64 oracle (through the tests
and the bench's CPU baseline) consume what it produces; it imports neither.

Workloads (the shapes the source pages discuss; see the module-level table
``CONFIGS``):

* ``tiny``        batch 1, 16 heads, 1 token, 1,024 positions, contiguous bf16
                  pool, 4 history partitions;
* ``long32k``     batch 1, 12 heads (one GPU's share of 96 at TP8), 1 token,
                  32,768 positions, shuffled paged bf16 pool, 16 partitions
                  (the partition count of the AITER assembly policy in the
                  pages' section 4);
* ``ragged``      batch 64, 16 heads, lengths uniform in [1024, 32768];
* ``ragged256``   the same with 256 requests (a large serving batch: past the 64
                  requests whose lengths travel in the kernel arguments);
* ``dcp_fp8``     batch 8, 96 heads (all heads on one DCP8 shard), 17,750
                  local positions (142,000 / 8, the conversation of the pages'
                  section 1 payload estimate), FP8 E4M3FN pool;
* ``spec_verify`` batch 8, 16 heads, 4 causal query tokens (the verification
                  positions of section 5) on a 131,072 + 4 history.

Draw order for a seed (numpy PCG64 ``default_rng``): lengths (ragged only),
page permutation, queries, then latents request-major, position-major, 576
contiguous values per position.  Values are fp32 standard normals rounded to
bf16 by round-to-nearest-even, or divided by sigma = max|x| / 448 and rounded
to E4M3FN.  Slots past a request's last position and the spare pages are
poisoned with NaN so that any read of them shows up in the output.
"""

from dataclasses import dataclass, field
import math

import numpy as np

PAGE_SIZE = 64
D_LATENT = 576
D_V = 512
SPARE_PAGES = 8
BF16_NAN = np.uint16(0x7FC0)
E4M3FN_NAN = np.uint8(0x7F)
E4M3FN_MAX = 448.0
SOFTMAX_SCALE = np.float32(1.0 / math.sqrt(192.0))

CONFIGS = {
    "tiny": dict(batch=1, q_len=1, num_heads=16, seq_len=1024, kv_format="bf16",
                 shuffled=False, num_splits=4),
    "long32k": dict(batch=1, q_len=1, num_heads=12, seq_len=32768, kv_format="bf16",
                    shuffled=True, num_splits=16),
    "ragged": dict(batch=64, q_len=1, num_heads=16, seq_len_range=(1024, 32768),
                   kv_format="bf16", shuffled=True, num_splits=0),
    "dcp_fp8": dict(batch=8, q_len=1, num_heads=96, seq_len=17750, kv_format="fp8_e4m3fn",
                    shuffled=True, num_splits=0),
    "spec_verify": dict(batch=8, q_len=4, num_heads=16, seq_len=131072 + 4, kv_format="bf16",
                        shuffled=True, num_splits=16),
    # (after the five workloads above, whose seeds are their positions 1 .. 5)
    "ragged256": dict(batch=256, q_len=1, num_heads=16, seq_len_range=(1024, 32768),
                      kv_format="bf16", shuffled=True, num_splits=0),
}


@dataclass
class Workload:
    name: str
    seed: int
    batch: int
    q_len: int
    num_heads: int
    seq_lens: np.ndarray  # int32 [B]
    kv_format: str  # "bf16" | "fp8_e4m3fn"
    kv_scale: np.float32
    block_table: np.ndarray  # int32 [B][max_pages]
    pool: np.ndarray  # uint16 or uint8 [num_pages][PAGE_SIZE][576]
    q_bits: np.ndarray  # uint16 [B][T][H][576]
    softmax_scale: np.float32 = SOFTMAX_SCALE
    causal: bool = True
    num_splits: int = 0
    page_size: int = PAGE_SIZE
    extra: dict = field(default_factory=dict)

    @property
    def num_pages(self):
        return self.pool.shape[0]


def to_bf16_bits(x32):
    """fp32 array -> bf16 bit patterns (uint16), round to nearest even."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def to_e4m3fn_codes(x32):
    """fp32 array (already divided by the scale, |x| <= 448) -> E4M3FN codes."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def e4m3fn_scale(max_abs):
    """Per-tensor scale: the fp32 sigma that maps max|x| to the largest finite code."""
    return np.float32(np.float32(max_abs) / np.float32(E4M3FN_MAX))


def build_block_table(seq_lens, page_size, perm):
    """Assign logical pages, request by request, to physical pages perm[0], perm[1], ...

    Returns (block_table int32 [B][max_pages], spare physical pages).
    Entries past a request's last page are -1 (never read).
    """
    pages = [-(-int(L) // page_size) for L in seq_lens]
    max_pages = max(pages) if pages else 0
    table = np.full((len(seq_lens), max(max_pages, 1)), -1, dtype=np.int32)
    k = 0
    for r, n in enumerate(pages):
        table[r, :n] = perm[k:k + n]
        k += n
    return table, np.asarray(perm[k:], dtype=np.int64)


def _write_rows(pool, table_row, rows, page_size):
    j = np.arange(rows.shape[0])
    pool[table_row[j // page_size], j % page_size, :] = rows


def make_pool(rng, seq_lens, block_table, num_pages, kv_format, page_size=PAGE_SIZE):
    """Draw latents request-major, position-major and store them in a fresh pool.

    Returns (pool, kv_scale).  Unwritten slots hold the format's NaN code.
    """
    if kv_format == "bf16":
        pool = np.full((num_pages, page_size, D_LATENT), BF16_NAN, dtype=np.uint16)
        for r, L in enumerate(seq_lens):
            x = rng.standard_normal((int(L), D_LATENT), dtype=np.float32)
            _write_rows(pool, block_table[r], to_bf16_bits(x), page_size)
        return pool, np.float32(1.0)
    if kv_format == "fp8_e4m3fn":
        xs = [rng.standard_normal((int(L), D_LATENT), dtype=np.float32) for L in seq_lens]
        max_abs = max((float(np.abs(x).max()) for x in xs if x.size), default=1.0)  # empty requests
        sigma = e4m3fn_scale(max_abs)
        pool = np.full((num_pages, page_size, D_LATENT), E4M3FN_NAN, dtype=np.uint8)
        for r, x in enumerate(xs):
            _write_rows(pool, block_table[r], to_e4m3fn_codes(x / sigma), page_size)
        return pool, sigma
    raise ValueError(f"unknown kv_format {kv_format!r}")


def make_workload(name=None, seed=None, **overrides):
    """Build a named workload (``CONFIGS``) or a custom one from keyword arguments.

    Keys: batch, q_len, num_heads, seq_len | seq_len_range | seq_lens, kv_format,
    shuffled, num_splits, causal, softmax_scale.
    """
    spec = dict(CONFIGS[name]) if name is not None else {}
    spec.update(overrides)
    if seed is None:
        seed = list(CONFIGS).index(name) + 1 if name in CONFIGS else 0
    rng = np.random.default_rng(seed)
    batch = int(spec["batch"])
    if "seq_lens" in spec:
        seq_lens = np.asarray(spec["seq_lens"], dtype=np.int32)
    elif "seq_len_range" in spec:
        lo, hi = spec["seq_len_range"]
        seq_lens = rng.integers(lo, hi + 1, size=batch).astype(np.int32)
    else:
        seq_lens = np.full(batch, int(spec["seq_len"]), dtype=np.int32)
    assert seq_lens.shape == (batch,)
    page_size = int(spec.get("page_size", PAGE_SIZE))
    total_pages = int(sum(-(-int(L) // page_size) for L in seq_lens))
    num_pages = total_pages + SPARE_PAGES
    perm = rng.permutation(num_pages) if spec.get("shuffled", True) else np.arange(num_pages)
    block_table, spare = build_block_table(seq_lens, page_size, perm)
    q_len, num_heads = int(spec["q_len"]), int(spec["num_heads"])
    q32 = rng.standard_normal((batch, q_len, num_heads, D_LATENT), dtype=np.float32)
    q_bits = to_bf16_bits(q32)
    kv_format = spec.get("kv_format", "bf16")
    pool, kv_scale = make_pool(rng, seq_lens, block_table, num_pages, kv_format, page_size)
    return Workload(
        name=name or "custom", seed=int(seed), batch=batch, q_len=q_len, num_heads=num_heads,
        seq_lens=seq_lens, kv_format=kv_format, kv_scale=kv_scale, block_table=block_table,
        pool=pool, q_bits=q_bits,
        softmax_scale=np.float32(spec.get("softmax_scale", SOFTMAX_SCALE)),
        causal=bool(spec.get("causal", True)), num_splits=int(spec.get("num_splits", 0)),
        page_size=page_size, extra={"spare_pages": spare},
    )


def layer_pool(wl, layer, seed=None):
    """Another layer's pool for the same requests and block table (bench rotation)."""
    rng = np.random.default_rng([wl.seed if seed is None else seed, 1000 + int(layer)])
    pool, scale = make_pool(rng, wl.seq_lens, wl.block_table, wl.num_pages, wl.kv_format,
                            wl.page_size)
    return pool, scale


def timing_workload(name, seed=None, **overrides):
    """A named workload's lengths, block table and queries drawn exactly as
    ``make_workload`` draws them, with no pool (``pool`` is None): for timing runs whose
    pools are drawn on the device (``device_pools``), where drawing a gigabyte-sized
    pool on the host would take most of the run."""
    spec = dict(CONFIGS[name]) if name is not None else {}
    spec.update(overrides)
    if seed is None:
        seed = list(CONFIGS).index(name) + 1 if name in CONFIGS else 0
    rng = np.random.default_rng(seed)
    batch = int(spec["batch"])
    if "seq_lens" in spec:
        seq_lens = np.asarray(spec["seq_lens"], dtype=np.int32)
    elif "seq_len_range" in spec:
        lo, hi = spec["seq_len_range"]
        seq_lens = rng.integers(lo, hi + 1, size=batch).astype(np.int32)
    else:
        seq_lens = np.full(batch, int(spec["seq_len"]), dtype=np.int32)
    page_size = int(spec.get("page_size", PAGE_SIZE))
    total_pages = int(sum(-(-int(L) // page_size) for L in seq_lens))
    num_pages = total_pages + SPARE_PAGES
    perm = rng.permutation(num_pages) if spec.get("shuffled", True) else np.arange(num_pages)
    block_table, spare = build_block_table(seq_lens, page_size, perm)
    q_len, num_heads = int(spec["q_len"]), int(spec["num_heads"])
    q_bits = to_bf16_bits(rng.standard_normal((batch, q_len, num_heads, D_LATENT), dtype=np.float32))
    return Workload(
        name=name or "custom", seed=int(seed), batch=batch, q_len=q_len, num_heads=num_heads,
        seq_lens=seq_lens, kv_format=spec.get("kv_format", "bf16"), kv_scale=np.float32(1.0),
        block_table=block_table, pool=None, q_bits=q_bits,
        softmax_scale=np.float32(spec.get("softmax_scale", SOFTMAX_SCALE)),
        causal=bool(spec.get("causal", True)), num_splits=int(spec.get("num_splits", 0)),
        page_size=page_size, extra={"spare_pages": spare, "num_pages": num_pages},
    )


def device_pools(wl, layers, seed, device="cuda"):
    """`layers` pools of a timing workload drawn on the device with torch's seeded
    generator: N(0,1) values rounded to bf16, or for FP8 divided by
    sigma = max|x| / 448 and cast to E4M3FN (the same recipe as ``make_pool``, other
    random numbers).  Returns a list of (pool tensor, kv_scale)."""
    import torch

    n = int(wl.extra["num_pages"])
    g = torch.Generator(device=device)
    out = []
    for layer in range(layers):
        g.manual_seed(int(seed) * 1000 + layer)
        x = torch.randn((n, wl.page_size, D_LATENT), generator=g, device=device, dtype=torch.float32)
        if wl.kv_format == "bf16":
            out.append((x.to(torch.bfloat16), 1.0))
        else:
            sigma = float(np.float32(float(x.abs().max()) / E4M3FN_MAX))
            out.append(((x / sigma).to(torch.float8_e4m3fn).view(torch.uint8), sigma))
        del x
    return out


# ---------------------------------------------------------------- counters

def elem_bytes(kv_format):
    return {"bf16": 2, "fp8_e4m3fn": 1}[kv_format]


def kv_bytes(seq_lens, kv_format):
    """Algorithmic KV bytes of one layer-step: every cached latent read once."""
    return int(np.sum(np.asarray(seq_lens, dtype=np.int64))) * D_LATENT * elem_bytes(kv_format)


def visible_positions(seq_lens, q_len, causal):
    """Sum over (request, token) of the positions that token attends to."""
    total = 0
    for L in np.asarray(seq_lens, dtype=np.int64):
        for t in range(q_len):
            total += int(L - q_len + t + 1) if causal else int(L)
    return total


def attention_flops(seq_lens, q_len, num_heads, causal=True):
    """Algorithmic flops: 2 * (576 + 512) per (real head, token, visible position)."""
    return 2 * (D_LATENT + D_V) * num_heads * visible_positions(seq_lens, q_len, causal)


def io_bytes(seq_lens, q_len, num_heads, kv_format, with_lse=True):
    """All algorithmic bytes: KV + bf16 queries + bf16 outputs (+ fp32 LSE) + table."""
    b = len(seq_lens)
    pages = int(sum(-(-int(L) // PAGE_SIZE) for L in seq_lens))
    rows = b * q_len * num_heads
    return (kv_bytes(seq_lens, kv_format) + rows * D_LATENT * 2 + rows * D_V * 2
            + (rows * 4 if with_lse else 0) + pages * 4 + b * 4)


# ------------------------------------------------------------- device staging

def to_device(wl, device="cuda", pool=None):
    """Copy a workload's inputs to device tensors (plumbing only).

    Returns a dict: q (bf16 [B][T][H][576]), pool (bf16 or uint8
    [num_pages][64][576]), block_table and seq_lens (int32), kv_scale (float).
    """
    import torch

    pool = wl.pool if pool is None else pool
    q = torch.from_numpy(wl.q_bits.view(np.int16)).to(device).view(torch.bfloat16)
    if wl.kv_format == "bf16":
        pool_t = torch.from_numpy(pool.view(np.int16)).to(device).view(torch.bfloat16)
    else:
        pool_t = torch.from_numpy(pool).to(device)
    return {
        "q": q,
        "pool": pool_t,
        "block_table": torch.from_numpy(np.ascontiguousarray(wl.block_table)).to(device),
        "seq_lens": torch.from_numpy(np.ascontiguousarray(wl.seq_lens)).to(device),
        "kv_scale": float(wl.kv_scale),
    }
