"""Absorbed-MLA decode attention and the normalisation-carrying merge, in fp64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What is computed (Kimi K3 on MI355X, section 4 "MLA: AITER assembly decode"
and section 1 "Cache", DCP8 paragraph):

* Every cached position of a request holds one latent row of 576 values.  In
  absorbed MLA the key of a position is the whole row and its value is the
  first 512 entries of the same row (the pages give 576 bytes per position per
  layer in FP8; the 512 + 64 split and the K/V column reading are taken from
  the workload definition the build follows).
* A query row attends to the visible positions of its own request with an
  ordinary softmax over scaled dot products.  Heads are independent.
* The history may be cut into pieces whose partial answers are merged exactly
  with softmax weights; each partial answer carries its log-sum-exp (the
  "normalisation information" of the DCP8 paragraph).

Readings where the pages are silent:

* the softmax scale is an argument; it is rounded to fp32 first, because that
  fp32 is what the GPU library receives;
* multi-token verification (T query tokens per request, whose latents are the
  last T cached positions): token t sees positions 0 .. L - T + t, itself
  included;
* LSE is the natural log of the sum of exp(scaled scores); an empty visible set
  gives O = 0 and LSE = -inf.

The oracle is the unsplit two-pass definition.  It performs no blocking, no
online rescaling and no splitting; the matrix products are library calls.
"""

import numpy as np

from .numerics import bf16_bits_to_f64, e4m3fn_codes_to_f64

D_LATENT = 576  # columns of a cached latent row; the key uses all of them
D_V = 512  # the value is the first D_V columns of the same row


def attention(q_rows, x, softmax_scale):
    """Softmax attention of ``q_rows`` over every row of ``x``.

    q_rows: fp64 [R][576] query rows.  x: fp64 [n][576] visible latent rows.
    Returns (O fp64 [R][512], LSE fp64 [R]).

    Steps, for each query row q:
      s_j = tau * sum_d q[d] * x[j, d]         (all 576 columns)
      m   = max_j s_j
      w_j = exp(s_j - m)
      l   = sum_j w_j
      O   = sum_j w_j * x[j, :512] / l
      LSE = m + ln l
    """
    q_rows = np.asarray(q_rows, dtype=np.float64)
    x = np.asarray(x, dtype=np.float64)
    assert q_rows.ndim == 2 and q_rows.shape[1] == D_LATENT
    assert x.ndim == 2 and x.shape[1] == D_LATENT
    tau = float(softmax_scale)
    n_rows = q_rows.shape[0]
    if x.shape[0] == 0:
        return np.zeros((n_rows, D_V)), np.full(n_rows, -np.inf)
    s = tau * (x @ q_rows.T)  # [n][R]
    m = s.max(axis=0)  # [R]
    w = np.exp(s - m[None, :])  # [n][R]
    l = w.sum(axis=0)  # [R]
    o = (w.T @ x[:, :D_V]) / l[:, None]  # [R][512]
    lse = m + np.log(l)
    return o, lse


def visible_count(seq_len, q_len, t, causal):
    """Number of leading positions that query token ``t`` of a request sees.

    The request's last ``q_len`` cached positions are its own query tokens
    (the drafts under verification).  With causal masking token t sees
    positions 0 .. seq_len - q_len + t; without it every token sees all
    ``seq_len`` positions.
    """
    if causal:
        return seq_len - q_len + t + 1
    return seq_len


def decode(q, latents, softmax_scale, causal=True, heads=None):
    """Decode a batch.

    q: fp64 [B][T][H][576].  latents: list of B fp64 arrays [L_r][576] (the
    request's logical history, in position order).  Returns
    (O fp64 [B][T][H'][512], LSE fp64 [B][T][H']) where H' = len(heads) when a
    head subset is given (outputs of the other heads are simply not computed:
    heads are independent).
    """
    q = np.asarray(q, dtype=np.float64)
    n_req, q_len, n_heads, d = q.shape
    assert d == D_LATENT and len(latents) == n_req
    heads = np.arange(n_heads) if heads is None else np.asarray(heads)
    tau = float(np.float32(softmax_scale))
    out = np.zeros((n_req, q_len, len(heads), D_V))
    lse = np.zeros((n_req, q_len, len(heads)))
    for r in range(n_req):
        x = latents[r]
        seq_len = x.shape[0]
        for t in range(q_len):
            n = visible_count(seq_len, q_len, t, causal)
            assert 0 <= n <= seq_len
            out[r, t], lse[r, t] = attention(q[r, t, heads], x[:n], tau)
    return out, lse


def gather_latents(pool, block_table_row, seq_len, page_size):
    """Logical history of one request from a paged pool.

    Position j lives in physical page ``block_table_row[j // page_size]`` at
    slot ``j % page_size``.  ``pool`` is [num_pages][page_size][576] of any
    element type; the rows are returned in position order, undecoded.
    """
    j = np.arange(seq_len)
    pages = np.asarray(block_table_row)[j // page_size]
    slots = j % page_size
    return pool[pages, slots, :]


def decode_latent_rows(raw_rows, kv_format, kv_scale):
    """Stored latent rows -> fp64.  bf16 bit patterns, or E4M3FN codes times
    the per-tensor fp32 scale."""
    if kv_format == "bf16":
        assert float(kv_scale) == 1.0
        return bf16_bits_to_f64(raw_rows)
    if kv_format == "fp8_e4m3fn":
        return e4m3fn_codes_to_f64(raw_rows) * float(np.float32(kv_scale))
    raise ValueError(f"unknown kv_format {kv_format!r}")


def decode_paged(q_bits, pool, kv_format, kv_scale, block_table, seq_lens, page_size,
                 softmax_scale, causal=True, requests=None, heads=None):
    """``decode`` on the stored (bit-level) inputs the GPU library reads.

    q_bits: uint16 bf16 patterns [B][T][H][576].  pool: uint16 (bf16) or uint8
    (E4M3FN) [num_pages][page_size][576].  block_table: int [B][max_pages].
    ``requests`` / ``heads`` select a subset of outputs (the others are not
    computed); results are indexed [len(requests)][T][len(heads)].
    """
    q = bf16_bits_to_f64(q_bits)
    requests = range(q.shape[0]) if requests is None else list(requests)
    lat = []
    for r in requests:
        raw = gather_latents(pool, block_table[r], int(seq_lens[r]), page_size)
        lat.append(decode_latent_rows(raw, kv_format, kv_scale))
    return decode(q[list(requests)], lat, softmax_scale, causal=causal, heads=heads)


def merge(o_parts, lse_parts):
    """Merge partial answers that carry their log-sum-exp.

    o_parts: [P][...][512], lse_parts: [P][...].  For every row:
      M = max_p LSE_p
      a_p = exp(LSE_p - M)
      O = sum_p a_p * O_p / sum_p a_p,   LSE = M + ln sum_p a_p
    A row whose parts are all empty (every LSE_p = -inf) gives O = 0 and
    LSE = -inf.  Parts with LSE_p = -inf get weight 0.
    """
    o_parts = np.asarray(o_parts, dtype=np.float64)
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    m = lse_parts.max(axis=0)
    empty = np.isneginf(m)
    m_safe = np.where(empty, 0.0, m)
    a = np.exp(lse_parts - m_safe[None])  # exp(-inf) = 0 for empty parts
    denom = a.sum(axis=0)
    denom_safe = np.where(empty, 1.0, denom)
    o = (a[..., None] * o_parts).sum(axis=0) / denom_safe[..., None]
    o = np.where(empty[..., None], 0.0, o)
    lse = np.where(empty, -np.inf, m_safe + np.log(denom_safe))
    return o, lse
