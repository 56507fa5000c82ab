"""Thin ctypes binding of ``libmla_decode.so`` (the C ABI of include/mla_decode.h).

Argument marshalling only: every step of the decode runs in the library's HIP
kernels.  Torch tensors supply device memory and the current stream.  If the
library is missing this module raises; there is no fallback path.
"""

import ctypes
import os

import numpy as np

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmla_decode.so")

MLA_OK = 0
MLA_ERR_INVALID_ARGUMENT = 1
MLA_ERR_UNSUPPORTED = 2
MLA_ERR_WORKSPACE_TOO_SMALL = 3
MLA_ERR_DEVICE = 4

MLA_BF16 = 0
MLA_FP8_E4M3FN = 1
MLA_FP32 = 2

PAGE_SIZE = 64
D_LATENT = 576
D_V = 512

# Every symbol the header declares, with its ctypes signature.
_SIGNATURES = None


class MlaPagedKV(ctypes.Structure):
    _fields_ = [
        ("pool", ctypes.c_void_p),
        ("num_pages", ctypes.c_int64),
        ("page_size", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32),
        ("kv_scale", ctypes.c_float),
        ("block_table", ctypes.c_void_p),
        ("max_pages_per_seq", ctypes.c_int32),
        ("seq_lens", ctypes.c_void_p),
    ]


class MlaDecodeShape(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("q_len", ctypes.c_int32),
        ("num_heads", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
        ("causal", ctypes.c_int32),
        ("num_splits", ctypes.c_int32),
        ("partials_bf16", ctypes.c_int32),
    ]


def _signatures():
    c = ctypes
    P = c.c_void_p
    return {
        "mla_plan_create": (c.c_int, [c.POINTER(MlaDecodeShape), P, c.c_int32, c.c_int32, c.c_int32,
                                      c.POINTER(c.c_void_p), c.POINTER(c.c_size_t)]),
        "mla_plan_destroy": (None, [P]),
        "mla_plan_num_units": (c.c_int32, [P]),
        "mla_plan_num_parts": (c.c_int32, [P]),
        "mla_plan_row_groups": (c.c_int32, [P]),
        "mla_plan_set_fp8_qk": (c.c_int, [P, c.c_int32]),
        "mla_plan_set_hidden": (c.c_int, [P, P]),
        "mla_plan_get_work": (c.c_int32, [P, P, c.c_int32]),
        "mla_decode_splitkv": (c.c_int, [P, P, c.POINTER(MlaPagedKV), P, c.c_size_t, P, c.c_int32,
                                         P, P]),
        "mla_merge_lse": (c.c_int, [P, c.c_int32, P, c.c_int32, c.c_int64, P, c.c_int32, P, P]),
        "mla_kv_append": (c.c_int, [P, c.c_int64, c.c_int32, c.c_int32, c.c_float, P, c.c_int32, P, P,
                                    c.c_int32, c.c_int32, P]),
        "mla_block_table_check": (c.c_int, [P, c.c_int32, c.c_int32, P, c.c_int32, c.c_int64]),
        "mla_page_bytes": (c.c_size_t, [c.c_int32, c.c_int32]),
        "mla_status_str": (c.c_char_p, [c.c_int]),
        "mla_last_error": (c.c_char_p, []),
        "mla_version": (c.c_char_p, []),
    }


_lib = None


def load(build_if_missing=True):
    """Load the library (building it first only if nothing is built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        if not build_if_missing:
            raise RuntimeError(f"{LIB_PATH} is not built")
        from . import build

        build.build()
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in _signatures().items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def exported_symbols():
    return list(_signatures())


class MlaError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"{status_str(status)}: {msg}")
        self.status = status


def status_str(status):
    return load().mla_status_str(status).decode()


def _check(status):
    if status != MLA_OK:
        raise MlaError(status, load().mla_last_error().decode())


def _ptr(x):
    """Device or host address of a tensor / numpy array; None -> NULL."""
    if x is None:
        return None
    if isinstance(x, np.ndarray):
        return x.ctypes.data
    return x.data_ptr()


def _stream(stream):
    if stream is not None:
        return ctypes.c_void_p(stream)
    import torch

    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


class Plan:
    """A decode plan (host object): partition of the histories into workgroup pieces."""

    def __init__(self, batch, q_len, num_heads, seq_lens_host, softmax_scale, causal=True,
                 num_splits=0, kv_dtype=MLA_BF16, num_cus=0, page_size=PAGE_SIZE,
                 partials_bf16=False, fp8_qk=False):
        lib = load()
        self.shape = MlaDecodeShape(int(batch), int(q_len), int(num_heads), float(softmax_scale),
                                    int(bool(causal)), int(num_splits), int(bool(partials_bf16)))
        sl = np.ascontiguousarray(np.asarray(seq_lens_host, dtype=np.int32))
        assert sl.shape == (batch,)
        h = ctypes.c_void_p()
        ws = ctypes.c_size_t()
        _check(lib.mla_plan_create(ctypes.byref(self.shape), sl.ctypes.data, int(page_size),
                                   int(kv_dtype), int(num_cus), ctypes.byref(h), ctypes.byref(ws)))
        self._h = h
        self.workspace_bytes = ws.value
        self.kv_dtype = kv_dtype
        self.batch, self.q_len, self.num_heads = int(batch), int(q_len), int(num_heads)
        if fp8_qk:
            self.set_fp8_qk(True)

    @property
    def handle(self):
        return self._h

    @property
    def num_units(self):
        return load().mla_plan_num_units(self._h)

    @property
    def num_parts(self):
        return load().mla_plan_num_parts(self._h)

    @property
    def row_groups(self):
        return load().mla_plan_row_groups(self._h)

    def set_hidden(self, hidden):
        """Per-(request, token) hidden tails: int32 device tensor [batch][q_len] or None.
        The tensor must stay alive while the plan is used."""
        if hidden is not None:
            import torch

            if (tuple(hidden.shape) != (self.batch, self.q_len) or hidden.dtype != torch.int32
                    or not hidden.is_cuda or not hidden.is_contiguous()):
                raise ValueError("hidden must be a contiguous int32 device tensor "
                                 f"[{self.batch}][{self.q_len}]")
        self._hidden = hidden  # keep it alive with the plan
        _check(load().mla_plan_set_hidden(self._h, _ptr(hidden)))

    def set_fp8_qk(self, enable):
        """q.k on the FP8 matrix cores (FP8 pool, two or more 16-row blocks)."""
        _check(load().mla_plan_set_fp8_qk(self._h, int(bool(enable))))

    def work(self):
        """Work list as int32 [n][5]: (workgroup, request, first page, end page, slot)."""
        lib = load()
        n = lib.mla_plan_get_work(self._h, None, 0)
        out = np.zeros((max(n, 1), 5), dtype=np.int32)
        m = lib.mla_plan_get_work(self._h, out.ctypes.data, n)
        assert m == n
        return out[:n]

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and _lib is not None:
            _lib.mla_plan_destroy(h)
            self._h = None


def paged_kv(pool, block_table, seq_lens, kv_dtype, kv_scale=1.0, page_size=PAGE_SIZE):
    """Descriptor of a paged pool held in device tensors."""
    return MlaPagedKV(_ptr(pool), int(pool.shape[0]), int(page_size), int(kv_dtype),
                      float(kv_scale), _ptr(block_table), int(block_table.shape[1]),
                      _ptr(seq_lens))


def workspace(plan, device="cuda"):
    """A device workspace for `plan` (no initialisation needed)."""
    import torch

    return torch.empty(max(plan.workspace_bytes, 256), dtype=torch.uint8, device=device)


def decode_splitkv(plan, q, kv, ws, out=None, out_dtype=MLA_BF16, out_lse=None, stream=None):
    """mla_decode_splitkv on torch tensors (q bf16 [B][T][H][576], out [B][T][H][512])."""
    lib = load()
    _check(lib.mla_decode_splitkv(plan.handle, _ptr(q), ctypes.byref(kv), _ptr(ws),
                                  ws.numel() * ws.element_size(), _ptr(out), int(out_dtype),
                                  _ptr(out_lse), _stream(stream)))


def kv_append(pool, block_table, seq_lens, latents, kv_dtype, kv_scale=1.0, stream=None,
              page_size=PAGE_SIZE):
    """mla_kv_append on torch tensors: pool [num_pages][page_size][576] (written in place),
    latents bf16 [batch][q_len][576]."""
    lib = load()
    batch, q_len = int(latents.shape[0]), int(latents.shape[1])
    _check(lib.mla_kv_append(_ptr(pool), int(pool.shape[0]), int(page_size), int(kv_dtype),
                             float(kv_scale), _ptr(block_table), int(block_table.shape[1]),
                             _ptr(seq_lens), _ptr(latents), batch, q_len, _stream(stream)))


def merge_lse(part_o, part_lse, out=None, out_lse=None, stream=None):
    """mla_merge_lse: part_o [P][rows][512] (bf16 or fp32), part_lse fp32 [P][rows]."""
    import torch

    lib = load()
    pd = MLA_BF16 if part_o.dtype == torch.bfloat16 else MLA_FP32
    od = MLA_BF16 if (out is not None and out.dtype == torch.bfloat16) else MLA_FP32
    n_parts, rows = int(part_o.shape[0]), int(part_o.numel() // (part_o.shape[0] * D_V))
    _check(lib.mla_merge_lse(_ptr(part_o), pd, _ptr(part_lse), n_parts, rows, _ptr(out), od,
                             _ptr(out_lse), _stream(stream)))


def block_table_check(block_table, seq_lens, page_size, num_pages):
    bt = np.ascontiguousarray(np.asarray(block_table, dtype=np.int32))
    sl = np.ascontiguousarray(np.asarray(seq_lens, dtype=np.int32))
    st = load().mla_block_table_check(bt.ctypes.data, bt.shape[0], bt.shape[1], sl.ctypes.data,
                                      int(page_size), int(num_pages))
    return st


def version():
    return load().mla_version().decode()
