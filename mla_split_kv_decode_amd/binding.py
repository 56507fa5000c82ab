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
        "mla_plan_get_work": (c.c_int32, [P, P, c.c_int32]),
        "mla_decode_splitkv": (c.c_int, [P, P, c.POINTER(MlaPagedKV), P, c.c_size_t, P, c.c_int32,
                                         P, P, P]),
        "mla_decode_splitkv_noalloc": (c.c_int, [P, P, c.POINTER(MlaPagedKV), P, c.c_int32, P, P, P]),
        "mla_merge_lse": (c.c_int, [P, c.c_int32, P, c.c_int32, c.c_int64, P, c.c_int32, P, P]),
        "mla_kv_append": (c.c_int, [P, c.c_int64, c.c_int32, c.c_int32, c.c_float, P, c.c_int32, P, P,
                                    c.c_int32, c.c_int32, P]),
        "mla_read_reference": (c.c_int, [P, c.c_size_t, c.c_int32, P, P]),
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


def _host_ptr(x):
    """Address of a host numpy array."""
    return x.ctypes.data


def _on_gpu(x):
    return x.is_cuda


def _device_tensor(x, name, dtypes, shape=None, device=None):
    """Check that x is a contiguous CUDA tensor of one of `dtypes` (any dtype for None;
    and `shape`, and on `device`); return its device address.  Raises ValueError otherwise, before anything
    reaches the library (which would take any address as a device pointer)."""
    import torch

    if not isinstance(x, torch.Tensor):
        raise ValueError(f"{name} must be a torch CUDA tensor, got {type(x).__name__}")
    if not _on_gpu(x):
        raise ValueError(f"{name} must be on a GPU (got device {x.device})")
    if device is not None and x.device != device:
        raise ValueError(f"{name} is on {x.device}, the other tensors on {device}")
    if dtypes is not None and x.dtype not in dtypes:
        raise ValueError(f"{name} has dtype {x.dtype}, expected one of {[str(d) for d in dtypes]}")
    if shape is not None and tuple(x.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(x.shape)}, expected {tuple(shape)}")
    if not x.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return x.data_ptr()


def _opt_device_tensor(x, name, dtypes, shape=None, device=None):
    return None if x is None else _device_tensor(x, name, dtypes, shape, device)


def _stream(stream):
    if stream is not None:
        return ctypes.c_void_p(stream)
    import torch

    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _pool_dtypes(kv_dtype):
    import torch

    if kv_dtype == MLA_BF16:
        return (torch.bfloat16,)
    if kv_dtype == MLA_FP8_E4M3FN:
        return (torch.uint8, torch.float8_e4m3fn)
    raise ValueError(f"kv_dtype {kv_dtype} is not MLA_BF16 or MLA_FP8_E4M3FN")


def _check_pool_and_table(pool, block_table, seq_lens, kv_dtype, page_size):
    """Checks shared by the paged-KV descriptor and the cache append; returns the device."""
    import torch

    _device_tensor(pool, "pool", _pool_dtypes(kv_dtype))
    dev = pool.device
    if pool.dim() != 3 or pool.shape[1] != page_size or pool.shape[2] != D_LATENT or pool.shape[0] < 1:
        raise ValueError(f"pool must be [num_pages][{page_size}][{D_LATENT}], got {tuple(pool.shape)}")
    _device_tensor(block_table, "block_table", (torch.int32,), device=dev)
    if block_table.dim() != 2 or block_table.shape[1] < 1:
        raise ValueError(f"block_table must be [batch][max_pages_per_seq], got {tuple(block_table.shape)}")
    _device_tensor(seq_lens, "seq_lens", (torch.int32,), shape=(block_table.shape[0],), device=dev)
    return dev


class Plan:
    """A decode plan (host object): partition of the histories into workgroup pieces."""

    def __init__(self, batch, q_len, num_heads, seq_lens_host, softmax_scale, causal=True,
                 num_splits=0, kv_dtype=MLA_BF16, num_cus=0, page_size=PAGE_SIZE, fp8_qk=False):
        lib = load()
        self.shape = MlaDecodeShape(int(batch), int(q_len), int(num_heads), float(softmax_scale),
                                    int(bool(causal)), int(num_splits))
        sl = np.ascontiguousarray(np.asarray(seq_lens_host, dtype=np.int32))
        if sl.shape != (int(batch),):
            raise ValueError(f"seq_lens_host must have shape ({batch},), got {sl.shape}")
        h = ctypes.c_void_p()
        ws = ctypes.c_size_t()
        _check(lib.mla_plan_create(ctypes.byref(self.shape), _host_ptr(sl), int(page_size),
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

    def set_fp8_qk(self, enable):
        """q.k on the FP8 matrix cores (FP8 pool, two or more 16-row blocks)."""
        _check(load().mla_plan_set_fp8_qk(self._h, int(bool(enable))))

    def work(self):
        """Work list as int32 [n][5]: (workgroup, request, first page, end page, slot)."""
        lib = load()
        n = lib.mla_plan_get_work(self._h, None, 0)
        out = np.zeros((max(n, 1), 5), dtype=np.int32)
        m = lib.mla_plan_get_work(self._h, _host_ptr(out), n)
        assert m == n
        return out[:n]

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and _lib is not None:
            _lib.mla_plan_destroy(h)
            self._h = None


def paged_kv(pool, block_table, seq_lens, kv_dtype, kv_scale=1.0, page_size=PAGE_SIZE):
    """Descriptor of a paged pool held in device tensors: pool [num_pages][64][576]
    (bf16 for MLA_BF16, uint8 or float8_e4m3fn for MLA_FP8_E4M3FN), block_table int32
    [batch][max_pages_per_seq], seq_lens int32 [batch], all contiguous on one GPU."""
    dev = _check_pool_and_table(pool, block_table, seq_lens, kv_dtype, page_size)
    kv = MlaPagedKV(pool.data_ptr(), int(pool.shape[0]), int(page_size), int(kv_dtype),
                    float(kv_scale), block_table.data_ptr(), int(block_table.shape[1]),
                    seq_lens.data_ptr())
    kv.device = dev
    kv.batch = int(block_table.shape[0])
    kv.tensors = (pool, block_table, seq_lens)  # kept alive with the descriptor
    return kv


def workspace(plan, device="cuda"):
    """A device workspace for `plan` (no initialisation needed)."""
    import torch

    return torch.empty(max(plan.workspace_bytes, 256), dtype=torch.uint8, device=device)


def _out_dtypes(out_dtype):
    import torch

    if out_dtype == MLA_BF16:
        return (torch.bfloat16,)
    if out_dtype == MLA_FP32:
        return (torch.float32,)
    raise ValueError(f"out_dtype {out_dtype} is not MLA_BF16 or MLA_FP32")


def decode_splitkv(plan, q, kv, ws, out=None, out_dtype=MLA_BF16, out_lse=None, hidden=None,
                   stream=None):
    """mla_decode_splitkv on torch tensors: q bf16 [B][T][H][576], out [B][T][H][512] of
    out_dtype, out_lse fp32 [B][T][H], hidden int32 [B][T] (or None), ws uint8 of at
    least plan.workspace_bytes; kv from paged_kv with B requests; all on one GPU."""
    import torch

    if not isinstance(kv, MlaPagedKV) or not hasattr(kv, "device"):
        raise ValueError("kv must come from paged_kv()")
    dev = kv.device
    B, T, H = plan.batch, plan.q_len, plan.num_heads
    if kv.batch != B:
        raise ValueError(f"the KV descriptor has {kv.batch} requests, the plan {B}")
    if kv.kv_dtype != plan.kv_dtype:
        raise ValueError(f"kv_dtype {kv.kv_dtype} differs from the plan's {plan.kv_dtype}")
    qp = _device_tensor(q, "q", (torch.bfloat16,), (B, T, H, D_LATENT), dev)
    wsp = _device_tensor(ws, "workspace", None, None, dev)
    ws_bytes = ws.numel() * ws.element_size()
    if ws_bytes < plan.workspace_bytes:
        raise ValueError(f"workspace of {ws_bytes} bytes < the plan's {plan.workspace_bytes}")
    op = _opt_device_tensor(out, "out", _out_dtypes(out_dtype), (B, T, H, D_V), dev)
    lp = _opt_device_tensor(out_lse, "out_lse", (torch.float32,), (B, T, H), dev)
    hp = _opt_device_tensor(hidden, "hidden", (torch.int32,), (B, T), dev)
    _check(load().mla_decode_splitkv(plan.handle, qp, ctypes.byref(kv), wsp, ws_bytes, op,
                                     int(out_dtype), lp, hp, _stream(stream)))


NOALLOC_SCRATCH_BYTES = 32 << 20


def decode_splitkv_noalloc(plan, q, kv, out=None, out_dtype=MLA_BF16, out_lse=None, hidden=None,
                           stream=None):
    """mla_decode_splitkv_noalloc: decode_splitkv with the library's per-GPU scratch in
    place of a workspace (nothing is allocated); same tensors and checks."""
    import torch

    if not isinstance(kv, MlaPagedKV) or not hasattr(kv, "device"):
        raise ValueError("kv must come from paged_kv()")
    dev = kv.device
    B, T, H = plan.batch, plan.q_len, plan.num_heads
    if kv.batch != B:
        raise ValueError(f"the KV descriptor has {kv.batch} requests, the plan {B}")
    qp = _device_tensor(q, "q", (torch.bfloat16,), (B, T, H, D_LATENT), dev)
    op = _opt_device_tensor(out, "out", _out_dtypes(out_dtype), (B, T, H, D_V), dev)
    lp = _opt_device_tensor(out_lse, "out_lse", (torch.float32,), (B, T, H), dev)
    hp = _opt_device_tensor(hidden, "hidden", (torch.int32,), (B, T), dev)
    _check(load().mla_decode_splitkv_noalloc(plan.handle, qp, ctypes.byref(kv), op, int(out_dtype),
                                             lp, hp, _stream(stream)))


def kv_append(pool, block_table, seq_lens, latents, kv_dtype, kv_scale=1.0, stream=None,
              page_size=PAGE_SIZE):
    """mla_kv_append on torch tensors: pool [num_pages][page_size][576] (written in place),
    latents bf16 [batch][q_len][576], block_table int32 [batch][max_pages], seq_lens int32
    [batch], all contiguous on one GPU."""
    import torch

    dev = _check_pool_and_table(pool, block_table, seq_lens, kv_dtype, page_size)
    _device_tensor(latents, "latents", (torch.bfloat16,), None, dev)
    if latents.dim() != 3 or latents.shape[0] != block_table.shape[0] or latents.shape[2] != D_LATENT:
        raise ValueError(f"latents must be [{block_table.shape[0]}][q_len][{D_LATENT}], "
                         f"got {tuple(latents.shape)}")
    batch, q_len = int(latents.shape[0]), int(latents.shape[1])
    _check(load().mla_kv_append(pool.data_ptr(), int(pool.shape[0]), int(page_size), int(kv_dtype),
                                float(kv_scale), block_table.data_ptr(), int(block_table.shape[1]),
                                seq_lens.data_ptr(), latents.data_ptr(), batch, q_len,
                                _stream(stream)))


def merge_lse(part_o, part_lse, out=None, out_lse=None, stream=None):
    """mla_merge_lse: part_o [P][rows][512] (bf16 or fp32; any shape [P][...][512]),
    part_lse fp32 [P][rows...], out [rows...][512] (bf16 or fp32), out_lse fp32 [rows...]."""
    import torch

    _device_tensor(part_o, "part_o", (torch.bfloat16, torch.float32))
    dev = part_o.device
    if part_o.dim() < 2 or part_o.shape[-1] != D_V or part_o.shape[0] < 1:
        raise ValueError(f"part_o must be [num_parts][...][{D_V}], got {tuple(part_o.shape)}")
    n_parts = int(part_o.shape[0])
    rows = int(part_o.numel() // (n_parts * D_V))
    lp = _device_tensor(part_lse, "part_lse", (torch.float32,), None, dev)
    if part_lse.numel() != n_parts * rows or part_lse.shape[0] != n_parts:
        raise ValueError(f"part_lse must hold [{n_parts}][{rows}] values, got {tuple(part_lse.shape)}")
    od = MLA_FP32
    op = None
    if out is not None:
        op = _device_tensor(out, "out", (torch.bfloat16, torch.float32), None, dev)
        if out.numel() != rows * D_V:
            raise ValueError(f"out must hold [{rows}][{D_V}] values, got {tuple(out.shape)}")
        od = MLA_BF16 if out.dtype == torch.bfloat16 else MLA_FP32
    olp = None
    if out_lse is not None:
        olp = _device_tensor(out_lse, "out_lse", (torch.float32,), None, dev)
        if out_lse.numel() != rows:
            raise ValueError(f"out_lse must hold {rows} values, got {tuple(out_lse.shape)}")
    pd = MLA_BF16 if part_o.dtype == torch.bfloat16 else MLA_FP32
    _check(load().mla_merge_lse(part_o.data_ptr(), pd, lp, n_parts, rows, op, od, olp,
                                _stream(stream)))


def read_reference(buf, mode, sink, stream=None):
    """mla_read_reference: read every byte of the device tensor `buf` once (mode 0: into
    registers, 1: into LDS as the partial stage copies pages, 2: an empty launch);
    sink is a device int32/uint32 tensor of at least one element."""
    import torch

    _device_tensor(buf, "buf", None)
    _device_tensor(sink, "sink", (torch.int32,), None, buf.device)
    _check(load().mla_read_reference(buf.data_ptr(), buf.numel() * buf.element_size(), int(mode),
                                     sink.data_ptr(), _stream(stream)))


def block_table_check(block_table, seq_lens, page_size, num_pages):
    """Host-side block-table check (numpy or lists); returns the status code."""
    bt = np.ascontiguousarray(np.asarray(block_table, dtype=np.int32))
    sl = np.ascontiguousarray(np.asarray(seq_lens, dtype=np.int32))
    if bt.ndim != 2 or sl.shape != (bt.shape[0],):
        raise ValueError("block_table must be [batch][max_pages] and seq_lens [batch]")
    return load().mla_block_table_check(_host_ptr(bt), bt.shape[0], bt.shape[1], _host_ptr(sl),
                                        int(page_size), int(num_pages))


def version():
    return load().mla_version().decode()
