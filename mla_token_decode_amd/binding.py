"""Thin ctypes binding of libmla_decode.so (include/mla_decode.h).

Argument marshalling only: every step of the decode runs in the library's HIP
kernels.  Torch tensors are accepted for device buffers (their data pointers
are passed through) and the current torch stream is used by default.  A
missing library raises; nothing falls back to another implementation.
"""
from __future__ import annotations

import ctypes
import os
import threading

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmla_decode.so")

MLA_OK = 0
MLA_ERR_INVALID_ARGUMENT = 1
MLA_ERR_UNSUPPORTED = 2
MLA_ERR_WORKSPACE_TOO_SMALL = 3
MLA_ERR_DEVICE = 4
MLA_ERR_OUT_OF_MEMORY = 5
MLA_KV_BF16 = 0
MLA_KV_FP8_E4M3 = 1
MLA_PLAN_AUTO = 0
MLA_PLAN_UNIFORM = 1
MLA_MERGE_AUTO = 0
MLA_MERGE_REDUCE = 1
MLA_MERGE_LAST_ARRIVER = 2
MLA_MERGE_GRID = 3
DQK = 576
DV = 512
KV_GRANULE = 64

MAX_SHARDS = 1024

EXPORTED = ["mla_decode_plan", "mla_decode_plan_shard", "mla_decode_run", "mla_decode_run_paged",
            "mla_decode_reduce", "mla_merge_shards", "mla_plan_destroy", "mla_last_error",
            "mla_plan_query", "mla_plan_info", "mla_decode_run_static", "mla_plan_order",
            "mla_plan_launch_info"]
STATIC_WORKSPACE_BYTES = 32 << 20

_lock = threading.Lock()
_lib = None


class MlaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"mla status {status}: {message}")
        self.status = status
        self.message = message


class _Options(ctypes.Structure):
    _fields_ = [("force_fold", ctypes.c_int32), ("force_splits", ctypes.c_int32),
                ("num_cus", ctypes.c_int32), ("plan_mode", ctypes.c_int32),
                ("merge_mode", ctypes.c_int32)]


def lib() -> ctypes.CDLL:
    """Load the in-tree library (raises FileNotFoundError if it was not built)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise FileNotFoundError(
                f"{LIB_PATH} is missing: build it with `python -m mla_token_decode_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        i32p = ctypes.POINTER(ctypes.c_int32)
        L.mla_decode_plan.argtypes = [ctypes.c_int32, ctypes.c_int32, i32p, i32p, ctypes.c_int,
                                      ctypes.POINTER(_Options), ctypes.POINTER(ctypes.c_void_p),
                                      ctypes.POINTER(ctypes.c_size_t)]
        L.mla_decode_plan.restype = ctypes.c_int
        L.mla_decode_plan_shard.argtypes = [ctypes.c_int32, ctypes.c_int32, i32p, i32p, i32p,
                                            ctypes.c_int, ctypes.POINTER(_Options),
                                            ctypes.POINTER(ctypes.c_void_p),
                                            ctypes.POINTER(ctypes.c_size_t)]
        L.mla_decode_plan_shard.restype = ctypes.c_int
        L.mla_merge_shards.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                       ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                       ctypes.c_void_p]
        L.mla_merge_shards.restype = ctypes.c_int
        L.mla_decode_run.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_float,
                                     ctypes.c_float, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                     ctypes.c_size_t, ctypes.c_void_p]
        L.mla_decode_run.restype = ctypes.c_int
        L.mla_decode_run_paged.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                           ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                           ctypes.c_int32, ctypes.c_float, ctypes.c_float,
                                           ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                           ctypes.c_size_t, ctypes.c_void_p]
        L.mla_decode_run_paged.restype = ctypes.c_int
        L.mla_decode_reduce.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                        ctypes.c_void_p, ctypes.c_void_p]
        L.mla_decode_reduce.restype = ctypes.c_int
        L.mla_decode_run_static.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                            ctypes.c_float, ctypes.c_float, ctypes.c_void_p,
                                            ctypes.c_void_p, ctypes.c_void_p]
        L.mla_decode_run_static.restype = ctypes.c_int
        L.mla_plan_destroy.argtypes = [ctypes.c_void_p]
        L.mla_plan_destroy.restype = None
        L.mla_last_error.argtypes = []
        L.mla_last_error.restype = ctypes.c_char_p
        L.mla_plan_order.argtypes = [ctypes.c_void_p, i32p]
        L.mla_plan_order.restype = ctypes.c_int
        L.mla_plan_query.argtypes = [ctypes.c_void_p, ctypes.c_int32, i32p, i32p, i32p, i32p]
        L.mla_plan_query.restype = ctypes.c_int
        L.mla_plan_info.argtypes = [ctypes.c_void_p, i32p, i32p, i32p, ctypes.POINTER(ctypes.c_size_t)]
        L.mla_plan_info.restype = ctypes.c_int
        L.mla_plan_launch_info.argtypes = [ctypes.c_void_p, ctypes.c_int32, i32p, i32p]
        L.mla_plan_launch_info.restype = ctypes.c_int
        _lib = L
        return L


def _check(status: int):
    if status != MLA_OK:
        msg = lib().mla_last_error()
        raise MlaError(status, msg.decode() if msg else "")


def _ptr(x):
    """Device pointer of a torch tensor (or an int / None passed through)."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


class Plan:
    """Owns an mla_plan (host memory); free with close() or by garbage collection."""

    def __init__(self, num_heads, q_len, kv_len, kv_fp8=False, *, causal_end=None, force_fold=0,
                 force_splits=0, num_cus=0, plan_mode=0, merge_mode=0):
        """causal_end: None (mla_decode_plan), or per-sequence causal ends of a
        key shard (mla_decode_plan_shard).  plan_mode: MLA_PLAN_AUTO (0) or
        MLA_PLAN_UNIFORM (1).  merge_mode: MLA_MERGE_AUTO (0), MLA_MERGE_REDUCE
        (1), MLA_MERGE_LAST_ARRIVER (2) or MLA_MERGE_GRID (3)."""
        L = lib()
        q_len = [int(v) for v in q_len]
        kv_len = [int(v) for v in kv_len]
        n = len(q_len)
        if len(kv_len) != n:
            raise ValueError("q_len and kv_len must have the same length")
        qa = (ctypes.c_int32 * max(n, 1))(*q_len)
        ka = (ctypes.c_int32 * max(n, 1))(*kv_len)
        opts = _Options(int(force_fold), int(force_splits), int(num_cus), int(plan_mode),
                        int(merge_mode))
        handle = ctypes.c_void_p()
        ws = ctypes.c_size_t(0)
        self._h = None
        self._lib = L  # the library that owns the handle also frees it
        dtype = MLA_KV_FP8_E4M3 if kv_fp8 else MLA_KV_BF16
        if causal_end is None:
            _check(L.mla_decode_plan(n, int(num_heads), qa, ka, dtype, ctypes.byref(opts),
                                     ctypes.byref(handle), ctypes.byref(ws)))
        else:
            causal_end = [int(v) for v in causal_end]
            if len(causal_end) != n:
                raise ValueError("causal_end must have one entry per sequence")
            ca = (ctypes.c_int32 * max(n, 1))(*causal_end)
            _check(L.mla_decode_plan_shard(n, int(num_heads), qa, ka, ca, dtype,
                                           ctypes.byref(opts), ctypes.byref(handle),
                                           ctypes.byref(ws)))
        self.causal_end = causal_end
        self._h = handle
        self.num_heads = int(num_heads)
        self.q_len = q_len
        self.kv_len = kv_len
        self.kv_fp8 = bool(kv_fp8)
        self.workspace_bytes = int(ws.value)
        nu, ns, nl = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
        _check(L.mla_plan_info(self._h, ctypes.byref(nu), ctypes.byref(ns), ctypes.byref(nl), None))
        self.num_units, self.num_split_tiles, self.num_launches = nu.value, ns.value, nl.value

    @property
    def handle(self):
        if self._h is None:
            raise ValueError("plan is closed")
        return self._h

    def launch(self, i: int):
        """(work units, merge mode) of main-kernel launch i; the merge mode is
        MLA_MERGE_REDUCE, _LAST_ARRIVER or _GRID, 0 when it has no split rows."""
        nu, mm = ctypes.c_int32(), ctypes.c_int32()
        _check(lib().mla_plan_launch_info(self.handle, int(i), ctypes.byref(nu), ctypes.byref(mm)))
        return nu.value, mm.value

    def order(self):
        """Caller indices of the sequences in the order their units run."""
        out = (ctypes.c_int32 * len(self.q_len))()
        _check(lib().mla_plan_order(self.handle, out))
        return list(out)

    def query(self, seq: int):
        """(fold F, tiles T, splits S_eff, chunk length L) of one sequence."""
        f, t, s, c = (ctypes.c_int32() for _ in range(4))
        _check(lib().mla_plan_query(self.handle, int(seq), ctypes.byref(f), ctypes.byref(t),
                                    ctypes.byref(s), ctypes.byref(c)))
        return f.value, t.value, s.value, c.value

    def close(self):
        if self._h is not None:
            self._lib.mla_plan_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def mla_decode_plan(num_heads, q_len, kv_len, kv_fp8=False, **opts) -> Plan:
    return Plan(num_heads, q_len, kv_len, kv_fp8, **opts)


def _check_tensor(t, name, dtypes, min_numel):
    """Validate a device buffer passed as a torch tensor before its pointer
    reaches the library: the kernels address buffers from the plan's sizes, so
    a short, strided, host or wrongly typed tensor would be read or written out
    of bounds on the device.  Raw integer pointers are passed through as they
    are (the caller vouches for them)."""
    if t is None or isinstance(t, int):
        return
    if not getattr(t, "is_cuda", False):
        raise ValueError(f"{name} must be a device (cuda) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if str(t.dtype).replace("torch.", "") not in dtypes:
        raise ValueError(f"{name} has dtype {t.dtype}; expected one of {dtypes}")
    if t.numel() < min_numel:
        raise ValueError(f"{name} holds {t.numel()} elements; the plan needs at least {min_numel}")


def _check_run_args(plan: Plan, q, kv, o, lse, workspace, workspace_bytes, kv_rows):
    rows = sum(plan.q_len) * plan.num_heads
    _check_tensor(q, "q", ("bfloat16",), rows * DQK)
    if q is not None and not isinstance(q, int) and q.numel() != rows * DQK:
        raise ValueError(f"q must hold sum(q_len) * H * 576 = {rows * DQK} elements")
    _check_tensor(kv, "kv", ("uint8", "float8_e4m3fn") if plan.kv_fp8 else ("bfloat16",),
                  kv_rows * DQK)
    _check_tensor(o, "o", ("bfloat16",), rows * DV)
    _check_tensor(lse, "lse", ("float32",), rows)
    if workspace is not None and not isinstance(workspace, int):
        _check_tensor(workspace, "workspace", ("uint8", "int8", "float32", "bfloat16", "int32"), 0)
        if workspace.numel() * workspace.element_size() < int(workspace_bytes):
            raise ValueError("workspace_bytes exceeds the workspace tensor")


def _workspace_bytes(workspace, workspace_bytes):
    if workspace_bytes is not None:
        return int(workspace_bytes)
    if workspace is None or isinstance(workspace, int):
        return 0
    return workspace.numel() * workspace.element_size()


def mla_decode_run(plan: Plan, q, kv, sm_scale: float, kv_scale: float, o, lse, workspace=None,
                   workspace_bytes=None, stream=None):
    workspace_bytes = _workspace_bytes(workspace, workspace_bytes)
    _check_run_args(plan, q, kv, o, lse, workspace, workspace_bytes, sum(plan.kv_len))
    _check(lib().mla_decode_run(plan.handle, _ptr(q), _ptr(kv), float(sm_scale), float(kv_scale),
                                _ptr(o), _ptr(lse), _ptr(workspace), int(workspace_bytes),
                                _stream(stream)))


def mla_decode_run_paged(plan: Plan, q, kv_pages, page_table, sm_scale: float, kv_scale: float, o,
                         lse, workspace=None, workspace_bytes=None, stream=None):
    """kv_pages: [num_pages, page_size, 576] pool (bf16, or uint8 e4m3 codes);
    page_table: int32 [batch, stride] page indices (key j of sequence b is row
    j % page_size of page page_table[b, j // page_size])."""
    if kv_pages.dim() != 3 or int(kv_pages.shape[2]) != DQK:
        raise ValueError("kv_pages must be [num_pages, page_size, 576]")
    if page_table.dim() != 2 or not page_table.is_contiguous() or str(page_table.dtype) != "torch.int32":
        raise ValueError("page_table must be a contiguous [batch, stride] int32 tensor")
    if int(page_table.shape[0]) < len(plan.q_len):
        raise ValueError("page_table needs one row per sequence of the plan")
    if not page_table.is_cuda:
        raise ValueError("page_table must be a device (cuda) tensor")
    workspace_bytes = _workspace_bytes(workspace, workspace_bytes)
    _check_run_args(plan, q, kv_pages, o, lse, workspace, workspace_bytes,
                    int(kv_pages.shape[0]) * int(kv_pages.shape[1]))
    _check(lib().mla_decode_run_paged(plan.handle, _ptr(q), _ptr(kv_pages), int(kv_pages.shape[0]),
                                      int(kv_pages.shape[1]), _ptr(page_table),
                                      int(page_table.shape[1]), float(sm_scale), float(kv_scale),
                                      _ptr(o), _ptr(lse), _ptr(workspace), int(workspace_bytes),
                                      _stream(stream)))


def mla_decode_run_static(plan: Plan, q, kv, sm_scale: float, kv_scale: float, o, lse,
                          stream=None):
    """Run + merge with the library's per-device static workspace (no
    allocation; calls that overlap on one device race)."""
    _check_run_args(plan, q, kv, o, lse, None, 0, sum(plan.kv_len))
    _check(lib().mla_decode_run_static(plan.handle, _ptr(q), _ptr(kv), float(sm_scale),
                                       float(kv_scale), _ptr(o), _ptr(lse), _stream(stream)))


def mla_decode_reduce(plan: Plan, workspace, o, lse, stream=None):
    rows = sum(plan.q_len) * plan.num_heads
    _check_tensor(o, "o", ("bfloat16",), rows * DV)
    _check_tensor(lse, "lse", ("float32",), rows)
    if workspace is not None and not isinstance(workspace, int):
        _check_tensor(workspace, "workspace", ("uint8", "int8", "float32", "bfloat16", "int32"), 0)
        if workspace.numel() * workspace.element_size() < plan.workspace_bytes:
            raise ValueError(f"workspace is smaller than the planned {plan.workspace_bytes} bytes")
    _check(lib().mla_decode_reduce(plan.handle, _ptr(workspace), _ptr(o), _ptr(lse),
                                   _stream(stream)))


def mla_merge_shards(o_shards, lse_shards, o, lse, stream=None):
    """Combine per-shard results: o_shards bf16 [W, rows, 512] (or [W, ..., 512]),
    lse_shards fp32 [W, rows] (matching), into o bf16 [rows, 512], lse [rows]."""
    num_shards = int(o_shards.shape[0])
    num_rows = int(lse_shards[0].numel())
    if int(lse_shards.shape[0]) != num_shards or int(o_shards[0].numel()) != num_rows * DV:
        raise ValueError("o_shards must be [W, rows, 512] and lse_shards [W, rows]")
    if int(o.numel()) != num_rows * DV or int(lse.numel()) != num_rows:
        raise ValueError("o must hold rows x 512 values and lse rows values")
    _check_tensor(o_shards, "o_shards", ("bfloat16",), num_shards * num_rows * DV)
    _check_tensor(lse_shards, "lse_shards", ("float32",), num_shards * num_rows)
    _check_tensor(o, "o", ("bfloat16",), num_rows * DV)
    _check_tensor(lse, "lse", ("float32",), num_rows)
    _check(lib().mla_merge_shards(num_rows, num_shards, _ptr(o_shards), _ptr(lse_shards), _ptr(o),
                                  _ptr(lse), _stream(stream)))


def alloc_outputs(plan: Plan, device="cuda"):
    """O (bf16 [sum q, H, 512]), LSE (fp32 [sum q, H]) and the workspace, via torch."""
    import torch
    sq = sum(plan.q_len)
    o = torch.empty((sq, plan.num_heads, DV), dtype=torch.bfloat16, device=device)
    lse = torch.empty((sq, plan.num_heads), dtype=torch.float32, device=device)
    ws = torch.empty((max(plan.workspace_bytes, 16),), dtype=torch.uint8, device=device)
    return o, lse, ws


def decode(plan: Plan, q, kv, sm_scale: float, kv_scale: float = 1.0, out=None, stream=None):
    """Run + reduce on the given (or freshly allocated) outputs; returns (O, LSE)."""
    o, lse, ws = out if out is not None else alloc_outputs(plan, q.device)
    mla_decode_run(plan, q, kv, sm_scale, kv_scale, o, lse, ws, ws.numel(), stream)
    mla_decode_reduce(plan, ws, o, lse, stream)
    return o, lse
