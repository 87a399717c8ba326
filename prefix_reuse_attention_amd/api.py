"""Thin torch-tensor binding over libbat's C ABI (include/bat.h).

Argument marshalling only: tensors become device pointers, the current torch
stream becomes the hipStream_t, status codes become exceptions.  Every step of
the computation runs in the HIP kernels; there is no fallback, and a missing
library raises.
"""
import ctypes
import os
from dataclasses import dataclass

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libbat.so")

BAT_OK, BAT_ERR_INVALID_ARG, BAT_ERR_UNSUPPORTED, BAT_ERR_BLOCK_TABLE, BAT_ERR_WORKSPACE, \
    BAT_ERR_HIP = range(6)
BAT_F32, BAT_BF16 = 0, 1
BAT_PREFIX_USER, BAT_PREFIX_ITEM = 0, 1

EXPORTED = ("bat_kv_build", "bat_attn_workspace_size", "bat_attn_prefill_workspace_size",
            "bat_attn_prefill", "bat_attn_prefill_noalloc", "bat_attn_noalloc_scratch_bytes",
            "bat_kv_build_fp8", "bat_attn_fp8_workspace_size", "bat_attn_prefill_fp8",
            "bat_attn_prefix_rows", "bat_attn_item_local", "bat_attn_isolated_workspace_size",
            "bat_attn_prefill_isolated", "bat_attn_gqa_workspace_size", "bat_attn_prefill_gqa",
            "bat_lse_merge", "bat_sched_state_size", "bat_sched_init", "bat_sched_step",
            "bat_sched_pools",
            "bat_status_string", "bat_version", "bat_last_hip_error")
BAT_POLICY_USER_PREFIX, BAT_POLICY_HOTNESS = 0, 1

_lib = None


class BatError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        cause = f" [{load().bat_last_hip_error().decode()}]" if status == BAT_ERR_HIP else ""
        super().__init__(f"{where}: {status_string(status)} (status {status}){cause}")


class SchedConfig(ctypes.Structure):
    _fields_ = [("policy", ctypes.c_int32), ("item_tokens", ctypes.c_int32),
                ("user_block", ctypes.c_int32), ("item_capacity", ctypes.c_int32),
                ("user_capacity_blocks", ctypes.c_int64), ("num_users", ctypes.c_int32),
                ("num_items", ctypes.c_int32)]


class KvPool(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("num_blocks", ctypes.c_int32), ("block_size", ctypes.c_int32)]


class KvPoolFp8(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("k_scale", ctypes.c_void_p), ("v_scale", ctypes.c_void_p),
                ("num_blocks", ctypes.c_int32), ("block_size", ctypes.c_int32)]


def load():
    """Load libbat.so (built by prefix_reuse_attention_amd.build); raise if absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"libbat.so is not built ({LIB_PATH}); run "
                           "`python -m prefix_reuse_attention_amd.build`")
    # torch first: its HIP runtime (the one its tensors and streams belong
    # to) is then already loaded, and libbat binds to that same copy instead
    # of loading a second runtime of its own from the ROCm install
    import torch  # noqa: F401
    lib = ctypes.CDLL(LIB_PATH)
    P, I, F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float
    PP = ctypes.POINTER(KvPool)
    lib.bat_kv_build.argtypes = [P, P, P, P, I, I, I, I, I, I, PP, P]
    lib.bat_kv_build.restype = I
    lib.bat_attn_workspace_size.argtypes = [I, I, I, I, I, I, I]
    lib.bat_attn_workspace_size.restype = ctypes.c_size_t
    lib.bat_attn_prefill_workspace_size.argtypes = [I, I, I, I, I]
    lib.bat_attn_prefill_workspace_size.restype = ctypes.c_size_t
    lib.bat_attn_prefill.argtypes = [P, P, P, P, P, P, P, I, PP, PP, I, I, I, I, F, I, I, I,
                                     P, P, P, ctypes.c_size_t, P]
    lib.bat_attn_prefill.restype = I
    lib.bat_attn_prefill_noalloc.argtypes = [P, P, P, P, P, P, P, I, PP, PP, I, I, I, I, F, I, I,
                                             I, P, P, P]
    lib.bat_attn_prefill_noalloc.restype = I
    P8 = ctypes.POINTER(KvPoolFp8)
    lib.bat_kv_build_fp8.argtypes = [P, P, P, P, I, I, I, I, I, I, P8, P]
    lib.bat_kv_build_fp8.restype = I
    lib.bat_attn_fp8_workspace_size.argtypes = [I, I, I, I, I, I]
    lib.bat_attn_fp8_workspace_size.restype = ctypes.c_size_t
    lib.bat_attn_prefill_fp8.argtypes = [P, P, P, P, P, P, P, I, P8, P8, I, I, I, F, I, I, I,
                                         P, P, P, ctypes.c_size_t, P]
    lib.bat_attn_prefill_fp8.restype = I
    lib.bat_attn_noalloc_scratch_bytes.argtypes = []
    lib.bat_attn_noalloc_scratch_bytes.restype = ctypes.c_size_t
    lib.bat_attn_prefix_rows.argtypes = [P, P, P, P, I, I, I, I, F, I, I, P, P, P,
                                         ctypes.c_size_t, P]
    lib.bat_attn_prefix_rows.restype = I
    lib.bat_attn_item_local.argtypes = [P, P, P, I, I, I, I, I, F, P, P, P]
    lib.bat_attn_item_local.restype = I
    lib.bat_attn_isolated_workspace_size.argtypes = [I, I, I, I, I, I, I]
    lib.bat_attn_isolated_workspace_size.restype = ctypes.c_size_t
    lib.bat_attn_prefill_isolated.argtypes = [P, P, P, P, P, P, P, I, PP, PP, I, I, I, I, F, I, I,
                                              I, I, P, P, P, ctypes.c_size_t, P]
    lib.bat_attn_prefill_isolated.restype = I
    lib.bat_attn_gqa_workspace_size.argtypes = [I, I, I, I, I, I, I, I]
    lib.bat_attn_gqa_workspace_size.restype = ctypes.c_size_t
    lib.bat_attn_prefill_gqa.argtypes = [P, P, P, P, P, P, P, I, PP, PP, I, I, I, I, I, F, I,
                                         I, I, P, P, P, ctypes.c_size_t, P]
    lib.bat_attn_prefill_gqa.restype = I
    lib.bat_lse_merge.argtypes = [P, P, I, I, I, I, I, P, P, P]
    lib.bat_lse_merge.restype = I
    SP = ctypes.POINTER(SchedConfig)
    lib.bat_sched_state_size.argtypes = [SP]
    lib.bat_sched_state_size.restype = ctypes.c_size_t
    lib.bat_sched_init.argtypes = [SP, P, P, ctypes.c_size_t]
    lib.bat_sched_init.restype = I
    lib.bat_sched_step.argtypes = [P, I, I, P, P, P, P, P, P, P, P, P]
    lib.bat_sched_step.restype = I
    lib.bat_sched_pools.argtypes = [P, P, P, P]
    lib.bat_sched_pools.restype = I
    lib.bat_status_string.argtypes = [I]
    lib.bat_status_string.restype = ctypes.c_char_p
    lib.bat_version.argtypes = []
    lib.bat_version.restype = I
    lib.bat_last_hip_error.argtypes = []
    lib.bat_last_hip_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().bat_status_string(int(status)).decode()


def version() -> int:
    return load().bat_version()


def _check(status, where):
    if status != BAT_OK:
        raise BatError(status, where)


def _torch():
    import torch
    return torch


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def default_scale(D) -> float:
    """1/sqrt(D) rounded once to float32 (what the kernels receive)."""
    import math
    import numpy as np
    return float(np.float32(1.0 / math.sqrt(D)))


def _max_len(cu):
    """Longest request of a cumulative-length array: a copy to the host, then numpy."""
    import numpy as np
    c = cu.cpu().numpy()
    return int(np.diff(c).max()) if c.shape[0] > 1 else 0


def _max_val(x):
    import numpy as np
    a = x.cpu().numpy()
    return int(a.max()) if a.size else 0


def _stream():
    return ctypes.c_void_p(_torch().cuda.current_stream().cuda_stream)


def _dtype_code(t):
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return BAT_BF16
    if t.dtype == torch.float32:
        return BAT_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _need(t, name, dtype=None):
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous device tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")


@dataclass
class Pool:
    """A paged K/V pool: k and v are [num_blocks, H, block_size, D] device tensors."""
    k: object
    v: object
    block_size: int

    @property
    def num_blocks(self) -> int:
        return int(self.k.shape[0])

    def struct(self):
        return KvPool(self.k.data_ptr(), self.v.data_ptr(), self.num_blocks, self.block_size)


def new_pool(num_blocks, H, block_size, D, dtype, fill=None):
    torch = _torch()
    k = torch.empty((num_blocks, H, block_size, D), dtype=dtype, device="cuda")
    v = torch.empty_like(k)
    if fill is not None:
        k.fill_(fill)
        v.fill_(fill)
    return Pool(k, v, block_size)


@dataclass
class PoolFp8:
    """An fp8 K/V pool: k and v are uint8 [num_blocks, H, block_size, D] E4M3
    codes, k_scale and v_scale float32 [num_blocks, H] device tensors."""
    k: object
    v: object
    k_scale: object
    v_scale: object
    block_size: int

    @property
    def num_blocks(self) -> int:
        return int(self.k.shape[0])

    def struct(self):
        return KvPoolFp8(self.k.data_ptr(), self.v.data_ptr(), self.k_scale.data_ptr(),
                         self.v_scale.data_ptr(), self.num_blocks, self.block_size)


def new_pool_fp8(num_blocks, H, block_size, D):
    torch = _torch()
    k = torch.zeros((num_blocks, H, block_size, D), dtype=torch.uint8, device="cuda")
    return PoolFp8(k, torch.zeros_like(k),
                   torch.zeros((num_blocks, H), dtype=torch.float32, device="cuda"),
                   torch.zeros((num_blocks, H), dtype=torch.float32, device="cuda"), block_size)


def kv_build_fp8(k, v, cu_lens, block_table, pool: PoolFp8):
    """Quantise packed prefix K/V [tokens, H, D] into `pool` (E4M3 codes and
    one power-of-two scale per block and head) through block_table."""
    torch = _torch()
    _need(k, "k"); _need(v, "v", k.dtype)
    _need(cu_lens, "cu_lens", torch.int32); _need(block_table, "block_table", torch.int32)
    for t, n in ((pool.k, "pool.k"), (pool.v, "pool.v")):
        _need(t, n, torch.uint8)
    for t, n in ((pool.k_scale, "pool.k_scale"), (pool.v_scale, "pool.v_scale")):
        _need(t, n, torch.float32)
    total, H, D = k.shape
    B = cu_lens.shape[0] - 1
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be [B, stride]")
    ps = pool.struct()
    st = load().bat_kv_build_fp8(_ptr(k), _ptr(v), _ptr(cu_lens), _ptr(block_table),
                                 block_table.shape[1], B, H, D, total, _dtype_code(k),
                                 ctypes.byref(ps), _stream())
    _check(st, "bat_kv_build_fp8")


def fp8_workspace_size(B, H, D, total_suffix, max_suffix_len, max_prefix_len) -> int:
    return int(load().bat_attn_fp8_workspace_size(B, H, D, total_suffix, max_suffix_len,
                                                  max_prefix_len))


def attn_prefill_fp8(q, k, v, cu_suffix_lens, prefix_lens, prefix_mode, block_table,
                     user_pool=None, item_pool=None, softmax_scale=None, max_suffix_len=None,
                     max_prefix_len=None, out=None, lse=None, workspace=None, want_lse=False):
    """attn_prefill over fp8 pools (PoolFp8); q/k/v/out bfloat16."""
    torch = _torch()
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n, torch.bfloat16)
    _need(cu_suffix_lens, "cu_suffix_lens", torch.int32)
    _need(prefix_lens, "prefix_lens", torch.int32)
    _need(prefix_mode, "prefix_mode", torch.uint8)
    if block_table is not None:
        _need(block_table, "block_table", torch.int32)
    total, H, D = q.shape
    B = cu_suffix_lens.shape[0] - 1
    if max_suffix_len is None:
        max_suffix_len = _max_len(cu_suffix_lens)
    if max_prefix_len is None:
        max_prefix_len = _max_val(prefix_lens)
    if softmax_scale is None:
        softmax_scale = default_scale(D)
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", q.dtype)
    if lse is None and want_lse:
        lse = torch.empty((H, total), dtype=torch.float32, device=q.device)
    if lse is not None:
        _need(lse, "lse", torch.float32)
    if workspace is None:
        n = fp8_workspace_size(B, H, D, total, max_suffix_len, max_prefix_len)
        workspace = torch.empty(max(n, 1), dtype=torch.uint8, device=q.device)
    up = user_pool.struct() if user_pool is not None else None
    ip = item_pool.struct() if item_pool is not None else None
    st = load().bat_attn_prefill_fp8(
        _ptr(q), _ptr(k), _ptr(v), _ptr(cu_suffix_lens), _ptr(prefix_lens), _ptr(prefix_mode),
        _ptr(block_table), 0 if block_table is None else block_table.shape[1],
        ctypes.byref(up) if up is not None else None,
        ctypes.byref(ip) if ip is not None else None,
        B, H, D, float(softmax_scale), total, int(max_suffix_len), int(max_prefix_len),
        _ptr(out), _ptr(lse), _ptr(workspace), workspace.numel(), _stream())
    _check(st, "bat_attn_prefill_fp8")
    return out, lse


def kv_build(k, v, cu_lens, block_table, pool: Pool):
    """Scatter packed prefix K/V [tokens, H, D] into `pool` through block_table."""
    torch = _torch()
    _need(k, "k"); _need(v, "v", k.dtype)
    _need(cu_lens, "cu_lens", torch.int32); _need(block_table, "block_table", torch.int32)
    _need(pool.k, "pool.k", k.dtype); _need(pool.v, "pool.v", k.dtype)
    total, H, D = k.shape
    B = cu_lens.shape[0] - 1
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be [B, stride]")
    ps = pool.struct()
    st = load().bat_kv_build(_ptr(k), _ptr(v), _ptr(cu_lens), _ptr(block_table),
                             block_table.shape[1], B, H, D, total, _dtype_code(k),
                             ctypes.byref(ps), _stream())
    _check(st, "bat_kv_build")


def workspace_size(B, H, D, dtype_code, total_suffix, max_suffix_len, max_prefix_len) -> int:
    return int(load().bat_attn_workspace_size(B, H, D, dtype_code, total_suffix,
                                              max_suffix_len, max_prefix_len))


def prefill_workspace_size(B, H, D, total_suffix, max_prefix_len) -> int:
    """The bound over both dtypes and every suffix bound up to total_suffix."""
    return int(load().bat_attn_prefill_workspace_size(B, H, D, total_suffix, max_prefix_len))


def attn_prefill(q, k, v, cu_suffix_lens, prefix_lens, prefix_mode, block_table,
                 user_pool=None, item_pool=None, softmax_scale=None, max_suffix_len=None,
                 max_prefix_len=None, out=None, lse=None, workspace=None, want_lse=False):
    """Suffix-row prefill over the cached prefix and the suffix itself.

    q/k/v: packed [total_suffix, H, D] (bf16 or fp32).  Returns (out, lse);
    lse is [H, total_suffix] float32 or None.  max_*_len are host-side upper
    bounds over the batch (pass them to avoid a device-to-host read).
    """
    torch = _torch()
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n, q.dtype)
    _need(cu_suffix_lens, "cu_suffix_lens", torch.int32)
    _need(prefix_lens, "prefix_lens", torch.int32)
    _need(prefix_mode, "prefix_mode", torch.uint8)
    if block_table is not None:
        _need(block_table, "block_table", torch.int32)
    total, H, D = q.shape
    B = cu_suffix_lens.shape[0] - 1
    if max_suffix_len is None:
        max_suffix_len = _max_len(cu_suffix_lens)
    if max_prefix_len is None:
        max_prefix_len = _max_val(prefix_lens)
    if softmax_scale is None:
        softmax_scale = default_scale(D)
    dt = _dtype_code(q)
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", q.dtype)
    if lse is None and want_lse:
        lse = torch.empty((H, total), dtype=torch.float32, device=q.device)
    if lse is not None:
        _need(lse, "lse", torch.float32)
    ws_bytes = workspace_size(B, H, D, dt, total, max_suffix_len, max_prefix_len)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=q.device)
    up = user_pool.struct() if user_pool is not None else None
    ip = item_pool.struct() if item_pool is not None else None
    if up is not None:
        _need(user_pool.k, "user_pool.k", q.dtype)
    if ip is not None:
        _need(item_pool.k, "item_pool.k", q.dtype)
    st = load().bat_attn_prefill(
        _ptr(q), _ptr(k), _ptr(v), _ptr(cu_suffix_lens), _ptr(prefix_lens), _ptr(prefix_mode),
        _ptr(block_table), 0 if block_table is None else block_table.shape[1],
        ctypes.byref(up) if up is not None else None,
        ctypes.byref(ip) if ip is not None else None,
        B, H, D, dt, float(softmax_scale), total, int(max_suffix_len), int(max_prefix_len),
        _ptr(out), _ptr(lse), _ptr(workspace), workspace.numel(), _stream())
    _check(st, "bat_attn_prefill")
    return out, lse


class PreparedPrefill:
    """One bat_attn_prefill call with its arguments marshalled once: calling
    it enqueues the call on the current stream (no per-call tensor checks or
    workspace sizing).  The tensors must stay alive and unchanged in shape."""

    def __init__(self, q, k, v, cu_suffix_lens, prefix_lens, prefix_mode, block_table,
                 user_pool, item_pool, softmax_scale, max_suffix_len, max_prefix_len, out, lse,
                 workspace):
        torch = _torch()
        for t, n in ((q, "q"), (k, "k"), (v, "v"), (out, "out")):
            _need(t, n, q.dtype)
        _need(cu_suffix_lens, "cu_suffix_lens", torch.int32)
        _need(prefix_lens, "prefix_lens", torch.int32)
        _need(prefix_mode, "prefix_mode", torch.uint8)
        if block_table is not None:
            _need(block_table, "block_table", torch.int32)
        if lse is not None:
            _need(lse, "lse", torch.float32)
        total, H, D = q.shape
        B = cu_suffix_lens.shape[0] - 1
        dt = _dtype_code(q)
        need = workspace_size(B, H, D, dt, total, max_suffix_len, max_prefix_len)
        if workspace.numel() < need:
            raise BatError(BAT_ERR_WORKSPACE, "PreparedPrefill")
        self._keep = (q, k, v, cu_suffix_lens, prefix_lens, prefix_mode, block_table, out, lse,
                      workspace)
        self._up = user_pool.struct() if user_pool is not None else None
        self._ip = item_pool.struct() if item_pool is not None else None
        self._args = (
            _ptr(q), _ptr(k), _ptr(v), _ptr(cu_suffix_lens), _ptr(prefix_lens),
            _ptr(prefix_mode), _ptr(block_table),
            0 if block_table is None else block_table.shape[1],
            ctypes.byref(self._up) if self._up is not None else None,
            ctypes.byref(self._ip) if self._ip is not None else None,
            B, H, D, dt, float(softmax_scale), total, int(max_suffix_len), int(max_prefix_len),
            _ptr(out), _ptr(lse), _ptr(workspace), workspace.numel())
        self._fn = load().bat_attn_prefill

    def __call__(self):
        _check(self._fn(*self._args, _stream()), "bat_attn_prefill")


def attn_prefill_noalloc(q, k, v, cu_suffix_lens, prefix_lens, prefix_mode, block_table,
                         user_pool, item_pool, softmax_scale, max_suffix_len, max_prefix_len,
                         out, lse=None):
    """bat_attn_prefill_noalloc: attn_prefill with no workspace; the library
    works in its own device array.  Nothing is allocated here either: out
    (and lse, if wanted) are the caller's, and every bound is passed in."""
    torch = _torch()
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (out, "out")):
        _need(t, n, q.dtype)
    _need(cu_suffix_lens, "cu_suffix_lens", torch.int32)
    _need(prefix_lens, "prefix_lens", torch.int32)
    _need(prefix_mode, "prefix_mode", torch.uint8)
    if block_table is not None:
        _need(block_table, "block_table", torch.int32)
    if lse is not None:
        _need(lse, "lse", torch.float32)
    total, H, D = q.shape
    B = cu_suffix_lens.shape[0] - 1
    up = user_pool.struct() if user_pool is not None else None
    ip = item_pool.struct() if item_pool is not None else None
    st = load().bat_attn_prefill_noalloc(
        _ptr(q), _ptr(k), _ptr(v), _ptr(cu_suffix_lens), _ptr(prefix_lens), _ptr(prefix_mode),
        _ptr(block_table), 0 if block_table is None else block_table.shape[1],
        ctypes.byref(up) if up is not None else None,
        ctypes.byref(ip) if ip is not None else None,
        B, H, D, _dtype_code(q), float(softmax_scale), total, int(max_suffix_len),
        int(max_prefix_len), _ptr(out), _ptr(lse), _stream())
    _check(st, "bat_attn_prefill_noalloc")
    return out, lse


def noalloc_scratch_bytes() -> int:
    return int(load().bat_attn_noalloc_scratch_bytes())


def attn_prefix_rows(q, k, v, cu_prefix_lens, softmax_scale=None, max_prefix_len=None,
                     out=None, lse=None, workspace=None, want_lse=False):
    """Prefix rows over their own request's prefix (packed [total_prefix, H, D]).

    Returns (out, lse); lse is [H, total_prefix] float32 or None.
    """
    torch = _torch()
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n, q.dtype)
    _need(cu_prefix_lens, "cu_prefix_lens", torch.int32)
    total, H, D = q.shape
    B = cu_prefix_lens.shape[0] - 1
    if max_prefix_len is None:
        max_prefix_len = _max_len(cu_prefix_lens)
    if softmax_scale is None:
        softmax_scale = default_scale(D)
    dt = _dtype_code(q)
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", q.dtype)
    if lse is None and want_lse:
        lse = torch.empty((H, total), dtype=torch.float32, device=q.device)
    if lse is not None:
        _need(lse, "lse", torch.float32)
    ws_bytes = workspace_size(B, H, D, dt, total, max_prefix_len, 0)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=q.device)
    st = load().bat_attn_prefix_rows(
        _ptr(q), _ptr(k), _ptr(v), _ptr(cu_prefix_lens), B, H, D, dt, float(softmax_scale),
        total, int(max_prefix_len), _ptr(out), _ptr(lse), _ptr(workspace), workspace.numel(),
        _stream())
    _check(st, "bat_attn_prefix_rows")
    return out, lse


def attn_item_local(q, k, v, tokens_per_item, softmax_scale=None, out=None, lse=None,
                    want_lse=False):
    """Each item's tokens attend within the item (packed [n_items * T, H, D])."""
    torch = _torch()
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n, q.dtype)
    total, H, D = q.shape
    T = int(tokens_per_item)
    if T <= 0 or total % T:
        raise ValueError("rows must be a whole number of items")
    if softmax_scale is None:
        softmax_scale = default_scale(D)
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", q.dtype)
    if lse is None and want_lse:
        lse = torch.empty((H, total), dtype=torch.float32, device=q.device)
    if lse is not None:
        _need(lse, "lse", torch.float32)
    st = load().bat_attn_item_local(_ptr(q), _ptr(k), _ptr(v), total // T, T, H, D,
                                    _dtype_code(q), float(softmax_scale), _ptr(out), _ptr(lse),
                                    _stream())
    _check(st, "bat_attn_item_local")
    return out, lse


def attn_prefill_gqa(q, k, v, cu_suffix_lens, prefix_lens, prefix_mode, block_table,
                     user_pool=None, item_pool=None, softmax_scale=None, max_suffix_len=None,
                     max_prefix_len=None, out=None, lse=None, workspace=None, want_lse=False):
    """attn_prefill with grouped key/value heads: q is [total, H, D], k/v and
    the pools carry H_kv heads (H a multiple of H_kv)."""
    torch = _torch()
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n, q.dtype)
    _need(cu_suffix_lens, "cu_suffix_lens", torch.int32)
    _need(prefix_lens, "prefix_lens", torch.int32)
    _need(prefix_mode, "prefix_mode", torch.uint8)
    if block_table is not None:
        _need(block_table, "block_table", torch.int32)
    total, H, D = q.shape
    H_kv = k.shape[1]
    B = cu_suffix_lens.shape[0] - 1
    if max_suffix_len is None:
        max_suffix_len = _max_len(cu_suffix_lens)
    if max_prefix_len is None:
        max_prefix_len = _max_val(prefix_lens)
    if softmax_scale is None:
        softmax_scale = default_scale(D)
    dt = _dtype_code(q)
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", q.dtype)
    if lse is None and want_lse:
        lse = torch.empty((H, total), dtype=torch.float32, device=q.device)
    if lse is not None:
        _need(lse, "lse", torch.float32)
    ws_bytes = int(load().bat_attn_gqa_workspace_size(B, H, H_kv, D, dt, total, max_suffix_len,
                                                       max_prefix_len))
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=q.device)
    up = user_pool.struct() if user_pool is not None else None
    ip = item_pool.struct() if item_pool is not None else None
    st = load().bat_attn_prefill_gqa(
        _ptr(q), _ptr(k), _ptr(v), _ptr(cu_suffix_lens), _ptr(prefix_lens), _ptr(prefix_mode),
        _ptr(block_table), 0 if block_table is None else block_table.shape[1],
        ctypes.byref(up) if up is not None else None,
        ctypes.byref(ip) if ip is not None else None,
        B, H, H_kv, D, dt, float(softmax_scale), total, int(max_suffix_len), int(max_prefix_len),
        _ptr(out), _ptr(lse), _ptr(workspace), workspace.numel(), _stream())
    _check(st, "bat_attn_prefill_gqa")
    return out, lse


def attn_prefill_isolated(q, k, v, cu_suffix_lens, prefix_lens, prefix_mode, block_table,
                          tokens_per_candidate, user_pool=None, item_pool=None,
                          softmax_scale=None, max_suffix_len=None, max_prefix_len=None,
                          out=None, lse=None, workspace=None, want_lse=False):
    """Suffix rows over the cached prefix and their own candidate of
    tokens_per_candidate tokens (arguments as attn_prefill)."""
    torch = _torch()
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n, q.dtype)
    _need(cu_suffix_lens, "cu_suffix_lens", torch.int32)
    _need(prefix_lens, "prefix_lens", torch.int32)
    _need(prefix_mode, "prefix_mode", torch.uint8)
    if block_table is not None:
        _need(block_table, "block_table", torch.int32)
    total, H, D = q.shape
    B = cu_suffix_lens.shape[0] - 1
    if max_suffix_len is None:
        max_suffix_len = _max_len(cu_suffix_lens)
    if max_prefix_len is None:
        max_prefix_len = _max_val(prefix_lens)
    if softmax_scale is None:
        softmax_scale = default_scale(D)
    dt = _dtype_code(q)
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", q.dtype)
    if lse is None and want_lse:
        lse = torch.empty((H, total), dtype=torch.float32, device=q.device)
    if lse is not None:
        _need(lse, "lse", torch.float32)
    ws_bytes = int(load().bat_attn_isolated_workspace_size(B, H, D, dt, total, max_suffix_len,
                                                            max_prefix_len))
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=q.device)
    up = user_pool.struct() if user_pool is not None else None
    ip = item_pool.struct() if item_pool is not None else None
    st = load().bat_attn_prefill_isolated(
        _ptr(q), _ptr(k), _ptr(v), _ptr(cu_suffix_lens), _ptr(prefix_lens), _ptr(prefix_mode),
        _ptr(block_table), 0 if block_table is None else block_table.shape[1],
        ctypes.byref(up) if up is not None else None,
        ctypes.byref(ip) if ip is not None else None,
        B, H, D, dt, float(softmax_scale), int(tokens_per_candidate), total,
        int(max_suffix_len), int(max_prefix_len), _ptr(out), _ptr(lse), _ptr(workspace),
        workspace.numel(), _stream())
    _check(st, "bat_attn_prefill_isolated")
    return out, lse


def lse_merge(o_parts, lse_parts, out_dtype, out=None, lse=None, want_lse=True):
    """Merge partials o_parts [n, rows, H, D] fp32 / lse_parts [n, H, rows] fp32."""
    torch = _torch()
    _need(o_parts, "o_parts", torch.float32)
    _need(lse_parts, "lse_parts", torch.float32)
    n, rows, H, D = o_parts.shape
    if out is None:
        out = torch.empty((rows, H, D), dtype=out_dtype, device=o_parts.device)
    if lse is None and want_lse:
        lse = torch.empty((H, rows), dtype=torch.float32, device=o_parts.device)
    st = load().bat_lse_merge(_ptr(o_parts), _ptr(lse_parts), n, rows, H, D,
                              _dtype_code(out), _ptr(out), _ptr(lse), _stream())
    _check(st, "bat_lse_merge")
    return out, lse


class Scheduler:
    """The library's prefix-mode choice over a stream of queries (host side).

    Holds the caller-owned state buffer bat_sched_* works in; numpy arrays
    in and out (the choice runs on the host, not on the GPU)."""

    def __init__(self, policy, item_tokens, user_block, user_capacity_blocks, item_capacity,
                 user_len, num_items):
        import numpy as np
        self._np = np
        self.user_len = np.ascontiguousarray(user_len, dtype=np.int32)
        self.cfg = SchedConfig(int(policy), int(item_tokens), int(user_block),
                               int(item_capacity), int(user_capacity_blocks),
                               len(self.user_len), int(num_items))
        lib = load()
        n = int(lib.bat_sched_state_size(ctypes.byref(self.cfg)))
        if n == 0:
            raise BatError(BAT_ERR_INVALID_ARG, "bat_sched_state_size")
        self.state = np.zeros((n + 7) // 8, dtype=np.int64)  # 8-byte aligned
        _check(lib.bat_sched_init(ctypes.byref(self.cfg), self.user_len.ctypes.data,
                                  self.state.ctypes.data, self.state.nbytes), "bat_sched_init")

    def step(self, user, items):
        """Serve queries in order; returns a dict of per-query arrays."""
        np = self._np
        user = np.ascontiguousarray(user, dtype=np.int32)
        items = np.ascontiguousarray(items, dtype=np.int32)
        R, m = items.shape
        if user.shape != (R,):
            raise BatError(BAT_ERR_INVALID_ARG, "Scheduler.step: user and items disagree")
        out = {"mode": np.empty(R, np.uint8), "user_hit": np.empty(R, np.uint8),
               "item_hits": np.empty(R, np.int32), "prefix_tokens": np.empty(R, np.int64),
               "suffix_tokens": np.empty(R, np.int64), "pairs": np.empty(R, np.int64),
               "item_slot": np.empty((R, m), np.int32)}
        _check(load().bat_sched_step(
            self.state.ctypes.data, R, m, user.ctypes.data, items.ctypes.data,
            *(out[k].ctypes.data for k in ("mode", "user_hit", "item_hits", "prefix_tokens",
                                           "suffix_tokens", "pairs", "item_slot"))),
            "bat_sched_step")
        return out

    def pools(self):
        """(resident users, most recent first; item in each slot, -1 unused)."""
        np = self._np
        users = np.empty(max(len(self.user_len), 1), np.int32)
        n = ctypes.c_int32(0)
        slots = np.empty(max(self.cfg.item_capacity, 1), np.int32)
        _check(load().bat_sched_pools(self.state.ctypes.data, users.ctypes.data,
                                      ctypes.addressof(n), slots.ctypes.data), "bat_sched_pools")
        return users[:n.value].copy(), slots[:self.cfg.item_capacity].copy()
