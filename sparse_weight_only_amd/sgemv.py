"""ctypes binding of the SparseGemv C ABI (``include/sgemv.h``).

Functions keep the C names without the ``sgemv_`` prefix and only marshal
arguments: NumPy arrays for host buffers, raw device pointers (ints) for
device buffers, a raw ``hipStream_t`` (int) for the stream. Errors raise
``SgemvError``. ``SparseGemvLayer`` bundles describe -> pack -> layout ->
upload with torch-owned device memory.

The library must have been built (``__graft_entry__.build()`` or
``python sparse_weight_only_amd/_build.py``); nothing here falls back to
another implementation.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# SGEMV_LIB may name another build of the same ABI (the tests load a
# host-only build with address and undefined-behaviour sanitizers this way)
_LIB_PATH = os.environ.get("SGEMV_LIB") or os.path.join(_HERE, "_lib", "libsgemv.so")
_lib = None

SGEMV_OK, SGEMV_EINVAL, SGEMV_ESIZE, SGEMV_EALIGN, SGEMV_EHIP = 0, -1, -2, -3, -4


class SgemvError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {strerror(code)} (status {code})")


class Desc(ctypes.Structure):
    _fields_ = [
        ("N", ctypes.c_int32), ("K", ctypes.c_int32), ("nk", ctypes.c_int32),
        ("n_blocks", ctypes.c_int32), ("chunks", ctypes.c_int32),
        ("g_min", ctypes.c_int32), ("g_max", ctypes.c_int32),
        ("class_rows", ctypes.c_int32 * 4), ("value_format", ctypes.c_int32),
        ("kept", ctypes.c_int64), ("vals_bytes", ctypes.c_int64), ("offs_bytes", ctypes.c_int64),
        ("n_groups", ctypes.c_int64), ("off_codes", ctypes.c_int64), ("off_offs", ctypes.c_int64),
        ("off_perm", ctypes.c_int64), ("off_sz", ctypes.c_int64), ("blob_bytes", ctypes.c_int64),
    ]

    def as_dict(self) -> dict:
        return {f: (list(getattr(self, f)) if f == "class_rows" else getattr(self, f)) for f, _ in self._fields_}


class Plan(ctypes.Structure):
    _fields_ = [
        ("grid", ctypes.c_int64), ("lds_bytes", ctypes.c_int64), ("block", ctypes.c_int32),
        ("waves", ctypes.c_int32), ("chunks_per_wave", ctypes.c_int32), ("phase_chunks", ctypes.c_int32),
        ("x_loads", ctypes.c_int32), ("row_blocks", ctypes.c_int32), ("full_waves", ctypes.c_int32),
    ]

    def as_dict(self) -> dict:
        return {f: getattr(self, f) for f, _ in self._fields_}


class Task(ctypes.Structure):
    """One layer of a several-layer launch (mirrors sgemv_task)."""
    _fields_ = [("desc", ctypes.POINTER(Desc)), ("blob_dev", ctypes.c_void_p),
                ("x_dev", ctypes.c_void_p), ("y_dev", ctypes.c_void_p)]


class ListLaunch(ctypes.Structure):
    """The launch of a task table (mirrors sgemv_list_launch)."""
    _fields_ = [("table_bytes", ctypes.c_int64), ("lds_bytes", ctypes.c_int64), ("workgroups", ctypes.c_int64),
                ("rows", ctypes.c_int32), ("row_width", ctypes.c_int32), ("tasks", ctypes.c_int32),
                ("block", ctypes.c_int32)]

    def as_dict(self) -> dict:
        return {f: getattr(self, f) for f, _ in self._fields_}


MAX_GROUP = 32


def lib_path() -> str:
    return _LIB_PATH


def lib():
    """Load the C-ABI library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"SparseGemv library not built: {_LIB_PATH} is missing "
                               "(run __graft_entry__.build())")
        L = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        i32, i64, u32, f64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32, ctypes.c_double
        D, PL, TK = ctypes.POINTER(Desc), ctypes.POINTER(Plan), ctypes.POINTER(Task)
        LL = ctypes.POINTER(ListLaunch)
        sigs = {
            "sgemv_describe": [i32, i32, i32, P, D],
            "sgemv_select_groups": [P, i32, i32, i32, P, i32, f64, i32, i32, P],
            "sgemv_pack": [P, i32, i32, i32, P, P, P, P, P, P, P],
            "sgemv_prune": [P, i32, i32, i32, P, i32, P],
            "sgemv_describe_fp16": [i32, i32, i32, D],
            "sgemv_pack_fp16": [P, i32, i32, i32, P, P, P],
            "sgemv_layout_fp16": [D, P, P, P],
            "sgemv_layout": [D, P, P, P, P, P, P],
            "sgemv_f64_to_f16": [P, P, i64],
            "sgemv_run": [D, P, P, P, i32, P],
            "sgemv_plan": [D, i32, PL],
            "sgemv_run_group": [TK, i32, i32, P],
            "sgemv_plan_group": [TK, i32, i32, PL],
            "sgemv_run_list": [TK, i32, i32, P],
            "sgemv_plan_list": [TK, i32, i32, PL],
            "sgemv_list_table": [TK, i32, i32, P, i64, LL],
            "sgemv_run_list_table": [P, LL, P],
            "sgemv_probe_read": [P, i64, P, i64, u32, P],
            "sgemv_probe_empty": [i32, i32, P],
        }
        for f, argtypes in sigs.items():
            if not hasattr(L, f):
                # only a host-only build named by SGEMV_LIB lacks the GPU entry points
                if "SGEMV_LIB" in os.environ:
                    continue
                raise RuntimeError(f"{_LIB_PATH} does not export {f}")
            getattr(L, f).argtypes = argtypes
            getattr(L, f).restype = ctypes.c_int
        L.sgemv_strerror.argtypes = [ctypes.c_int]
        L.sgemv_strerror.restype = ctypes.c_char_p
        _lib = L
    return _lib


def strerror(code: int) -> str:
    return lib().sgemv_strerror(int(code)).decode()


def _check(code: int, where: str):
    if code != SGEMV_OK:
        raise SgemvError(code, where)


def _host(a: np.ndarray, dtype) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != dtype:
        raise TypeError(f"expected {np.dtype(dtype)}, got {a.dtype}")
    return a


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def describe(N: int, K: int, nk: int, group_size) -> Desc:
    gs = _host(np.asarray(group_size, dtype=np.int32), np.int32)
    if gs.shape != (N,):
        raise ValueError("group_size must have one entry per row")
    d = Desc()
    _check(lib().sgemv_describe(N, K, nk, _ptr(gs), ctypes.byref(d)), "sgemv_describe")
    return d


def select_groups(w16: np.ndarray, nk: int, xcal16: np.ndarray, frac_fine: float = 0.10,
                  g_fine: int = 32, g_coarse: int = 128) -> np.ndarray:
    w = _host(np.asarray(w16).view(np.uint16), np.uint16)
    xc = _host(np.asarray(xcal16).view(np.uint16), np.uint16)
    N, K = w.shape
    if xc.ndim != 2 or xc.shape[1] != K:
        # the library reads T x K halves at xcal's address
        raise ValueError("xcal must be [T, K]")
    out = np.empty(N, dtype=np.int32)
    _check(lib().sgemv_select_groups(_ptr(w), N, K, nk, _ptr(xc), xc.shape[0], float(frac_fine),
                                     g_fine, g_coarse, _ptr(out)), "sgemv_select_groups")
    return out


def prune(w16: np.ndarray, nk: int, xcal16=None) -> np.ndarray:
    """Activation-aware N:M pruning (score |w| * ||x_k||; |w| without xcal):
    FP16 [N, K] with the kept values and +0 elsewhere."""
    w = _host(np.asarray(w16).view(np.uint16), np.uint16)
    N, K = w.shape
    out = np.empty((N, K), dtype=np.uint16)
    if xcal16 is None:
        _check(lib().sgemv_prune(_ptr(w), N, K, nk, None, 0, _ptr(out)), "sgemv_prune")
    else:
        xc = _host(np.asarray(xcal16).view(np.uint16), np.uint16)
        if xc.ndim != 2 or xc.shape[1] != K:
            raise ValueError("xcal must be [T, K]")
        _check(lib().sgemv_prune(_ptr(w), N, K, nk, _ptr(xc), xc.shape[0], _ptr(out)), "sgemv_prune")
    return out.view(np.float16)


def pack(w16: np.ndarray, nk: int, group_size) -> dict:
    """Dense FP16 [N, K] -> canonical 2bit-CSR arrays (dict of NumPy arrays)."""
    w = _host(np.asarray(w16).view(np.uint16), np.uint16)
    N, K = w.shape
    gs = _host(np.asarray(group_size, dtype=np.int32), np.int32)
    if gs.shape != (N,):
        raise ValueError("group_size must have one entry per row")
    if K % 256 or nk not in (1, 2, 4):
        _check(SGEMV_EINVAL, "sgemv_pack")
    kpr = K * nk // 4
    ng = int(np.sum(K // np.maximum(gs.astype(np.int64), 1)))
    vals = np.empty((N, kpr // 2), dtype=np.uint8)
    offs = np.empty((N, 0 if nk == 4 else kpr // 4), dtype=np.uint8)   # dense (nk = 4): no offsets
    scale = np.empty(max(ng, 1), dtype=np.uint16)
    zero = np.empty(max(ng, 1), dtype=np.uint16)
    gptr = np.empty(N + 1, dtype=np.int32)
    rowptr = np.empty(N + 1, dtype=np.int32)
    _check(lib().sgemv_pack(_ptr(w), N, K, nk, _ptr(gs), _ptr(vals), _ptr(offs), _ptr(scale),
                            _ptr(zero), _ptr(gptr), _ptr(rowptr)), "sgemv_pack")
    return {"N": N, "K": K, "nk": nk, "group_size": gs, "vals": vals, "offs": offs,
            "scale": scale[:ng], "zero": zero[:ng], "gptr": gptr, "rowptr": rowptr}


def layout(desc: Desc, canon: dict) -> np.ndarray:
    """Canonical arrays -> kernel-layout blob (host uint8 array of desc.blob_bytes)."""
    blob = np.empty(desc.blob_bytes, dtype=np.uint8)
    arrs = [_host(canon["vals"], np.uint8), _host(canon["offs"], np.uint8),
            _host(canon["scale"], np.uint16), _host(canon["zero"], np.uint16),
            _host(canon["gptr"], np.int32)]
    _check(lib().sgemv_layout(ctypes.byref(desc), *[_ptr(a) for a in arrs], _ptr(blob)), "sgemv_layout")
    return blob


def f64_to_f16(x: np.ndarray) -> np.ndarray:
    """The packer's FP64 -> FP16 conversion (round to nearest even, one step):
    FP16 bit patterns (uint16) of the same shape."""
    a = _host(np.asarray(x, dtype=np.float64), np.float64)
    out = np.empty(a.shape, dtype=np.uint16)
    _check(lib().sgemv_f64_to_f16(_ptr(a), _ptr(out), a.size), "sgemv_f64_to_f16")
    return out


def probe_read(src_dev: int, nbytes: int, dst_dev: int, store_bytes: int, magic: int = 0x9E3779B9,
               stream: int = 0) -> None:
    """Enqueue the plain-read probe (16 bytes per lane; store_bytes written)."""
    _check(lib().sgemv_probe_read(ctypes.c_void_p(src_dev), int(nbytes), ctypes.c_void_p(dst_dev),
                                  int(store_bytes), int(magic) & 0xFFFFFFFF, ctypes.c_void_p(stream)),
           "sgemv_probe_read")


def probe_empty(grid: int = 1, block: int = 64, stream: int = 0) -> None:
    """Enqueue the empty-kernel probe."""
    _check(lib().sgemv_probe_empty(int(grid), int(block), ctypes.c_void_p(stream)), "sgemv_probe_empty")


def describe_fp16(N: int, K: int, nk: int) -> Desc:
    """Descriptor of the FP16-valued form (no groups)."""
    d = Desc()
    _check(lib().sgemv_describe_fp16(N, K, nk, ctypes.byref(d)), "sgemv_describe_fp16")
    return d


def pack_fp16(w16: np.ndarray, nk: int) -> dict:
    """Dense FP16 [N, K] -> N:M prune -> FP16-valued 2bit-CSR arrays."""
    w = _host(np.asarray(w16).view(np.uint16), np.uint16)
    N, K = w.shape
    if K % 256 or nk not in (1, 2):
        _check(SGEMV_EINVAL, "sgemv_pack_fp16")
    kpr = K * nk // 4
    vals16 = np.empty((N, kpr), dtype=np.uint16)
    offs = np.empty((N, kpr // 4), dtype=np.uint8)
    rowptr = np.empty(N + 1, dtype=np.int32)
    _check(lib().sgemv_pack_fp16(_ptr(w), N, K, nk, _ptr(vals16), _ptr(offs), _ptr(rowptr)), "sgemv_pack_fp16")
    return {"N": N, "K": K, "nk": nk, "vals16": vals16, "offs": offs, "rowptr": rowptr}


def layout_fp16(desc: Desc, canon16: dict) -> np.ndarray:
    """FP16-valued canonical arrays -> kernel-layout blob (host uint8 array)."""
    blob = np.empty(desc.blob_bytes, dtype=np.uint8)
    v = _host(canon16["vals16"], np.uint16)
    o = _host(canon16["offs"], np.uint8)
    _check(lib().sgemv_layout_fp16(ctypes.byref(desc), _ptr(v), _ptr(o), _ptr(blob)), "sgemv_layout_fp16")
    return blob


def run(desc: Desc, blob_dev: int, x_dev: int, y_dev: int, B: int, stream: int = 0) -> None:
    """Enqueue y = W' x on ``stream`` (raw device pointers as ints)."""
    _check(lib().sgemv_run(ctypes.byref(desc), ctypes.c_void_p(blob_dev), ctypes.c_void_p(x_dev),
                           ctypes.c_void_p(y_dev), B, ctypes.c_void_p(stream)), "sgemv_run")


def plan(desc: Desc, B: int) -> Plan:
    """The launch sgemv_run would make for (desc, B); no GPU needed."""
    pl = Plan()
    _check(lib().sgemv_plan(ctypes.byref(desc), B, ctypes.byref(pl)), "sgemv_plan")
    return pl


def _tasks(tasks):
    """[(desc, blob_dev, x_dev, y_dev), ...] -> ctypes array of Task (descs kept alive by the caller)."""
    arr = (Task * max(1, len(tasks)))()
    for i, (d, blob, x, y) in enumerate(tasks):
        arr[i] = Task(ctypes.pointer(d), ctypes.c_void_p(blob), ctypes.c_void_p(x), ctypes.c_void_p(y))
    return arr


def run_group(tasks, B: int, stream: int = 0) -> None:
    """Enqueue several independent GEMVs (same N:M choice) as one launch;
    ``tasks`` lists (desc, blob_dev, x_dev, y_dev) with raw device pointers."""
    _check(lib().sgemv_run_group(_tasks(tasks), len(tasks), B, ctypes.c_void_p(stream)), "sgemv_run_group")


def plan_group(tasks, B: int) -> Plan:
    """The launch sgemv_run_group would make; no GPU needed (pointers may be 0)."""
    pl = Plan()
    _check(lib().sgemv_plan_group(_tasks(tasks), len(tasks), B, ctypes.byref(pl)), "sgemv_plan_group")
    return pl


LIST_MAX = 48


def run_list(tasks, B: int = 1, stream: int = 0) -> None:
    """Enqueue up to LIST_MAX independent one-vector GEMVs (INT4 form, 2:4
    and 1:4 may mix, any shapes) as one launch; ``tasks`` lists (desc,
    blob_dev, x_dev, y_dev) with raw device pointers."""
    _check(lib().sgemv_run_list(_tasks(tasks), len(tasks), B, ctypes.c_void_p(stream)), "sgemv_run_list")


def plan_list(tasks, B: int = 1) -> Plan:
    """The launch sgemv_run_list would make; no GPU needed (pointers may be 0)."""
    pl = Plan()
    _check(lib().sgemv_plan_list(_tasks(tasks), len(tasks), B, ctypes.byref(pl)), "sgemv_plan_list")
    return pl


LIST_TABLE_MAX = 4096


def list_table(tasks, B: int = 1):
    """Plan one launch over up to LIST_TABLE_MAX one-vector GEMVs: returns
    (table, launch), the table as a host uint8 array to be copied to device
    memory, and the ListLaunch that sgemv_run_list_table takes with it."""
    arr = _tasks(tasks)
    launch = ListLaunch()
    _check(lib().sgemv_list_table(arr, len(tasks), B, None, 0, ctypes.byref(launch)), "sgemv_list_table")
    table = np.zeros(launch.table_bytes, dtype=np.uint8)
    _check(lib().sgemv_list_table(arr, len(tasks), B, _ptr(table), table.size, ctypes.byref(launch)),
           "sgemv_list_table")
    return table, launch


def run_list_table(table_dev: int, launch: ListLaunch, stream: int = 0) -> None:
    """Enqueue the launch of a task table held at ``table_dev`` (device pointer as int)."""
    _check(lib().sgemv_run_list_table(ctypes.c_void_p(table_dev), ctypes.byref(launch), ctypes.c_void_p(stream)),
           "sgemv_run_list_table")


def algorithmic_bytes(desc: Desc, B: int) -> int:
    """Bytes the method must move per call: values (INT4 codes or FP16) + offsets
    + FP16 scale/zero (INT4 form only) + x + y."""
    return int(desc.vals_bytes + desc.offs_bytes + 4 * desc.n_groups + 2 * B * desc.K + 2 * B * desc.N)


class SparseGemvLayer:
    """One packed layer resident on the GPU (torch-owned device blob)."""

    def __init__(self, desc: Desc, canon: dict, blob_host: np.ndarray, device="cuda"):
        import torch
        self.desc = desc
        self.canon = canon
        self.blob_host = blob_host
        self.blob = torch.from_numpy(blob_host).to(device)
        if self.blob.data_ptr() % 256:
            raise RuntimeError("device blob is not 256-byte aligned")

    @classmethod
    def from_dense(cls, w16: np.ndarray, nk: int, group_size=None, xcal16: Optional[np.ndarray] = None,
                   frac_fine: float = 0.10, g_fine: int = 32, g_coarse: int = 128,
                   device="cuda") -> "SparseGemvLayer":
        w16 = np.asarray(w16, dtype=np.float16)
        N, K = w16.shape
        if group_size is None:
            group_size = np.full(N, g_coarse, dtype=np.int32)
        elif isinstance(group_size, str) and group_size == "adaptive":
            if xcal16 is None:
                raise ValueError("adaptive groups need a calibration batch")
            group_size = select_groups(w16, nk, xcal16, frac_fine, g_fine, g_coarse)
        canon = pack(w16, nk, group_size)
        desc = describe(N, K, nk, group_size)
        return cls(desc, canon, layout(desc, canon), device)

    @classmethod
    def from_dense_fp16(cls, w16: np.ndarray, nk: int, device="cuda") -> "SparseGemvLayer":
        """The FP16-valued form: N:M pruning only, the kept values in FP16."""
        w16 = np.asarray(w16, dtype=np.float16)
        N, K = w16.shape
        canon = pack_fp16(w16, nk)
        desc = describe_fp16(N, K, nk)
        return cls(desc, canon, layout_fp16(desc, canon), device)

    def run(self, x, y=None, stream=None):
        """y = W' x for a torch FP16 tensor x of shape [K] or [B, K] on the device."""
        import torch
        squeeze = x.dim() == 1
        x2 = x.reshape(1, -1) if squeeze else x
        if x2.dim() != 2 or x2.dtype != torch.float16 or not x2.is_contiguous() or x2.shape[1] != self.desc.K:
            raise ValueError("x must be a contiguous FP16 tensor of shape [K] or [B, K]")
        if x2.device != self.blob.device:
            raise ValueError(f"x is on {x2.device}, the layer on {self.blob.device}")
        B = x2.shape[0]
        if y is None:
            y = torch.empty((B, self.desc.N), dtype=torch.float16, device=x.device)
        elif (y.dtype != torch.float16 or not y.is_contiguous() or y.device != self.blob.device
              or y.numel() != B * self.desc.N):
            # the kernel writes B * N FP16 values at y's address: anything else
            # would be written past the end of a smaller buffer
            raise ValueError(f"y must be a contiguous FP16 tensor of {B * self.desc.N} elements on {self.blob.device}")
        s = stream if stream is not None else torch.cuda.current_stream(x.device)
        run(self.desc, self.blob.data_ptr(), x2.data_ptr(), y.data_ptr(), B, s.cuda_stream)
        return y.reshape(-1) if squeeze else y
