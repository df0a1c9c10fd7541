"""fp16 sum-reduction on AMD Instinct MI355X (gfx950).

Thin Python binding over the C ABI of ``libarmx.so`` (declared in
``include/armx.h``): it checks tensor types, allocates output and workspace
with PyTorch on the input's device, passes raw device pointers and the
current HIP stream, and turns status codes into exceptions.  Every step of
the reduction runs in the library's HIP kernels; there is no fallback.

Entry points (same names as the C ABI):

* ``reduce_sum(x)`` -- sum of a float16 tensor as a 0-dim float32 tensor, by
  chained MFMAs against an all-ones operand ("GPU Tensor Cores for fast
  Arithmetic Reductions", arXiv 2001.05585, Abstract); ``plain=True`` selects
  the MFMA-free comparison design, ``mma_levels=True`` the recursive form in
  which every level reduces chains with MFMAs only, one launch per level.
* ``reduce_rows(x)`` -- float32 sum of every row of a 2-D float16 tensor.
* ``reduce_sum_fixed_order(x)`` -- sum in one prescribed balanced-tree order,
  bit-identical for every configuration ("Taming Bitwise Behavior in GPU
  Kernels with Tensor Core", arXiv 2609.11356, Abstract); ``mma_leaves=True``
  selects the prescribed order whose leaves are MFMAs.
* ``reduce_rows_fixed_order(x)`` -- the same order per row: each row's bits
  depend on that row only (batch invariance, same Abstract); ``mma_leaves``
  as above.
* ``reduce_sum_exact(x)`` -- the correctly rounded float32 of the exact sum
  (and, with ``fixed=``, the exact sum as a 128-bit count of 2^-24), the
  same bits for every configuration.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

__all__ = [
    "reduce_sum", "reduce_rows", "reduce_sum_fixed_order", "reduce_rows_fixed_order",
    "reduce_sum_exact", "reduce_sum_noalloc", "fixed_to_int", "workspace_bytes", "launch_plan", "ArmxError", "Config",
    "PlanInfo", "LIB_PATH",
    "OP_SUM", "OP_ROWS", "OP_FIXED", "OP_ROWS_FIXED", "OP_EXACT",
    "FLAG_PLAIN", "FLAG_CACHED_LOADS", "FLAG_ONE_CHAIN", "FLAG_TWO_PASS", "FLAG_MMA_LEVELS",
    "FLAG_MMA_LEAVES", "FLAG_ALL_ONES", "FLAG_INT_LIMBS",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libarmx.so")

OP_SUM, OP_ROWS, OP_FIXED, OP_ROWS_FIXED, OP_EXACT = 0, 1, 2, 3, 4
FLAG_PLAIN, FLAG_CACHED_LOADS, FLAG_ONE_CHAIN, FLAG_TWO_PASS = 0x1, 0x2, 0x4, 0x8
FLAG_MMA_LEVELS = 0x10
FLAG_MMA_LEAVES = 0x20
FLAG_ALL_ONES = 0x40
FLAG_INT_LIMBS = 0x80
# the counter region at the start of every non-empty workspace (zero before
# first use; every call leaves it zero)
COUNTER_BYTES = 65536

_STATUS = {
    0: "ARMX_OK", -1: "ARMX_ERR_NULL", -2: "ARMX_ERR_ALIGN", -3: "ARMX_ERR_CONFIG",
    -4: "ARMX_ERR_WORKSPACE", -5: "ARMX_ERR_SHAPE", -6: "ARMX_ERR_HIP",
}


class ArmxError(RuntimeError):
    """A call into libarmx returned a negative status."""

    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status
        self.name = _STATUS.get(status, "unknown")


class Config(ctypes.Structure):
    """Mirror of ``armx_config``."""

    _fields_ = [("block_threads", ctypes.c_int), ("chain_r", ctypes.c_int),
                ("grid_blocks", ctypes.c_int), ("flags", ctypes.c_uint),
                ("start_event", ctypes.c_void_p), ("stop_event", ctypes.c_void_p)]


class PlanInfo(ctypes.Structure):
    """Mirror of ``armx_plan_info``."""

    _fields_ = [("grid_blocks", ctypes.c_int), ("block_threads", ctypes.c_int),
                ("chain_r", ctypes.c_int), ("waves_per_cu", ctypes.c_double),
                ("workspace_bytes", ctypes.c_size_t), ("lds_bytes", ctypes.c_size_t),
                ("launches", ctypes.c_int)]


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with "
            "`python arithmetic_reduction_matrix_amd/_build.py` (or __graft_entry__.build())")
    lib = ctypes.CDLL(LIB_PATH)
    vp, sz, cfgp = ctypes.c_void_p, ctypes.c_size_t, ctypes.POINTER(Config)
    lib.reduce_sum.argtypes = [vp, sz, vp, vp, sz, cfgp, vp]
    lib.reduce_sum_fixed_order.argtypes = [vp, sz, vp, vp, sz, cfgp, vp]
    lib.reduce_rows.argtypes = [vp, sz, sz, sz, vp, vp, sz, cfgp, vp]
    lib.reduce_rows_fixed_order.argtypes = [vp, sz, sz, sz, vp, vp, sz, cfgp, vp]
    lib.reduce_sum_exact.argtypes = [vp, sz, vp, vp, vp, sz, cfgp, vp]
    lib.reduce_sum_noalloc.argtypes = [vp, sz, vp, cfgp, vp]
    for f in (lib.reduce_sum, lib.reduce_sum_fixed_order, lib.reduce_rows,
              lib.reduce_rows_fixed_order, lib.reduce_sum_exact, lib.reduce_sum_noalloc):
        f.restype = ctypes.c_int
    lib.armx_workspace_bytes.argtypes = [ctypes.c_int, sz, sz, cfgp]
    lib.armx_workspace_bytes.restype = sz
    lib.armx_status_string.argtypes = [ctypes.c_int]
    lib.armx_status_string.restype = ctypes.c_char_p
    lib.armx_version.argtypes = []
    lib.armx_version.restype = ctypes.c_int
    lib.armx_launch_plan.argtypes = [ctypes.c_int, sz, sz, cfgp, ctypes.POINTER(PlanInfo)]
    lib.armx_launch_plan.restype = ctypes.c_int
    return lib


lib = _load()


def _event_handle(ev) -> int | None:
    """The hipEvent_t behind a torch.cuda.Event (created on first use)."""
    if ev is None:
        return None
    if not ev.cuda_event:
        ev.record()   # torch creates the HIP event lazily
    return ev.cuda_event


def _config(block_threads=0, chain_r=0, grid_blocks=0, plain=False, cached_loads=False,
            one_chain=False, two_pass=False, mma_levels=False, mma_leaves=False,
            all_ones=False, int_limbs=False, start_event=None, stop_event=None) -> Config:
    flags = ((FLAG_PLAIN if plain else 0) | (FLAG_CACHED_LOADS if cached_loads else 0)
             | (FLAG_ONE_CHAIN if one_chain else 0) | (FLAG_TWO_PASS if two_pass else 0)
             | (FLAG_MMA_LEVELS if mma_levels else 0) | (FLAG_MMA_LEAVES if mma_leaves else 0)
             | (FLAG_ALL_ONES if all_ones else 0) | (FLAG_INT_LIMBS if int_limbs else 0))
    return Config(int(block_threads), int(chain_r), int(grid_blocks), flags,
                  _event_handle(start_event), _event_handle(stop_event))


def _check(status: int, what: str) -> None:
    if status != 0:
        msg = lib.armx_status_string(status).decode()
        raise ArmxError(status, f"{what}: {msg}")


def workspace_bytes(op: int, n_or_rows: int, cols: int = 0, **cfg) -> int:
    """Bytes of workspace the matching call needs (0 if none)."""
    c = _config(**cfg)
    v = lib.armx_workspace_bytes(int(op), int(n_or_rows), int(cols), ctypes.byref(c))
    if v == ctypes.c_size_t(-1).value:
        raise ArmxError(-3, "armx_workspace_bytes: invalid op or configuration")
    return int(v)


def launch_plan(op: int, n_or_rows: int, cols: int = 0, **cfg) -> dict:
    """The launch shape the matching call would use on the current device
    (``armx_launch_plan``): grid_blocks, block_threads, chain_r,
    waves_per_cu, workspace_bytes, lds_bytes, launches."""
    c = _config(**cfg)
    info = PlanInfo()
    _check(lib.armx_launch_plan(int(op), int(n_or_rows), int(cols), ctypes.byref(c),
                                ctypes.byref(info)), "armx_launch_plan")
    return {name: getattr(info, name) for name, _ in PlanInfo._fields_}


# Zero-filled workspaces, one per (device, stream); a call leaves its
# workspace's counter at zero, so calls on one stream can share one.
_ws_lock = threading.Lock()
_ws_cache: dict[tuple[int, int], torch.Tensor] = {}


def _workspace(device: torch.device, stream: int, nbytes: int) -> torch.Tensor | None:
    if nbytes == 0:
        return None
    key = (device.index, stream)
    with _ws_lock:
        ws = _ws_cache.get(key)
        if ws is None or ws.numel() < nbytes:
            size = max(nbytes, 1 << 16)
            ws = torch.zeros(size, dtype=torch.uint8, device=device)
            _ws_cache[key] = ws
        return ws


def _check_input(x: torch.Tensor, ndim: int | None, name: str) -> None:
    if not isinstance(x, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor")
    if x.dtype != torch.float16:
        raise TypeError(f"{name}: expected float16, got {x.dtype}")
    if not x.is_cuda:
        raise ValueError(f"{name}: the input must be on a GPU (HIP) device")
    if ndim is not None and x.dim() != ndim:
        raise ValueError(f"{name}: expected a {ndim}-D tensor, got {x.dim()}-D")


class _on_device:
    """Makes `dev` the current device for the duration, only if it is not."""

    def __init__(self, dev: torch.device):
        self.dev = dev.index if dev.index is not None else torch.cuda.current_device()
        self.prev = None

    def __enter__(self):
        cur = torch.cuda.current_device()
        if cur != self.dev:
            self.prev = cur
            torch.cuda.set_device(self.dev)

    def __exit__(self, *exc):
        if self.prev is not None:
            torch.cuda.set_device(self.prev)


def _flat_call(fn, op: int, x: torch.Tensor, out, workspace, cfg: Config, name: str,
               fixed=None):
    _check_input(x, None, name)
    if not x.is_contiguous():
        raise ValueError(f"{name}: the input must be contiguous")
    n = x.numel()
    dev = x.device
    with _on_device(dev):
        stream = torch.cuda.current_stream(dev).cuda_stream
        if out is None:
            out = torch.empty((), dtype=torch.float32, device=dev)
        elif out.dtype != torch.float32 or out.device != dev or out.numel() < 1:
            raise ValueError(f"{name}: out must be a float32 tensor on {dev}")
        if workspace is None:
            need = lib.armx_workspace_bytes(op, n, 0, ctypes.byref(cfg))
            if need == ctypes.c_size_t(-1).value:
                _check(-3, name)
            ws = _workspace(dev, stream, need)
        else:
            ws = workspace
        ws_ptr = ws.data_ptr() if ws is not None else None
        ws_bytes = ws.numel() * ws.element_size() if ws is not None else 0
        if op == OP_EXACT:
            if fixed is not None and (fixed.dtype != torch.int64 or fixed.device != dev
                                      or fixed.numel() < 2 or not fixed.is_contiguous()):
                raise ValueError(f"{name}: fixed must be a contiguous int64 tensor of 2 on {dev}")
            st = fn(x.data_ptr() if n else None, n, out.data_ptr(),
                    fixed.data_ptr() if fixed is not None else None, ws_ptr, ws_bytes,
                    ctypes.byref(cfg), stream)
        else:
            st = fn(x.data_ptr() if n else None, n, out.data_ptr(), ws_ptr, ws_bytes,
                    ctypes.byref(cfg), stream)
    _check(st, name)
    return out


def reduce_sum(x: torch.Tensor, *, out: torch.Tensor | None = None,
               workspace: torch.Tensor | None = None, **cfg) -> torch.Tensor:
    """Sum of all elements of a contiguous float16 GPU tensor, as float32.

    Keyword configuration: block_threads, chain_r, grid_blocks, plain,
    all_ones, cached_loads, one_chain, two_pass, mma_levels (see
    ``include/armx.h``),
    and start_event / stop_event (torch.cuda.Event with timing) which the
    main kernel's dispatch stamps when it starts and completes (with
    mma_levels: the first level's start and the last level's completion).  A workspace
    passed explicitly must be zero-filled before its first use.
    """
    return _flat_call(lib.reduce_sum, OP_SUM, x, out, workspace, _config(**cfg), "reduce_sum")


def reduce_sum_noalloc(x: torch.Tensor, *, out: torch.Tensor, **cfg) -> torch.Tensor:
    """reduce_sum into a caller-allocated ``out`` (a float32 GPU tensor) with
    no workspace: the library's static per-device scratch array stands in
    for it, so the call allocates nothing.  Calls that may overlap on one
    device race on that array."""
    _check_input(x, None, "reduce_sum_noalloc")
    if not x.is_contiguous():
        raise ValueError("reduce_sum_noalloc: the input must be contiguous")
    dev = x.device
    if out.dtype != torch.float32 or out.device != dev or out.numel() < 1:
        raise ValueError(f"reduce_sum_noalloc: out must be a float32 tensor on {dev}")
    n = x.numel()
    with _on_device(dev):
        stream = torch.cuda.current_stream(dev).cuda_stream
        c = _config(**cfg)
        st = lib.reduce_sum_noalloc(x.data_ptr() if n else None, n, out.data_ptr(),
                                    ctypes.byref(c), stream)
    _check(st, "reduce_sum_noalloc")
    return out


def reduce_sum_fixed_order(x: torch.Tensor, *, out: torch.Tensor | None = None,
                           workspace: torch.Tensor | None = None, **cfg) -> torch.Tensor:
    """Balanced-tree-order sum of a contiguous float16 GPU tensor, as float32;
    the same bits for every configuration."""
    return _flat_call(lib.reduce_sum_fixed_order, OP_FIXED, x, out, workspace, _config(**cfg),
                      "reduce_sum_fixed_order")


def reduce_sum_exact(x: torch.Tensor, *, out: torch.Tensor | None = None,
                     fixed: torch.Tensor | None = None,
                     workspace: torch.Tensor | None = None, **cfg) -> torch.Tensor:
    """The float32 nearest (ties to even) to the exact sum of a contiguous
    float16 GPU tensor; the same bits for every configuration.  If ``fixed``
    (an int64 GPU tensor of 2) is given, the exact sum is also written there
    as a 128-bit count of 2^-24 (low word, high word); ``fixed_to_int``
    turns it into a Python int."""
    return _flat_call(lib.reduce_sum_exact, OP_EXACT, x, out, workspace, _config(**cfg),
                      "reduce_sum_exact", fixed=fixed)


def fixed_to_int(fixed) -> int:
    """The 128-bit count written by reduce_sum_exact (two int64 words, low
    first) as a Python int."""
    lo, hi = (int(v) for v in fixed.reshape(-1)[:2].tolist())
    return (hi << 64) + (lo & ((1 << 64) - 1))


def _rows_call(fn, op: int, x: torch.Tensor, out, workspace, cfg: Config,
               name: str) -> torch.Tensor:
    _check_input(x, 2, name)
    rows, cols = x.shape
    if cols > 1 and x.stride(1) != 1:
        raise ValueError(f"{name}: rows must be contiguous (stride(1) == 1)")
    ld = x.stride(0) if rows > 1 and cols > 0 else cols
    dev = x.device
    with _on_device(dev):
        stream = torch.cuda.current_stream(dev).cuda_stream
        if out is None:
            out = torch.empty(rows, dtype=torch.float32, device=dev)
        elif out.dtype != torch.float32 or out.device != dev or out.numel() < rows:
            raise ValueError(f"{name}: out must be a float32 tensor of {rows} on {dev}")
        if workspace is None:
            # few long rows are split over wavefronts of several blocks, which
            # takes a workspace (none for other shapes)
            need = lib.armx_workspace_bytes(op, rows, cols, ctypes.byref(cfg))
            if need == ctypes.c_size_t(-1).value:
                need = 0   # the call itself reports the configuration error
            ws = _workspace(dev, stream, need)
        else:
            ws = workspace
        ws_ptr = ws.data_ptr() if ws is not None else None
        ws_bytes = ws.numel() * ws.element_size() if ws is not None else 0
        st = fn(x.data_ptr() if x.numel() else None, rows, cols, ld,
                out.data_ptr() if rows else None, ws_ptr, ws_bytes, ctypes.byref(cfg), stream)
    _check(st, name)
    return out


def reduce_rows(x: torch.Tensor, *, out: torch.Tensor | None = None,
                workspace: torch.Tensor | None = None, **cfg) -> torch.Tensor:
    """float32 sum of every row of a 2-D float16 GPU tensor whose rows are
    contiguous (``x.stride(1) == 1``) with a row pitch that is a multiple of 8.
    A workspace is used only when rows are split over wavefronts of several
    blocks (too few rows to fill the device, or a row stream whose last round
    would be poorly filled); by default one is taken from a per-stream
    cache."""
    return _rows_call(lib.reduce_rows, OP_ROWS, x, out, workspace, _config(**cfg),
                      "reduce_rows")


def reduce_rows_fixed_order(x: torch.Tensor, *, out: torch.Tensor | None = None,
                            workspace: torch.Tensor | None = None, **cfg) -> torch.Tensor:
    """Balanced-tree-order float32 sum of every row (as reduce_rows): row r's
    bits depend on row r's values only (batch invariant).  ``mma_leaves=True``
    gives each row the order with MFMA leaves of reduce_sum_fixed_order."""
    return _rows_call(lib.reduce_rows_fixed_order, OP_ROWS_FIXED, x, out, workspace,
                      _config(**cfg), "reduce_rows_fixed_order")
