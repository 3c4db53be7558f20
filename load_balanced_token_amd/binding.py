"""Thin Python binding of liblbt.so (include/lbt.h): ctypes argument
marshalling only.  Every step of the path runs in the HIP kernels; PyTorch
supplies device memory and the current stream.  A missing library raises.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "liblbt.so")

SOFTMAX = 0
SIGMOID = 1
Y_F32 = 0
Y_BF16 = 1

OK = 0                   # return codes (LBT_OK, LBT_E*)
EINVAL = -1
EHIP = -2
EUNSUPPORTED = -3

ST_BADCOUNT = 1
ST_CAPACITY = 2
ST_BADID = 4
ST_DUPID = 8

ABI_VERSION = 4          # LBT_VERSION of include/lbt.h this binding's structs follow

HDR_N_PIECES = 0
HDR_MAX_T = 1
HDR_MAX_L = 2
HDR_TOTAL_OVERFLOW = 3
HDR_N_DEFICIT_RANKS = 4
HDR_N_OVERFLOW_RANKS = 5
HDR_N_OVERFLOW_EXPERTS = 6
HDR_STATUS = 7
HDR_P = 8
HDR_TAU = 9
HDR_MAX_REPLICAS = 10
HDR_FEASIBLE = 11
HDR_LOCAL = 12

EXPORTS = ("lbt_query_sizes", "lbt_route_topk", "lbt_histogram", "lbt_plan_balance",
           "lbt_route_plan", "lbt_front", "lbt_front_dispatch",
           "lbt_plan_quota", "lbt_align_sort", "lbt_align_sort_noalloc", "lbt_align_dispatch",
           "lbt_dispatch",
           "lbt_combine",
           "lbt_prefetch_weights", "lbt_reduce_grad", "lbt_combine_bwd", "lbt_dispatch_bwd",
           "lbt_strerror", "lbt_last_hip_error", "lbt_version")


class LbtShape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("E", "K", "R", "S", "H", "B", "blk", "score_fn", "renorm", "cap", "tau_max")]


_SIZE_FIELDS = (
    "N", "P", "SK", "C", "n_blocks", "tile_tokens", "tiles_per_rank", "n_tiles", "work_words",
    "max_seg", "max_pieces", "plan_words",
    "off_hdr", "off_T", "off_h", "off_O", "off_home_row", "off_L", "off_def", "off_D",
    "off_n_seg", "off_n_rows_padded", "off_n_slots", "off_n_remote",
    "off_seg_expert", "off_seg_wrow", "off_seg_count", "off_seg_start",
    "off_piece_expert", "off_piece_rank", "off_piece_count", "off_piece_line", "off_piece_row",
    "off_piece_wrow", "off_home_local", "off_piece_local",
)


class LbtSizes(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in _SIZE_FIELDS]


class LbtError(RuntimeError):
    pass


_lib = None


def lib() -> ctypes.CDLL:
    """Load liblbt.so (built in-tree by load_balanced_token_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise LbtError(f"{LIB_PATH} is missing: build it with "
                           "`python -m load_balanced_token_amd.build`")
        # torch first: it ships its own HIP runtime under the soname the
        # library links against, so loading torch before the library makes
        # both use that one runtime.  Loaded the other way round, the library
        # would bind to the system runtime and torch would load a second
        # copy, whose streams and memory the library's launches cannot use.
        _torch()
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        I = ctypes.c_int
        SP = ctypes.POINTER(LbtShape)
        L.lbt_query_sizes.argtypes = [SP, ctypes.POINTER(LbtSizes)]
        L.lbt_route_topk.argtypes = [SP, P, P, P, P, P, P, P]
        L.lbt_histogram.argtypes = [SP, P, P, P, P, P]
        L.lbt_plan_balance.argtypes = [SP, P, P, P, P]
        L.lbt_plan_quota.argtypes = [SP, P, P, P, P]
        L.lbt_route_plan.argtypes = [SP, P, P, P, P, P, P, P, P, P]
        L.lbt_front.argtypes = [SP, P, P, P, P, P, P, P, P, P, P, P, P, P]
        L.lbt_front_dispatch.argtypes = [SP, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P]
        L.lbt_align_dispatch.argtypes = [SP, P, P, P, P, P, P, P, P, P, P, P]
        L.lbt_align_sort.argtypes = [SP, P, P, P, P, P, P, P, P, P]
        L.lbt_align_sort_noalloc.argtypes = [SP, P, P, P, P, P, P, P, P]
        L.lbt_dispatch.argtypes = [SP, P, P, P, P]
        L.lbt_combine.argtypes = [SP, P, P, P, ctypes.c_int32, P, P]
        L.lbt_prefetch_weights.argtypes = [SP, P, P, P, ctypes.c_int64, P]
        L.lbt_reduce_grad.argtypes = [SP, P, P, P, ctypes.c_int64, P]
        L.lbt_combine_bwd.argtypes = [SP, P, P, P, ctypes.c_int32, P, P, P, P]
        L.lbt_dispatch_bwd.argtypes = [SP, P, P, ctypes.c_int32, P, P]
        L.lbt_strerror.argtypes = [I]
        L.lbt_strerror.restype = ctypes.c_char_p
        L.lbt_last_hip_error.argtypes = []
        L.lbt_last_hip_error.restype = ctypes.c_char_p
        L.lbt_version.argtypes = []
        for n in EXPORTS:
            if n not in ("lbt_strerror", "lbt_last_hip_error"):
                getattr(L, n).restype = I
        if L.lbt_version() != ABI_VERSION:
            raise LbtError(f"{LIB_PATH} is ABI version {L.lbt_version()}, this binding expects "
                           f"{ABI_VERSION} (the lbt_sizes layout differs): rebuild it")
        _lib = L
    return _lib


def _check(rc: int, what: str) -> None:
    if rc != 0:
        msg = f"{what}: {lib().lbt_strerror(rc).decode()} (code {rc}"
        if rc == EHIP:
            msg += f", {lib().lbt_last_hip_error().decode()}"
        raise LbtError(msg + ")")


@dataclasses.dataclass(frozen=True)
class Shape:
    E: int
    K: int
    R: int
    S: int
    H: int
    B: int
    blk: int
    score_fn: int = SIGMOID
    renorm: int = 0
    cap: int = 0
    tau_max: int = 0

    def c(self) -> LbtShape:
        return LbtShape(*(int(getattr(self, f.name)) for f in dataclasses.fields(self)))

    @property
    def N(self) -> int:
        return self.R * self.S

    @property
    def P(self) -> int:
        return self.R * self.S * self.K


def query_sizes(shape: Shape) -> dict:
    z = LbtSizes()
    sh = shape.c()
    _check(lib().lbt_query_sizes(ctypes.byref(sh), ctypes.byref(z)), "lbt_query_sizes")
    return {n: int(getattr(z, n)) for n in _SIZE_FIELDS}


# --------------------------------------------------------------------------- torch side
def _torch():
    import torch
    return torch


def _ptr(t, dtype, numel, name, align16=False):
    torch = _torch()
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise LbtError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise LbtError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise LbtError(f"{name} must be contiguous")
    if t.numel() < numel:
        raise LbtError(f"{name} has {t.numel()} elements, needs {numel}")
    p = t.data_ptr()
    if align16 and p % 16:
        raise LbtError(f"{name} must be 16-byte aligned")
    return p


def _raw(t, name):
    """Device pointer of a contiguous tensor of any dtype (byte-level calls)."""
    torch = _torch()
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise LbtError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise LbtError(f"{name} must be contiguous")
    return t.data_ptr()


def _stream(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


class Path:
    """The five calls of the path for one shape, on caller-owned tensors.

    ``alloc()`` returns a dict of correctly sized device buffers (int32
    tables, bf16 rows stored as int16 bit patterns, fp32 gates/y)."""

    def __init__(self, shape: Shape):
        self.shape = shape
        self.sizes = query_sizes(shape)
        self._c = shape.c()

    def alloc(self, device="cuda", y_bf16=False):
        torch = _torch()
        s, z = self.shape, self.sizes
        i32 = dict(dtype=torch.int32, device=device)
        return {
            "ids": torch.empty(s.N, s.K, **i32),
            "gates": torch.empty(s.N, s.K, dtype=torch.float32, device=device),
            "counts": torch.empty(s.R, s.E, **i32),
            "work": torch.empty(max(1, z["work_words"]), **i32),
            "plan": torch.empty(z["plan_words"], **i32),
            "status": torch.zeros(1, **i32),
            "slot": torch.empty(max(1, z["P"]), **i32),
            "sorted_ids": torch.empty(s.R * z["C"], **i32),
            "block_wrow": torch.empty(s.R, z["n_blocks"], **i32),
            "block_expert": torch.empty(s.R, z["n_blocks"], **i32),
            "recv": torch.empty(s.R * z["C"], s.H, dtype=torch.int16, device=device),
            "y": torch.empty(s.N, s.H, dtype=torch.int16 if y_bf16 else torch.float32,
                             device=device),
        }

    # a1 + a2
    def route_topk(self, logits, ids, gates, counts, work, sel_bias=None, stream=None):
        torch = _torch()
        s, z = self.shape, self.sizes
        rc = lib().lbt_route_topk(
            ctypes.byref(self._c),
            _ptr(logits, torch.float32, s.N * s.E, "logits"),
            _ptr(sel_bias, torch.float32, s.E, "sel_bias"),
            _ptr(ids, torch.int32, s.N * s.K, "ids"),
            _ptr(gates, torch.float32, s.N * s.K, "gates"),
            _ptr(counts, torch.int32, s.R * s.E, "counts"),
            _ptr(work, torch.int32, z["work_words"], "work"),
            _stream(stream))
        _check(rc, "lbt_route_topk")

    def histogram(self, ids, counts, work, status=None, stream=None):
        torch = _torch()
        s, z = self.shape, self.sizes
        rc = lib().lbt_histogram(
            ctypes.byref(self._c),
            _ptr(ids, torch.int32, s.N * s.K, "ids"),
            _ptr(counts, torch.int32, s.R * s.E, "counts"),
            _ptr(work, torch.int32, z["work_words"], "work"),
            _ptr(status, torch.int32, 1, "status"),
            _stream(stream))
        _check(rc, "lbt_histogram")

    # a3
    def plan_balance(self, counts, plan, status=None, stream=None):
        torch = _torch()
        s, z = self.shape, self.sizes
        rc = lib().lbt_plan_balance(
            ctypes.byref(self._c),
            _ptr(counts, torch.int32, s.R * s.E, "counts"),
            _ptr(plan, torch.int32, z["plan_words"], "plan"),
            _ptr(status, torch.int32, 1, "status"),
            _stream(stream))
        _check(rc, "lbt_plan_balance")

    # a1 + a2 + a3 in one call (one launch for small batches)
    def route_plan(self, logits, ids, gates, counts, work, plan, status=None, sel_bias=None,
                   stream=None):
        torch = _torch()
        s, z = self.shape, self.sizes
        rc = lib().lbt_route_plan(
            ctypes.byref(self._c),
            _ptr(logits, torch.float32, s.N * s.E, "logits"),
            _ptr(sel_bias, torch.float32, s.E, "sel_bias"),
            _ptr(ids, torch.int32, s.N * s.K, "ids"),
            _ptr(gates, torch.float32, s.N * s.K, "gates"),
            _ptr(counts, torch.int32, s.R * s.E, "counts"),
            _ptr(work, torch.int32, z["work_words"], "work"),
            _ptr(plan, torch.int32, z["plan_words"], "plan"),
            _ptr(status, torch.int32, 1, "status"),
            _stream(stream))
        _check(rc, "lbt_route_plan")

    # a1 + a2 + a3 + a4 in one call (one launch for small batches)
    def front(self, logits, buf, sel_bias=None, stream=None):
        """Route, histogram, fixed-rule plan and align into the buffers of
        ``alloc()`` (ids, gates, counts, work, plan, slot, sorted_ids,
        block_wrow, block_expert, status)."""
        torch = _torch()
        s, z = self.shape, self.sizes
        rc = lib().lbt_front(
            ctypes.byref(self._c),
            _ptr(logits, torch.float32, s.N * s.E, "logits"),
            _ptr(sel_bias, torch.float32, s.E, "sel_bias"),
            _ptr(buf["ids"], torch.int32, s.N * s.K, "ids"),
            _ptr(buf["gates"], torch.float32, s.N * s.K, "gates"),
            _ptr(buf["counts"], torch.int32, s.R * s.E, "counts"),
            _ptr(buf["work"], torch.int32, z["work_words"], "work"),
            _ptr(buf["plan"], torch.int32, z["plan_words"], "plan"),
            _ptr(buf["slot"], torch.int32, z["P"], "slot"),
            _ptr(buf["sorted_ids"], torch.int32, s.R * z["C"], "sorted_ids"),
            _ptr(buf["block_wrow"], torch.int32, s.R * z["n_blocks"], "block_wrow"),
            _ptr(buf["block_expert"], torch.int32, s.R * z["n_blocks"], "block_expert"),
            _ptr(buf["status"], torch.int32, 1, "status"),
            _stream(stream))
        _check(rc, "lbt_front")

    # a3, quota variant
    def plan_quota(self, counts, plan, status=None, stream=None):
        torch = _torch()
        s, z = self.shape, self.sizes
        rc = lib().lbt_plan_quota(
            ctypes.byref(self._c),
            _ptr(counts, torch.int32, s.R * s.E, "counts"),
            _ptr(plan, torch.int32, z["plan_words"], "plan"),
            _ptr(status, torch.int32, 1, "status"),
            _stream(stream))
        _check(rc, "lbt_plan_quota")

    # a4
    def front_dispatch(self, logits, x, buf, sel_bias=None, stream=None):
        """lbt_front then lbt_dispatch in one call, into the buffers of
        ``alloc()`` (those of front, and recv)."""
        torch = _torch()
        s, z = self.shape, self.sizes
        rc = lib().lbt_front_dispatch(
            ctypes.byref(self._c),
            _ptr(logits, torch.float32, s.N * s.E, "logits"),
            _ptr(sel_bias, torch.float32, s.E, "sel_bias"),
            _ptr(buf["ids"], torch.int32, s.N * s.K, "ids"),
            _ptr(buf["gates"], torch.float32, s.N * s.K, "gates"),
            _ptr(buf["counts"], torch.int32, s.R * s.E, "counts"),
            _ptr(buf["work"], torch.int32, z["work_words"], "work"),
            _ptr(buf["plan"], torch.int32, z["plan_words"], "plan"),
            _ptr(buf["slot"], torch.int32, z["P"], "slot"),
            _ptr(buf["sorted_ids"], torch.int32, s.R * z["C"], "sorted_ids"),
            _ptr(buf["block_wrow"], torch.int32, s.R * z["n_blocks"], "block_wrow"),
            _ptr(buf["block_expert"], torch.int32, s.R * z["n_blocks"], "block_expert"),
            _ptr(x, torch.int16, s.N * s.H, "x", align16=True),
            _ptr(buf["recv"], torch.int16, s.R * z["C"] * s.H, "recv", align16=True),
            _ptr(buf["status"], torch.int32, 1, "status"),
            _stream(stream))
        _check(rc, "lbt_front_dispatch")

    # a4 + a5 in one call
    def align_dispatch(self, ids, work, plan, x, slot, sorted_ids, block_wrow, block_expert,
                       recv, status=None, stream=None):
        torch = _torch()
        s, z = self.shape, self.sizes
        rc = lib().lbt_align_dispatch(
            ctypes.byref(self._c),
            _ptr(ids, torch.int32, s.N * s.K, "ids"),
            _ptr(work, torch.int32, z["work_words"], "work"),
            _ptr(plan, torch.int32, z["plan_words"], "plan"),
            _ptr(x, torch.int16, s.N * s.H, "x", align16=True),
            _ptr(slot, torch.int32, z["P"], "slot"),
            _ptr(sorted_ids, torch.int32, s.R * z["C"], "sorted_ids"),
            _ptr(block_wrow, torch.int32, s.R * z["n_blocks"], "block_wrow"),
            _ptr(block_expert, torch.int32, s.R * z["n_blocks"], "block_expert"),
            _ptr(recv, torch.int16, s.R * z["C"] * s.H, "recv", align16=True),
            _ptr(status, torch.int32, 1, "status"),
            _stream(stream))
        _check(rc, "lbt_align_dispatch")

    def align_sort(self, ids, work, plan, slot, sorted_ids, block_wrow, block_expert,
                   status=None, stream=None):
        torch = _torch()
        s, z = self.shape, self.sizes
        rc = lib().lbt_align_sort(
            ctypes.byref(self._c),
            _ptr(ids, torch.int32, s.N * s.K, "ids"),
            _ptr(work, torch.int32, z["work_words"], "work"),
            _ptr(plan, torch.int32, z["plan_words"], "plan"),
            _ptr(slot, torch.int32, z["P"], "slot"),
            _ptr(sorted_ids, torch.int32, s.R * z["C"], "sorted_ids"),
            _ptr(block_wrow, torch.int32, s.R * z["n_blocks"], "block_wrow"),
            _ptr(block_expert, torch.int32, s.R * z["n_blocks"], "block_expert"),
            _ptr(status, torch.int32, 1, "status"),
            _stream(stream))
        _check(rc, "lbt_align_sort")

    # a2 + a4 with the library's static workspace (no allocation, no work buffer)
    def align_sort_noalloc(self, ids, plan, slot, sorted_ids, block_wrow, block_expert,
                           status=None, stream=None):
        torch = _torch()
        s, z = self.shape, self.sizes
        rc = lib().lbt_align_sort_noalloc(
            ctypes.byref(self._c),
            _ptr(ids, torch.int32, s.N * s.K, "ids"),
            _ptr(plan, torch.int32, z["plan_words"], "plan"),
            _ptr(slot, torch.int32, z["P"], "slot"),
            _ptr(sorted_ids, torch.int32, s.R * z["C"], "sorted_ids"),
            _ptr(block_wrow, torch.int32, s.R * z["n_blocks"], "block_wrow"),
            _ptr(block_expert, torch.int32, s.R * z["n_blocks"], "block_expert"),
            _ptr(status, torch.int32, 1, "status"),
            _stream(stream))
        _check(rc, "lbt_align_sort_noalloc")

    # a5
    def dispatch(self, x, slot, recv, stream=None):
        torch = _torch()
        s, z = self.shape, self.sizes
        rc = lib().lbt_dispatch(
            ctypes.byref(self._c),
            _ptr(x, torch.int16, s.N * s.H, "x", align16=True),
            _ptr(slot, torch.int32, z["P"], "slot"),
            _ptr(recv, torch.int16, s.R * z["C"] * s.H, "recv", align16=True),
            _stream(stream))
        _check(rc, "lbt_dispatch")

    # a6
    def combine(self, out, slot, gates, y, stream=None):
        torch = _torch()
        s, z = self.shape, self.sizes
        y_bf16 = y.dtype == torch.int16
        rc = lib().lbt_combine(
            ctypes.byref(self._c),
            _ptr(out, torch.int16, s.R * z["C"] * s.H, "out", align16=True),
            _ptr(slot, torch.int32, z["P"], "slot"),
            _ptr(gates, torch.float32, s.N * s.K, "gates"),
            Y_BF16 if y_bf16 else Y_F32,
            _ptr(y, torch.int16 if y_bf16 else torch.float32, s.N * s.H, "y", align16=True),
            _stream(stream))
        _check(rc, "lbt_combine")

    # replica weights and gradients (one expert projection per call)
    def prefetch_weights(self, plan, weights, slots, stream=None):
        """weights: [E, ...] tensor of home weight rows; slots: [R, B, ...]
        of the same row size and dtype."""
        torch = _torch()
        s, z = self.shape, self.sizes
        row_bytes = weights[0].numel() * weights.element_size() if weights.shape[0] else 0
        if weights.shape[0] != s.E or (s.B and tuple(slots.shape[:2]) != (s.R, s.B)):
            raise LbtError("prefetch_weights: weights must be [E, ...] and slots [R, B, ...]")
        if slots.numel() * slots.element_size() < s.R * s.B * row_bytes:
            raise LbtError("prefetch_weights: slots too small")
        rc = lib().lbt_prefetch_weights(
            ctypes.byref(self._c), _ptr(plan, torch.int32, z["plan_words"], "plan"),
            _raw(weights, "weights"), _raw(slots, "slots"), row_bytes, _stream(stream))
        _check(rc, "lbt_prefetch_weights")

    def reduce_grad(self, plan, slot_grads, grads, stream=None):
        """slot_grads fp32 [R, B, ...], grads fp32 [E, ...] of the same row size."""
        torch = _torch()
        s, z = self.shape, self.sizes
        row = grads[0].numel() if grads.shape[0] else 0
        if grads.shape[0] != s.E or (s.B and tuple(slot_grads.shape[:2]) != (s.R, s.B)):
            raise LbtError("reduce_grad: grads must be [E, ...] and slot_grads [R, B, ...]")
        rc = lib().lbt_reduce_grad(
            ctypes.byref(self._c), _ptr(plan, torch.int32, z["plan_words"], "plan"),
            _ptr(slot_grads, torch.float32, s.R * s.B * row, "slot_grads"),
            _ptr(grads, torch.float32, s.E * row, "grads"), row, _stream(stream))
        _check(rc, "lbt_reduce_grad")

    # backward of a6 and a5
    def combine_bwd(self, out, slot, gates, dy, d_out, d_gates, stream=None):
        torch = _torch()
        s, z = self.shape, self.sizes
        dy_bf16 = dy.dtype == torch.int16
        rc = lib().lbt_combine_bwd(
            ctypes.byref(self._c),
            _ptr(out, torch.int16, s.R * z["C"] * s.H, "out", align16=True),
            _ptr(slot, torch.int32, z["P"], "slot"),
            _ptr(gates, torch.float32, s.N * s.K, "gates"),
            Y_BF16 if dy_bf16 else Y_F32,
            _ptr(dy, torch.int16 if dy_bf16 else torch.float32, s.N * s.H, "dy", align16=True),
            _ptr(d_out, torch.int16, s.R * z["C"] * s.H, "d_out", align16=True),
            _ptr(d_gates, torch.float32, s.N * s.K, "d_gates"),
            _stream(stream))
        _check(rc, "lbt_combine_bwd")

    def dispatch_bwd(self, d_recv, slot, dx, stream=None):
        torch = _torch()
        s, z = self.shape, self.sizes
        dx_bf16 = dx.dtype == torch.int16
        rc = lib().lbt_dispatch_bwd(
            ctypes.byref(self._c),
            _ptr(d_recv, torch.int16, s.R * z["C"] * s.H, "d_recv", align16=True),
            _ptr(slot, torch.int32, z["P"], "slot"),
            Y_BF16 if dx_bf16 else Y_F32,
            _ptr(dx, torch.int16 if dx_bf16 else torch.float32, s.N * s.H, "dx", align16=True),
            _stream(stream))
        _check(rc, "lbt_dispatch_bwd")

    def step(self, logits, x, buf, sel_bias=None, out=None, stream=None, planner="fixed"):
        """One pass of the whole path; ``out`` defaults to recv (identity
        expert); ``planner`` is "fixed" (route, plan, align and dispatch in
        one lbt_front_dispatch call) or "quota" (lbt_route_topk,
        lbt_plan_quota, lbt_align_dispatch); then lbt_combine.  Returns
        nothing; results land in ``buf``."""
        if planner not in ("fixed", "quota"):
            raise LbtError(f"unknown planner {planner!r}")
        if planner == "fixed":
            self.front_dispatch(logits, x, buf, sel_bias=sel_bias, stream=stream)
        else:
            self.route_topk(logits, buf["ids"], buf["gates"], buf["counts"], buf["work"],
                            sel_bias=sel_bias, stream=stream)
            self.plan_quota(buf["counts"], buf["plan"], buf["status"], stream=stream)
            self.align_dispatch(buf["ids"], buf["work"], buf["plan"], x, buf["slot"],
                                buf["sorted_ids"], buf["block_wrow"], buf["block_expert"],
                                buf["recv"], buf["status"], stream=stream)
        self.combine(buf["recv"] if out is None else out, buf["slot"], buf["gates"], buf["y"],
                     stream=stream)

    def recv_views(self, recv, n_rows_padded, zero_copy=True):
        """Per-rank views recv[r, :n_rows_padded[r]] of the static buffer;
        ``n_rows_padded`` is a host sequence.  Zero-copy views are
        overwritten by the next dispatch into ``recv`` and must not be kept
        past it (autograd must not save them); zero_copy=False returns
        clones that may be kept ([MoonEP-GR] "Ένα ρεαλιστικό πλαίσιο
        αξιολόγησης": views are replaced by the next dispatch or combine)."""
        C = self.sizes["C"]
        views = [recv[r * C: r * C + int(n)] for r, n in enumerate(n_rows_padded)]
        return views if zero_copy else [v.clone() for v in views]


# --------------------------------------------------------------------------- plan blob
def plan_fields(plan_words, sizes: dict, R: int, E: int) -> dict:
    """Named views (numpy) of a plan blob copied to the host."""
    p = np.asarray(plan_words, dtype=np.int32)
    z = sizes
    ms, mp = z["max_seg"], z["max_pieces"]

    def at(key, n, shape=None):
        a = p[z[key]: z[key] + n]
        return a.reshape(shape) if shape else a

    return {
        "hdr": at("off_hdr", 16),
        "T": at("off_T", E), "h": at("off_h", E), "O": at("off_O", E),
        "home_row": at("off_home_row", E),
        "L": at("off_L", R), "def": at("off_def", R), "D": at("off_D", R + 1),
        "n_seg": at("off_n_seg", R), "n_rows_padded": at("off_n_rows_padded", R),
        "n_slots": at("off_n_slots", R), "n_remote": at("off_n_remote", R),
        "seg_expert": at("off_seg_expert", R * ms, (R, ms)),
        "seg_wrow": at("off_seg_wrow", R * ms, (R, ms)),
        "seg_count": at("off_seg_count", R * ms, (R, ms)),
        "seg_start": at("off_seg_start", R * (ms + 1), (R, ms + 1)),
        "piece_expert": at("off_piece_expert", mp), "piece_rank": at("off_piece_rank", mp),
        "piece_count": at("off_piece_count", mp), "piece_line": at("off_piece_line", mp),
        "piece_row": at("off_piece_row", mp), "piece_wrow": at("off_piece_wrow", mp),
        "home_local": at("off_home_local", E), "piece_local": at("off_piece_local", mp),
    }
