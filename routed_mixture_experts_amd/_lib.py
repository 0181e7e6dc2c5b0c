"""ctypes binding of libmoe.so (include/moe.h).

Argument marshalling only: every step runs in the HIP library.  PyTorch
provides device memory (output tensors are allocated with torch) and the
current HIP stream.  Importing this module never falls back to anything: if
the library is missing, every call raises.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe.so")

MOE_OK, MOE_EINVAL, MOE_ENOTSUP, MOE_ENOSPACE, MOE_EHIP = range(5)
MOE_DTYPE_F32, MOE_DTYPE_BF16 = 0, 1
SCORES = {"softmax": 0, "sigmoid": 1, "sqrtsoftplus": 2}
GROUP_SCORES = {"max": 0, "top2sum": 1}
STAGES = ["router", "downproj", "route", "permute", "gemm1", "gemm2", "combine", "shared", "tail"]
MOE_NUM_STAGES = len(STAGES)

MOE_WEIGHT_DTYPE, MOE_WEIGHT_FP8_E4M3, MOE_WEIGHT_MXFP4 = 0, 1, 2
ACTIVATIONS = {"silu": 0, "gelu": 1, "gelu_tanh": 2, "swiglu_clip": 3}

EXPORTS = ["moe_route", "moe_permute_workspace", "moe_permute", "moe_experts_workspace",
           "moe_experts", "moe_combine", "moe_forward_workspace", "moe_forward",
           "moe_experts_ex", "moe_forward_ex", "moe_forward_workspace_ex", "moe_log2phy",
           "moe_load_accumulate", "moe_forward_noalloc", "moe_status_string"]
MOE_NOALLOC_SCRATCH_BYTES = 64 << 20


class moe_route_cfg_t(ctypes.Structure):
    _fields_ = [("num_experts", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("num_groups", ctypes.c_int32), ("topk_group", ctypes.c_int32),
                ("score", ctypes.c_int32), ("group_score", ctypes.c_int32),
                ("renormalize", ctypes.c_int32), ("routed_scaling", ctypes.c_float)]


class moe_latent_t(ctypes.Structure):
    _fields_ = [("w_down", ctypes.c_void_p), ("gamma", ctypes.c_void_p),
                ("w_up", ctypes.c_void_p), ("latent", ctypes.c_int32),
                ("rms_eps", ctypes.c_float)]


class moe_shared_t(ctypes.Structure):
    _fields_ = [("w13", ctypes.c_void_p), ("w2", ctypes.c_void_p), ("inter", ctypes.c_int32)]


class moe_expert_weights_t(ctypes.Structure):
    _fields_ = [("format", ctypes.c_int32), ("w13", ctypes.c_void_p), ("w2", ctypes.c_void_p),
                ("w13_scale", ctypes.c_void_p), ("w2_scale", ctypes.c_void_p),
                ("activation", ctypes.c_int32), ("act_alpha", ctypes.c_float),
                ("act_limit", ctypes.c_float)]


class moe_placement_t(ctypes.Structure):
    _fields_ = [("num_physical", ctypes.c_int32), ("log2phy", ctypes.c_void_p),
                ("load", ctypes.c_void_p)]


class MoeError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


@dataclass(frozen=True)
class RouteConfig:
    """Routing settings (num_experts, top_k, grouped top-k, score, ...)."""

    num_experts: int
    top_k: int
    num_groups: int = 1
    topk_group: int = 1
    score: str = "softmax"
    group_score: str = "max"
    renormalize: bool = True
    routed_scaling: float = 1.0

    def c(self) -> moe_route_cfg_t:
        return moe_route_cfg_t(self.num_experts, self.top_k, self.num_groups, self.topk_group,
                               SCORES[self.score], GROUP_SCORES[self.group_score],
                               int(bool(self.renormalize)), float(self.routed_scaling))


_lib = None

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32
_SZ = ctypes.c_size_t


def load() -> ctypes.CDLL:
    """Load libmoe.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it first "
                           "(python -m routed_mixture_experts_amd.build)")
    lib = ctypes.CDLL(LIB_PATH)
    lib.moe_status_string.restype = ctypes.c_char_p
    lib.moe_status_string.argtypes = [_I32]
    lib.moe_route.restype = _I32
    lib.moe_route.argtypes = [ctypes.POINTER(moe_route_cfg_t), _I64, _P, _P, _P, _P, _P]
    lib.moe_permute_workspace.restype = _SZ
    lib.moe_permute_workspace.argtypes = [_I64, _I32, _I32]
    lib.moe_permute.restype = _I32
    lib.moe_permute.argtypes = [_I64, _I32, _I32, _P, _P, _P, _P, _P, _P, _SZ, _P]
    lib.moe_experts_workspace.restype = _SZ
    lib.moe_experts_workspace.argtypes = [_I32, _I64, _I32, _I32, _I32, _I32]
    lib.moe_experts.restype = _I32
    lib.moe_experts.argtypes = [_I32, _I64, _I32, _I32, _I32, _I32, _P, _P, _P, _P, _P, _P, _P,
                                _SZ, _P]
    lib.moe_combine.restype = _I32
    lib.moe_combine.argtypes = [_I32, _I64, _I32, _I32, _P, _P, _P, _P, _P]
    lib.moe_forward_workspace.restype = _SZ
    lib.moe_forward_workspace.argtypes = [ctypes.POINTER(moe_route_cfg_t), _I32, _I64, _I32,
                                          _I32, ctypes.POINTER(moe_latent_t),
                                          ctypes.POINTER(moe_shared_t)]
    lib.moe_experts_ex.restype = _I32
    lib.moe_experts_ex.argtypes = [_I32, _I64, _I32, _I32, _I32, _I32, _P, _P, _P,
                                   ctypes.POINTER(moe_expert_weights_t), _P, _P, _SZ, _P]
    lib.moe_forward_ex.restype = _I32
    lib.moe_forward_ex.argtypes = [ctypes.POINTER(moe_route_cfg_t), _I32, _I64, _I32, _I32, _P,
                                   _P, _P, _P, _P, ctypes.POINTER(moe_expert_weights_t),
                                   ctypes.POINTER(moe_placement_t),
                                   ctypes.POINTER(moe_latent_t), ctypes.POINTER(moe_shared_t),
                                   _P, _P, _P, _P, _P, _P, _P, _SZ, _P]
    lib.moe_forward_workspace_ex.restype = _SZ
    lib.moe_forward_workspace_ex.argtypes = [ctypes.POINTER(moe_route_cfg_t), _I32, _I64, _I32,
                                             _I32, ctypes.POINTER(moe_latent_t),
                                             ctypes.POINTER(moe_shared_t),
                                             ctypes.POINTER(moe_placement_t)]
    lib.moe_log2phy.restype = _I32
    lib.moe_log2phy.argtypes = [_I64, _I32, _I32, _I32, _P, _P, _P, _P]
    lib.moe_load_accumulate.restype = _I32
    lib.moe_load_accumulate.argtypes = [_I32, _P, _P, _P]
    lib.moe_forward_noalloc.restype = _I32
    lib.moe_forward_noalloc.argtypes = [ctypes.POINTER(moe_route_cfg_t), _I32, _I64, _I32, _I32,
                                        _P, _P, _P, _P, _P,
                                        ctypes.POINTER(moe_expert_weights_t),
                                        ctypes.POINTER(moe_placement_t),
                                        ctypes.POINTER(moe_latent_t),
                                        ctypes.POINTER(moe_shared_t), _P, _P, _P, _P, _P, _P]
    lib.moe_forward.restype = _I32
    lib.moe_forward.argtypes = [ctypes.POINTER(moe_route_cfg_t), _I32, _I64, _I32, _I32, _P, _P,
                                _P, _P, _P, _P, _P, ctypes.POINTER(moe_latent_t),
                                ctypes.POINTER(moe_shared_t), _P, _P, _P, _P, _P, _P, _P, _SZ,
                                _P]
    _lib = lib
    return lib


_library = load  # the loader, for functions whose arguments shadow its name


def _check(st: int):
    if st != MOE_OK:
        raise MoeError(st, load().moe_status_string(st).decode())


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors passed to the HIP library must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors passed to the HIP library must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.float32:
        return MOE_DTYPE_F32
    if dt == torch.bfloat16:
        return MOE_DTYPE_BF16
    raise ValueError(f"unsupported dtype {dt}")


def _need(t: Optional[torch.Tensor], dtype: torch.dtype, name: str):
    if t is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")


# ----------------------------------------------------------------- calls ---

def moe_route(cfg: RouteConfig, logits: torch.Tensor, correction_bias=None,
              topk_ids=None, topk_weights=None):
    """Scoring, grouped top-k, renormalisation, routed scaling -> (ids, weights)."""
    lib = load()
    T = logits.shape[0]
    _need(logits, torch.float32, "logits")
    _need(correction_bias, torch.float32, "correction_bias")
    if topk_ids is None:
        topk_ids = torch.empty((T, cfg.top_k), dtype=torch.int32, device=logits.device)
    if topk_weights is None:
        topk_weights = torch.empty((T, cfg.top_k), dtype=torch.float32, device=logits.device)
    c = cfg.c()
    _check(lib.moe_route(ctypes.byref(c), T, _ptr(logits), _ptr(correction_bias),
                         _ptr(topk_ids), _ptr(topk_weights), _stream()))
    return topk_ids, topk_weights


def moe_permute(topk_ids: torch.Tensor, num_experts: int, workspace=None):
    """-> (counts[E], offsets[E+1], row_to_pair[P], pair_to_row[P]), all int32."""
    lib = load()
    T, k = topk_ids.shape
    _need(topk_ids, torch.int32, "topk_ids")
    dev = topk_ids.device
    counts = torch.empty(num_experts, dtype=torch.int32, device=dev)
    offsets = torch.empty(num_experts + 1, dtype=torch.int32, device=dev)
    r2p = torch.empty(T * k, dtype=torch.int32, device=dev)
    p2r = torch.empty(T * k, dtype=torch.int32, device=dev)
    nbytes = lib.moe_permute_workspace(T, k, num_experts)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    _check(lib.moe_permute(T, k, num_experts, _ptr(topk_ids), _ptr(counts), _ptr(offsets),
                           _ptr(r2p), _ptr(p2r), _ptr(workspace), workspace.numel(), _stream()))
    return counts, offsets, r2p, p2r


def moe_experts(x: torch.Tensor, expert_offsets: torch.Tensor, row_to_pair: torch.Tensor,
                w13: torch.Tensor, w2: torch.Tensor, top_k: int, y_rows=None, workspace=None):
    """Grouped gate/up + SwiGLU and down over expert-sorted rows -> y_rows[P, D] f32."""
    lib = load()
    T, D = x.shape
    E, twoI, D2 = w13.shape
    I = twoI // 2
    if D2 != D or tuple(w2.shape) != (E, D, I):
        raise ValueError("w13 must be [E, 2I, D] and w2 [E, D, I]")
    _need(w13, x.dtype, "w13")
    _need(w2, x.dtype, "w2")
    _need(expert_offsets, torch.int32, "expert_offsets")
    _need(row_to_pair, torch.int32, "row_to_pair")
    dt = _dtype_code(x.dtype)
    if y_rows is None:
        y_rows = torch.empty((T * top_k, D), dtype=torch.float32, device=x.device)
    nbytes = lib.moe_experts_workspace(dt, T, top_k, E, D, I)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=x.device)
    _check(lib.moe_experts(dt, T, top_k, E, D, I, _ptr(x), _ptr(expert_offsets),
                           _ptr(row_to_pair), _ptr(w13), _ptr(w2), _ptr(y_rows),
                           _ptr(workspace), workspace.numel(), _stream()))
    return y_rows


class ExpertWeights:
    """Routed expert weights for moe_experts_ex / moe_forward_ex.

    ``ExpertWeights(w13, w2)``: weights in the layer dtype.
    ``ExpertWeights.fp8(w13, w2, w13_scale, w2_scale)``: OCP e4m3 codes
    (torch.uint8 or torch.float8_e4m3fn) [E, 2I, D] / [E, D, I] with one fp32
    scale per weight row, [E, 2I] / [E, D].
    ``ExpertWeights.mxfp4(w13, w2, w13_scale, w2_scale)``: OCP MXFP4, uint8
    [E, 2I, D/2] / [E, D, I/2] E2M1 code pairs (even element in the low
    nibble) with one uint8 E8M0 exponent per 32 elements of a row,
    [E, 2I, D/32] / [E, D, I/32].
    ``activation``: "silu" (SwiGLU, default), "gelu", "gelu_tanh" or
    "swiglu_clip" (with ``alpha`` and ``limit``)."""

    def __init__(self, w13: torch.Tensor, w2: torch.Tensor, w13_scale=None, w2_scale=None,
                 fmt: int = MOE_WEIGHT_DTYPE, activation: str = "silu", alpha: float = 1.702,
                 limit: float = 7.0):
        self.w13, self.w2 = w13, w2
        self.w13_scale, self.w2_scale = w13_scale, w2_scale
        self.format = fmt
        if activation not in ACTIVATIONS:
            raise ValueError(f"activation must be one of {sorted(ACTIVATIONS)}")
        self.activation, self.alpha, self.limit = activation, float(alpha), float(limit)
        E, twoI, D = w13.shape
        if fmt == MOE_WEIGHT_MXFP4:
            D = 2 * D  # two codes per byte
        self.E, self.I, self.D = E, twoI // 2, D
        if fmt == MOE_WEIGHT_MXFP4:
            if tuple(w2.shape) != (E, D, self.I // 2):
                raise ValueError("MXFP4 w13 must be [E, 2I, D/2] and w2 [E, D, I/2]")
            for name, t in (("w13", w13), ("w2", w2)):
                if t.dtype != torch.uint8 or not t.is_contiguous():
                    raise ValueError(f"{name} must be contiguous uint8 code pairs")
            if w13_scale is None or w2_scale is None:
                raise ValueError("MXFP4 weights need w13_scale and w2_scale")
            _need(w13_scale, torch.uint8, "w13_scale")
            _need(w2_scale, torch.uint8, "w2_scale")
            if (tuple(w13_scale.shape) != (E, 2 * self.I, D // 32)
                    or tuple(w2_scale.shape) != (E, D, self.I // 32)):
                raise ValueError("w13_scale must be [E, 2I, D/32] and w2_scale [E, D, I/32]")
        elif tuple(w2.shape) != (E, D, self.I):
            raise ValueError("w13 must be [E, 2I, D] and w2 [E, D, I]")
        if fmt == MOE_WEIGHT_FP8_E4M3:
            for name, t in (("w13", w13), ("w2", w2)):
                if t.dtype not in (torch.uint8, torch.float8_e4m3fn) or not t.is_contiguous():
                    raise ValueError(f"{name} must be contiguous uint8 / float8_e4m3fn codes")
            _need(w13_scale, torch.float32, "w13_scale")
            _need(w2_scale, torch.float32, "w2_scale")
            if w13_scale is None or w2_scale is None:
                raise ValueError("FP8 weights need w13_scale and w2_scale")
            if tuple(w13_scale.shape) != (E, 2 * self.I) or tuple(w2_scale.shape) != (E, D):
                raise ValueError("w13_scale must be [E, 2I] and w2_scale [E, D]")

    @classmethod
    def fp8(cls, w13, w2, w13_scale, w2_scale, **act) -> "ExpertWeights":
        return cls(w13, w2, w13_scale, w2_scale, MOE_WEIGHT_FP8_E4M3, **act)

    @classmethod
    def mxfp4(cls, w13, w2, w13_scale, w2_scale, **act) -> "ExpertWeights":
        return cls(w13, w2, w13_scale, w2_scale, MOE_WEIGHT_MXFP4, **act)

    def c(self) -> moe_expert_weights_t:
        return moe_expert_weights_t(self.format, _ptr(self.w13), _ptr(self.w2),
                                    _ptr(self.w13_scale), _ptr(self.w2_scale),
                                    ACTIVATIONS[self.activation], self.alpha, self.limit)

    def check_dtype(self, dtype: torch.dtype):
        if self.format == MOE_WEIGHT_DTYPE:
            _need(self.w13, dtype, "w13")
            _need(self.w2, dtype, "w2")


def moe_experts_ex(x: torch.Tensor, expert_offsets: torch.Tensor, row_to_pair: torch.Tensor,
                   weights: ExpertWeights, top_k: int, y_rows=None, workspace=None):
    """moe_experts with the weights described by an ExpertWeights."""
    lib = load()
    T, D = x.shape
    if weights.D != D:
        raise ValueError("weights do not match x's width")
    weights.check_dtype(x.dtype)
    _need(expert_offsets, torch.int32, "expert_offsets")
    _need(row_to_pair, torch.int32, "row_to_pair")
    dt = _dtype_code(x.dtype)
    E, I = weights.E, weights.I
    if y_rows is None:
        y_rows = torch.empty((T * top_k, D), dtype=torch.float32, device=x.device)
    nbytes = lib.moe_experts_workspace(dt, T, top_k, E, D, I)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=x.device)
    wc = weights.c()
    _check(lib.moe_experts_ex(dt, T, top_k, E, D, I, _ptr(x), _ptr(expert_offsets),
                              _ptr(row_to_pair), ctypes.byref(wc), _ptr(y_rows),
                              _ptr(workspace), workspace.numel(), _stream()))
    return y_rows


class Placement:
    """Logical -> physical expert placement for moe_forward_ex.

    ``log2phy``: int32 [num_experts], the physical slot of each logical
    expert; ``num_physical``: slots (the expert weights are laid out by slot);
    ``load``: optional int64 [num_physical] that accumulates the tokens sent
    to each slot, once per call."""

    def __init__(self, log2phy: torch.Tensor, num_physical: int, load=None):
        _need(log2phy, torch.int32, "log2phy")
        _need(load, torch.int64, "load")
        if load is not None and load.numel() != num_physical:
            raise ValueError("load must have num_physical entries")
        self.log2phy, self.num_physical, self.load = log2phy, int(num_physical), load

    def c(self) -> moe_placement_t:
        return moe_placement_t(self.num_physical, _ptr(self.log2phy), _ptr(self.load))


def moe_log2phy(topk_ids: torch.Tensor, log2phy: torch.Tensor, num_physical: int, out=None):
    """phys_ids[t, j] = log2phy[topk_ids[t, j]] (int32, same shape)."""
    lib = load()
    _need(topk_ids, torch.int32, "topk_ids")
    _need(log2phy, torch.int32, "log2phy")
    T, k = topk_ids.shape
    if out is None:
        out = torch.empty_like(topk_ids)
    _check(lib.moe_log2phy(T, k, log2phy.numel(), num_physical, _ptr(log2phy), _ptr(topk_ids),
                           _ptr(out), _stream()))
    return out


def moe_load_accumulate(counts: torch.Tensor, load: torch.Tensor):
    """load += counts (int32 counts into an int64 accumulator, on the stream)."""
    lib = _library()
    _need(counts, torch.int32, "counts")
    _need(load, torch.int64, "load")
    if counts.numel() != load.numel():
        raise ValueError("counts and load differ in length")
    _check(lib.moe_load_accumulate(counts.numel(), _ptr(counts), _ptr(load), _stream()))
    return load


def moe_combine(y_rows: torch.Tensor, pair_to_row: torch.Tensor, topk_weights: torch.Tensor,
                out_dtype: torch.dtype = torch.bfloat16, out=None):
    """out[t] = sum_j w[t,j] * y_rows[pair_to_row[t*k+j]] (fp32 sum, one rounding)."""
    lib = load()
    T, k = topk_weights.shape
    D = y_rows.shape[1]
    _need(y_rows, torch.float32, "y_rows")
    _need(pair_to_row, torch.int32, "pair_to_row")
    _need(topk_weights, torch.float32, "topk_weights")
    if out is None:
        out = torch.empty((T, D), dtype=out_dtype, device=y_rows.device)
    _check(lib.moe_combine(_dtype_code(out.dtype), T, k, D, _ptr(y_rows), _ptr(pair_to_row),
                           _ptr(topk_weights), _ptr(out), _stream()))
    return out


def _latent_struct(latent: Optional[dict]):
    if latent is None:
        return None
    return moe_latent_t(_ptr(latent["w_down"]), _ptr(latent["gamma"]), _ptr(latent["w_up"]),
                        latent["w_down"].shape[0], float(latent.get("eps", 1e-6)))


def _shared_struct(shared: Optional[dict]):
    if shared is None:
        return None
    return moe_shared_t(_ptr(shared["w13"]), _ptr(shared["w2"]), shared["w2"].shape[1])


def moe_forward_workspace(cfg: RouteConfig, dtype: torch.dtype, max_T: int, H: int, I: int,
                          latent=None, shared=None) -> int:
    lib = load()
    c = cfg.c()
    lat = _latent_struct(latent)
    sh = _shared_struct(shared)
    return lib.moe_forward_workspace(ctypes.byref(c), _dtype_code(dtype), max_T, H, I,
                                     ctypes.byref(lat) if lat else None,
                                     ctypes.byref(sh) if sh else None)


def _forward(cfg, x, I, experts, w_router, router_bias, router_logits, correction_bias,
             latent, shared, out, logits_out, topk_ids_out, topk_weights_out,
             expert_counts_out, stage_events, workspace, stream, placement=None):
    lib = load()
    T, H = x.shape
    dt = _dtype_code(x.dtype)
    _need(w_router, x.dtype, "w_router")
    for name, t in (("router_bias", router_bias), ("router_logits", router_logits),
                    ("correction_bias", correction_bias)):
        _need(t, torch.float32, name)
    c = cfg.c()
    lat = _latent_struct(latent)
    sh = _shared_struct(shared)
    pl = placement.c() if placement is not None else None
    nbytes = lib.moe_forward_workspace_ex(ctypes.byref(c), dt, T, H, I,
                                          ctypes.byref(lat) if lat else None,
                                          ctypes.byref(sh) if sh else None,
                                          ctypes.byref(pl) if pl else None)
    if nbytes == 0:
        raise MoeError(MOE_EINVAL, "moe_forward_workspace rejected the shapes")
    # Buffers made here belong to the stream the layer runs on: torch's
    # caching allocator then hands their blocks to no other stream while the
    # layer's kernels (on `stream`, and on the side stream joined back into
    # it) may still use them.
    with torch.cuda.stream(stream) if stream is not None else contextlib.nullcontext():
        if out is None:
            out = torch.empty((T, H), dtype=x.dtype, device=x.device)
        if workspace is None:
            workspace = torch.empty(nbytes, dtype=torch.uint8, device=x.device)
    ev = None
    if stage_events is not None:
        if len(stage_events) != 2 * MOE_NUM_STAGES:
            raise ValueError("stage_events needs 2*MOE_NUM_STAGES events")
        ev = (ctypes.c_void_p * len(stage_events))(*[e.cuda_event for e in stage_events])
    common = (ctypes.byref(lat) if lat else None, ctypes.byref(sh) if sh else None, _ptr(out),
              _ptr(logits_out), _ptr(topk_ids_out), _ptr(topk_weights_out),
              _ptr(expert_counts_out), ev, _ptr(workspace), workspace.numel(), _stream(stream))
    head = (ctypes.byref(c), dt, T, H, I, _ptr(x), _ptr(w_router), _ptr(router_bias),
            _ptr(router_logits), _ptr(correction_bias))
    if isinstance(experts, ExpertWeights):
        wc = experts.c()
        _check(lib.moe_forward_ex(*head, ctypes.byref(wc), ctypes.byref(pl) if pl else None,
                                  *common))
    else:
        w13, w2 = experts
        _check(lib.moe_forward(*head, _ptr(w13), _ptr(w2), *common))
    return out


def moe_forward(cfg: RouteConfig, x: torch.Tensor, w13: torch.Tensor, w2: torch.Tensor, *,
                w_router=None, router_bias=None, router_logits=None, correction_bias=None,
                latent: Optional[dict] = None, shared: Optional[dict] = None, out=None,
                logits_out=None, topk_ids_out=None, topk_weights_out=None,
                expert_counts_out=None, stage_events=None, workspace=None, stream=None):
    """The whole layer on one stream.  ``latent`` = dict(w_down, gamma, w_up, eps);
    ``shared`` = dict(w13, w2).  ``stage_events``: list of 2*MOE_NUM_STAGES
    recorded torch.cuda.Event objects (start/end per stage) or None."""
    _need(w13, x.dtype, "w13")
    _need(w2, x.dtype, "w2")
    return _forward(cfg, x, w2.shape[2], (w13, w2), w_router, router_bias, router_logits,
                    correction_bias, latent, shared, out, logits_out, topk_ids_out,
                    topk_weights_out, expert_counts_out, stage_events, workspace, stream)


def moe_forward_ex(cfg: RouteConfig, x: torch.Tensor, experts: ExpertWeights, *,
                   w_router=None, router_bias=None, router_logits=None, correction_bias=None,
                   latent: Optional[dict] = None, shared: Optional[dict] = None, out=None,
                   logits_out=None, topk_ids_out=None, topk_weights_out=None,
                   expert_counts_out=None, stage_events=None, workspace=None, stream=None,
                   placement: Optional[Placement] = None):
    """moe_forward with the routed experts given as an ExpertWeights, and an
    optional logical -> physical Placement (the weights are then laid out by
    physical slot; topk_ids_out stays logical, expert_counts_out is per slot)."""
    experts.check_dtype(x.dtype)
    return _forward(cfg, x, experts.I, experts, w_router, router_bias, router_logits,
                    correction_bias, latent, shared, out, logits_out, topk_ids_out,
                    topk_weights_out, expert_counts_out, stage_events, workspace, stream,
                    placement)


def moe_forward_noalloc(cfg: RouteConfig, x: torch.Tensor, experts: ExpertWeights,
                        out: torch.Tensor, *, w_router=None, router_bias=None,
                        router_logits=None, correction_bias=None, latent: Optional[dict] = None,
                        shared: Optional[dict] = None, logits_out=None, topk_ids_out=None,
                        topk_weights_out=None, expert_counts_out=None, stream=None,
                        placement: Optional[Placement] = None):
    """moe_forward_ex with no workspace: the library's fixed device scratch
    array (MOE_NOALLOC_SCRATCH_BYTES per GPU) holds the intermediates.  Nothing
    is allocated here either: the caller passes ``out`` and any optional
    outputs.  Calls that overlap in time on one GPU race on the array."""
    lib = load()
    T, H = x.shape
    experts.check_dtype(x.dtype)
    _need(w_router, x.dtype, "w_router")
    _need(out, x.dtype, "out")
    for name, t in (("router_bias", router_bias), ("router_logits", router_logits),
                    ("correction_bias", correction_bias)):
        _need(t, torch.float32, name)
    if tuple(out.shape) != (T, H):
        raise ValueError("out must be [T, H]")
    c = cfg.c()
    lat = _latent_struct(latent)
    sh = _shared_struct(shared)
    pl = placement.c() if placement is not None else None
    wc = experts.c()
    _check(lib.moe_forward_noalloc(
        ctypes.byref(c), _dtype_code(x.dtype), T, H, experts.I, _ptr(x), _ptr(w_router),
        _ptr(router_bias), _ptr(router_logits), _ptr(correction_bias), ctypes.byref(wc),
        ctypes.byref(pl) if pl else None, ctypes.byref(lat) if lat else None,
        ctypes.byref(sh) if sh else None, _ptr(out), _ptr(logits_out), _ptr(topk_ids_out),
        _ptr(topk_weights_out), _ptr(expert_counts_out), _stream(stream)))
    return out
