"""Python binding of libqgalore.so (ctypes): argument marshalling only.

Every step of the optimizer runs in the library's gfx950 kernels; this module checks dtypes,
shapes and devices of torch tensors, passes their device pointers and the current HIP stream
across the C ABI, and turns status codes into exceptions. There is no fallback: if the
library is missing, loading it raises.
"""
from __future__ import annotations

import ctypes
import dataclasses
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqgalore.so")

GROUP = 256

c_int64, c_uint32, c_int32, c_float, c_void_p, c_size_t, c_uint64 = (
    ctypes.c_int64, ctypes.c_uint32, ctypes.c_int32, ctypes.c_float, ctypes.c_void_p,
    ctypes.c_size_t, ctypes.c_uint64)

STATUS = {0: "QG_OK", 1: "QG_ERR_NULL", 2: "QG_ERR_SHAPE", 3: "QG_ERR_ALIGN",
          4: "QG_ERR_WORKSPACE", 5: "QG_ERR_ARG", 6: "QG_ERR_HIP", 7: "QG_ERR_NO_DEVICE"}


class LayerDesc(ctypes.Structure):
    _fields_ = [("m", c_int64), ("n", c_int64), ("r", c_int64), ("layer_id", c_uint32),
                ("lr", c_float), ("beta1", c_float), ("beta2", c_float), ("eps", c_float),
                ("alpha", c_float), ("M_scale", c_void_p), ("V_scale", c_void_p),
                ("R_out", c_void_p), ("U_out", c_void_p), ("workspace", c_void_p),
                ("workspace_bytes", c_size_t), ("stream", c_void_p), ("p_format", c_int32),
                ("dequant_mode", c_int32)]


class Layer(ctypes.Structure):
    _fields_ = [("desc", LayerDesc), ("G", c_void_p), ("W_q", c_void_p), ("W_scale", c_void_p),
                ("P_q", c_void_p), ("P_scale", c_void_p), ("M_q", c_void_p), ("V_q", c_void_p)]


class Proj(ctypes.Structure):
    _fields_ = [("m", c_int64), ("r", c_int64), ("q", c_void_p), ("scale", c_void_p),
                ("format", c_int32)]


# projection storage formats (qg_p_format)
P_FORMATS = {"int4": 0, "int8": 1, "bf16": 2}
# where an INT4 projection is dequantized (qg_dequant_mode)
DEQUANT_MODES = {"auto": 0, "inline": 1, "pass": 2}


class Sched(ctypes.Structure):
    _fields_ = [("delta", c_int64), ("next_refresh", c_int64), ("count", c_int64),
                ("gamma", c_float), ("last_cossim", c_float)]


EXPORTS = {
    "qgalore_workspace_bytes": (c_size_t, [c_int64, c_int64, c_int64]),
    "qgalore_layer_workspace_bytes": (c_size_t, [ctypes.POINTER(LayerDesc)]),
    "qgalore_step": (c_int32, [ctypes.POINTER(LayerDesc), c_void_p, c_void_p, c_void_p, c_void_p,
                               c_void_p, c_void_p, c_void_p, c_int64, c_uint64]),
    "qgalore_step_noalloc": (c_int32, [ctypes.POINTER(LayerDesc), c_void_p, c_void_p, c_void_p,
                                       c_void_p, c_void_p, c_void_p, c_void_p, c_int64, c_uint64]),
    "qgalore_plan_create": (c_int32, [ctypes.POINTER(Layer), c_int32, ctypes.POINTER(c_void_p)]),
    "qgalore_plan_workspace_bytes": (c_size_t, [c_void_p]),
    "qgalore_plan_step": (c_int32, [c_void_p, c_int64, c_uint64, c_void_p, c_size_t, c_void_p]),
    "qgalore_plan_destroy": (c_int32, [c_void_p]),
    "qgalore_plan_enable_timing": (c_int32, [c_void_p, c_int32]),
    "qgalore_plan_cache_proj": (c_int32, [c_void_p, c_int32]),
    "qgalore_plan_proj_changed": (c_int32, [c_void_p, c_int32]),
    "qgalore_plan_kernel_times": (c_int32, [c_void_p, ctypes.POINTER(c_float),
                                           ctypes.POINTER(c_int32)]),
    "qgalore_cossim_workspace_bytes": (c_size_t, [c_int64, c_int64]),
    "qgalore_cossim_async": (c_int32, [ctypes.POINTER(Proj), ctypes.POINTER(Proj), c_void_p,
                                       c_size_t, c_void_p, c_void_p]),
    "qgalore_cossim_batch_workspace_bytes": (c_size_t, [c_int64, c_int32]),
    "qgalore_cossim_batch": (c_int32, [ctypes.POINTER(Proj), ctypes.POINTER(Proj), c_int32,
                                       c_void_p, c_size_t, c_void_p, c_void_p]),
    "qgalore_cossim": (c_int32, [ctypes.POINTER(Proj), ctypes.POINTER(Proj), c_void_p, c_size_t,
                                 c_void_p, ctypes.POINTER(c_float)]),
    "qgalore_quantize_proj": (c_int32, [c_void_p, c_int64, c_int64, c_void_p, c_void_p, c_void_p]),
    "qgalore_quantize_proj_int8": (c_int32, [c_void_p, c_int64, c_int64, c_void_p, c_void_p,
                                             c_void_p]),
    "qgalore_refresh_workspace_bytes": (c_size_t, [c_int64, c_int64, c_int64, c_int32]),
    "qgalore_refresh_proj": (c_int32, [c_void_p, c_int64, c_int64, c_int64, c_void_p, c_int32,
                                       c_int32, c_void_p, c_void_p, c_void_p, c_void_p,
                                       c_void_p, c_size_t, c_void_p]),
    "qgalore_int8_linear_fwd": (c_int32, [c_void_p, c_void_p, c_void_p, c_int64, c_int64,
                                          c_int64, c_void_p, c_void_p]),
    "qgalore_int8_linear_bwd_data": (c_int32, [c_void_p, c_void_p, c_void_p, c_int64, c_int64,
                                               c_int64, c_void_p, c_void_p]),
    "qgalore_linear_bwd_weight": (c_int32, [c_void_p, c_void_p, c_int64, c_int64, c_int64,
                                            c_void_p, c_void_p]),
    "qgalore_sched_init": (c_int32, [ctypes.POINTER(Sched), c_int64, c_float]),
    "qgalore_sched_due": (c_int32, [ctypes.POINTER(Sched), c_int64]),
    "qgalore_sched_refresh": (c_int32, [ctypes.POINTER(Sched), c_int64, c_float,
                                        ctypes.POINTER(c_int32)]),
    "qgalore_mfma_probe": (c_int32, [c_void_p, c_int64, c_void_p, c_int32, c_int32, c_void_p]),
    "qgalore_status_str": (ctypes.c_char_p, [c_int32]),
    "qgalore_last_error": (ctypes.c_char_p, []),
    "qgalore_version": (ctypes.c_char_p, []),
}

_lib = None


def lib() -> ctypes.CDLL:
    """Load libqgalore.so (built in-tree by build.py); raises if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python quantized_rank_gradient_amd/build.py`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in EXPORTS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


class QgError(RuntimeError):
    def __init__(self, status: int, where: str):
        L = lib()
        text = L.qgalore_status_str(status).decode()
        if status == 6:
            text += ": " + L.qgalore_last_error().decode()
        super().__init__(f"{where}: {STATUS.get(status, status)} ({text})")
        self.status = status


def _check(status: int, where: str) -> None:
    if status != 0:
        raise QgError(status, where)


def n_groups(numel: int) -> int:
    return -(-int(numel) // GROUP)


def _ptr(t, dtype, shape=None, name="tensor"):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU (got {t.device})")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


@dataclasses.dataclass
class LayerTensors:
    """One linear layer's optimizer state on the GPU (see include/qgalore.h for layouts)."""
    layer_id: int
    G: torch.Tensor          # bf16 m x n
    Wq: torch.Tensor         # int8 m x n
    Ws: torch.Tensor         # fp32 [groups(m*n)]
    Pq: torch.Tensor         # int4: uint8 [ceil(m*r/2)]; int8: int8 m*r; bf16: bf16 m*r
    Ps: torch.Tensor         # fp32 [groups(m*r)] (None for bf16)
    Mq: torch.Tensor         # int8 r x n
    Ms: torch.Tensor         # fp32 [groups(r*n)]
    Vq: torch.Tensor         # int8 r x n
    Vs: torch.Tensor         # fp32 [groups(r*n)]
    r: int
    p_format: str = "int4"   # storage format of P: "int4", "int8" or "bf16"

    @property
    def m(self) -> int:
        return int(self.Wq.shape[0])

    @property
    def n(self) -> int:
        return int(self.Wq.shape[1])


def _proj_codes(Pq, m: int, r: int, fmt: str):
    """Pointer to a projection's codes (or bf16 values) in format fmt, checked."""
    if fmt == "int4":
        return _ptr(Pq, torch.uint8, ((m * r + 1) // 2,), "P_q")
    if fmt == "int8":
        return _ptr(Pq, torch.int8, (m * r,), "P_q")
    if fmt == "bf16":
        return _ptr(Pq.reshape(-1) if Pq is not None else None, torch.bfloat16, (m * r,), "P_q")
    raise ValueError(f"unknown projection format {fmt!r}")


def _fill_desc(d: LayerDesc, L: LayerTensors, hp: dict, R_out=None, U_out=None,
               dequant: str = "auto"):
    m, n, r = L.m, L.n, L.r
    d.m, d.n, d.r = m, n, r
    d.layer_id = L.layer_id
    d.lr, d.beta1, d.beta2 = hp.get("lr", 1e-3), hp.get("beta1", 0.9), hp.get("beta2", 0.999)
    d.eps, d.alpha = hp.get("eps", 1e-8), hp.get("alpha", 0.25)
    d.M_scale = _ptr(L.Ms, torch.float32, (n_groups(r * n),), "Ms")
    d.V_scale = _ptr(L.Vs, torch.float32, (n_groups(r * n),), "Vs")
    d.R_out = _ptr(R_out, torch.float32, (r, n), "R_out")
    d.U_out = _ptr(U_out, torch.float32, (m, n), "U_out")
    d.p_format = P_FORMATS[L.p_format]
    d.dequant_mode = DEQUANT_MODES[dequant]
    ptrs = dict(G=_ptr(L.G, torch.bfloat16, (m, n), "G"),
                W_q=_ptr(L.Wq, torch.int8, (m, n), "Wq"),
                W_scale=_ptr(L.Ws, torch.float32, (n_groups(m * n),), "Ws"),
                P_q=_proj_codes(L.Pq, m, r, L.p_format),
                P_scale=_ptr(L.Ps, torch.float32, (n_groups(m * r),), "Ps"),
                M_q=_ptr(L.Mq, torch.int8, (r, n), "Mq"),
                V_q=_ptr(L.Vq, torch.int8, (r, n), "Vq"))
    return ptrs


def workspace_bytes(m: int, n: int, r: int) -> int:
    return int(lib().qgalore_workspace_bytes(m, n, r))


def alloc_workspace(nbytes: int, device="cuda") -> torch.Tensor:
    return torch.empty(max(int(nbytes), 16), dtype=torch.uint8, device=device)


def step(L: LayerTensors, t: int, seed: int, hp: dict | None = None, workspace=None,
         R_out=None, U_out=None, stream=None, dequant: str = "auto") -> None:
    """One optimizer step of one layer (asynchronous on the current stream). `dequant`:
    where an INT4 projection is dequantized ("auto", "inline", "pass"; qg_dequant_mode)."""
    hp = hp or {}
    d = LayerDesc()
    ptrs = _fill_desc(d, L, hp, R_out, U_out, dequant)
    need = int(lib().qgalore_layer_workspace_bytes(ctypes.byref(d)))
    if workspace is None:
        workspace = alloc_workspace(need, L.Wq.device)
    d.workspace = _ptr(workspace, torch.uint8, None, "workspace")
    d.workspace_bytes = workspace.numel()
    d.stream = _stream(stream)
    _check(lib().qgalore_step(ctypes.byref(d), ptrs["G"], ptrs["W_q"], ptrs["W_scale"],
                              ptrs["P_q"], ptrs["P_scale"], ptrs["M_q"], ptrs["V_q"], int(t),
                              int(seed) & (2 ** 64 - 1)), "qgalore_step")


# size of the library's own scratch array used by step_noalloc (QG_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 64 << 20


def step_noalloc(L: LayerTensors, t: int, seed: int, hp: dict | None = None, R_out=None,
                 U_out=None, stream=None, dequant: str = "auto") -> None:
    """qgalore_step_noalloc: one layer's step with the library's fixed scratch array instead
    of a workspace (no device allocation anywhere on this path)."""
    hp = hp or {}
    d = LayerDesc()
    ptrs = _fill_desc(d, L, hp, R_out, U_out, dequant)
    d.stream = _stream(stream)
    _check(lib().qgalore_step_noalloc(ctypes.byref(d), ptrs["G"], ptrs["W_q"], ptrs["W_scale"],
                                      ptrs["P_q"], ptrs["P_scale"], ptrs["M_q"], ptrs["V_q"],
                                      int(t), int(seed) & (2 ** 64 - 1)), "qgalore_step_noalloc")


class Plan:
    """A grouped step over many layers: one launch per kernel for the whole set."""

    def __init__(self, layers: list, hp: dict | None = None, per_layer_hp: list | None = None,
                 R_out: list | None = None, U_out: list | None = None, dequant="auto"):
        """`dequant`: one qg_dequant_mode name for every layer, or a list with one per layer."""
        hp = hp or {}
        arr = (Layer * len(layers))()
        self._keep = list(layers) + list(R_out or []) + list(U_out or [])
        for k, L in enumerate(layers):
            h = per_layer_hp[k] if per_layer_hp else hp
            dq = dequant if isinstance(dequant, str) else dequant[k]
            ptrs = _fill_desc(arr[k].desc, L, h, R_out[k] if R_out else None,
                              U_out[k] if U_out else None, dq)
            for name, val in ptrs.items():
                setattr(arr[k], name, val)
        handle = c_void_p()
        _check(lib().qgalore_plan_create(arr, len(layers), ctypes.byref(handle)),
               "qgalore_plan_create")
        self._h = handle
        self.workspace_bytes = int(lib().qgalore_plan_workspace_bytes(handle))
        self.workspace = None

    def step(self, t: int, seed: int, workspace=None, stream=None) -> None:
        if workspace is None:
            if self.workspace is None:
                self.workspace = alloc_workspace(self.workspace_bytes, self._keep[0].Wq.device)
            workspace = self.workspace
        _check(lib().qgalore_plan_step(self._h, int(t), int(seed) & (2 ** 64 - 1),
                                       _ptr(workspace, torch.uint8, None, "workspace"),
                                       workspace.numel(), _stream(stream)), "qgalore_plan_step")

    def cache_proj(self, enable: bool = True) -> None:
        """Keep dequantized projections between steps (qgalore_plan_cache_proj); the caller
        then reports every projection it rewrites with proj_changed()."""
        _check(lib().qgalore_plan_cache_proj(self._h, 1 if enable else 0),
               "qgalore_plan_cache_proj")

    def proj_changed(self, layer: int) -> None:
        _check(lib().qgalore_plan_proj_changed(self._h, int(layer)), "qgalore_plan_proj_changed")

    def enable_timing(self, max_steps: int) -> None:
        _check(lib().qgalore_plan_enable_timing(self._h, int(max_steps)),
               "qgalore_plan_enable_timing")

    def kernel_times(self):
        """Mean (dequant, projection, Adam, back-projection) kernel milliseconds over the
        recorded steps, and the number of steps recorded."""
        out = (c_float * 4)()
        steps = c_int32(0)
        _check(lib().qgalore_plan_kernel_times(self._h, out, ctypes.byref(steps)),
               "qgalore_plan_kernel_times")
        return [float(x) for x in out], int(steps.value)

    def close(self) -> None:
        if self._h:
            _check(lib().qgalore_plan_destroy(self._h), "qgalore_plan_destroy")
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def _proj(Pq, Ps, m, r, fmt="int4") -> Proj:
    p = Proj()
    p.m, p.r = m, r
    p.q = _proj_codes(Pq, m, r, fmt)
    p.scale = _ptr(Ps, torch.float32, (n_groups(m * r),), "P_scale")
    p.format = P_FORMATS[fmt]
    return p


def cossim_workspace_bytes(m: int, r: int) -> int:
    return int(lib().qgalore_cossim_workspace_bytes(m, r))


def cossim_async(Pq_new, Ps_new, Pq_old, Ps_old, m: int, r: int, out: torch.Tensor,
                 workspace=None, stream=None, fmt: str = "int4") -> None:
    """CosSim of two stored projections into out[0] (device fp32), asynchronously."""
    a, b = _proj(Pq_new, Ps_new, m, r, fmt), _proj(Pq_old, Ps_old, m, r, fmt)
    if workspace is None:
        workspace = alloc_workspace(cossim_workspace_bytes(m, r), Pq_new.device)
    _check(lib().qgalore_cossim_async(ctypes.byref(a), ctypes.byref(b),
                                      _ptr(workspace, torch.uint8, None, "workspace"),
                                      workspace.numel(), _stream(stream),
                                      _ptr(out, torch.float32, None, "out")),
           "qgalore_cossim_async")


def cossim_batch_workspace_bytes(r: int, count: int) -> int:
    return int(lib().qgalore_cossim_batch_workspace_bytes(r, count))


def cossim_batch(pairs, r: int, out: torch.Tensor, workspace=None, stream=None) -> None:
    """pairs: list of (Pq_new, Ps_new, Pq_old, Ps_old, m[, format]); out[k] (device fp32)
    receives CosSim of pair k, asynchronously. All pairs share the rank r."""
    n = len(pairs)
    A = (Proj * n)()
    Bp = (Proj * n)()
    for k, pr in enumerate(pairs):
        qn, sn, qo, so, m = pr[:5]
        fmt = pr[5] if len(pr) > 5 else "int4"
        A[k] = _proj(qn, sn, m, r, fmt)
        Bp[k] = _proj(qo, so, m, r, fmt)
    if workspace is None:
        workspace = alloc_workspace(cossim_batch_workspace_bytes(r, n), pairs[0][0].device)
    _check(lib().qgalore_cossim_batch(A, Bp, n, _ptr(workspace, torch.uint8, None, "workspace"),
                                      workspace.numel(), _stream(stream),
                                      _ptr(out, torch.float32, None, "out")),
           "qgalore_cossim_batch")


def cossim(Pq_new, Ps_new, Pq_old, Ps_old, m: int, r: int, workspace=None, stream=None,
           fmt: str = "int4") -> float:
    a, b = _proj(Pq_new, Ps_new, m, r, fmt), _proj(Pq_old, Ps_old, m, r, fmt)
    if workspace is None:
        workspace = alloc_workspace(cossim_workspace_bytes(m, r), Pq_new.device)
    out = c_float()
    _check(lib().qgalore_cossim(ctypes.byref(a), ctypes.byref(b),
                                _ptr(workspace, torch.uint8, None, "workspace"),
                                workspace.numel(), _stream(stream), ctypes.byref(out)),
           "qgalore_cossim")
    return float(out.value)


def quantize_proj(P: torch.Tensor, stream=None, fmt: str = "int4"):
    """Group quantization of an fp32 m x r projection -> (P_q, P_scale): INT4 (uint8 packed
    codes), INT8 (int8 codes), or for "bf16" the bf16 values (a cast; no scales)."""
    m, r = P.shape
    src = _ptr(P, torch.float32, (m, r), "P")
    if fmt == "bf16":
        return P.to(torch.bfloat16).reshape(-1).contiguous(), None
    Ps = torch.empty(n_groups(m * r), dtype=torch.float32, device=P.device)
    if fmt == "int8":
        Pq = torch.empty(m * r, dtype=torch.int8, device=P.device)
        _check(lib().qgalore_quantize_proj_int8(src, m, r, Pq.data_ptr(), Ps.data_ptr(),
                                                _stream(stream)), "qgalore_quantize_proj_int8")
        return Pq, Ps
    if fmt != "int4":
        raise ValueError(f"unknown projection format {fmt!r}")
    Pq = torch.empty((m * r + 1) // 2, dtype=torch.uint8, device=P.device)
    _check(lib().qgalore_quantize_proj(src, m, r, Pq.data_ptr(), Ps.data_ptr(), _stream(stream)),
           "qgalore_quantize_proj")
    return Pq, Ps


def mfma_probe(operands: torch.Tensor, out: torch.Tensor, grid: int, iters: int,
               stream=None) -> float:
    """Launch the MFMA calibration kernel on bf16 `operands` (see qgalore_mfma_probe);
    returns the flops the launch performs."""
    if operands.dtype != torch.bfloat16 or not operands.is_contiguous():
        raise TypeError("operands must be a contiguous bf16 tensor")
    if out.dtype != torch.float32 or out.numel() < grid * 256:
        raise ValueError("out must hold grid * 256 float32 values")
    _check(lib().qgalore_mfma_probe(operands.data_ptr(), operands.numel(), out.data_ptr(), grid,
                                    iters, _stream(stream)), "qgalore_mfma_probe")
    return float(grid) * 4 * iters * 16 * 32768


def refresh_workspace_bytes(m: int, n: int, r: int, oversample: int = 8) -> int:
    return int(lib().qgalore_refresh_workspace_bytes(m, n, r, oversample))


def refresh_proj(G: torch.Tensor, r: int, Omega: torch.Tensor, power_iters: int = 2,
                 P_out=None, sigma_out=None, workspace=None, stream=None):
    """New projection of the gradient G (bf16 m x n): the r leading left singular vectors by
    the library's randomized range finder with the caller's sketch Omega (bf16 n x k,
    k = r + oversample), quantized to INT4 -> (P_q, P_scale). P_out (fp32 m x r) and
    sigma_out (fp32 r) optionally receive P before quantization and the singular values."""
    m, n = G.shape
    k = Omega.shape[1]
    g = _ptr(G, torch.bfloat16, (m, n), "G")
    om = _ptr(Omega, torch.bfloat16, (n, k), "Omega")
    Pq = torch.empty((m * r + 1) // 2, dtype=torch.uint8, device=G.device)
    Ps = torch.empty(n_groups(m * r), dtype=torch.float32, device=G.device)
    if workspace is None:
        nbytes = refresh_workspace_bytes(m, n, r, k - r)
        if nbytes == 0:
            raise ValueError(f"refresh of a {m} x {n} gradient at rank {r} with sketch width "
                             f"{k} is not supported")
        workspace = alloc_workspace(nbytes, G.device)
    _check(lib().qgalore_refresh_proj(
        g, m, n, r, om, k - r, int(power_iters), Pq.data_ptr(), Ps.data_ptr(),
        _ptr(P_out, torch.float32, (m, r), "P_out"), _ptr(sigma_out, torch.float32, (r,), "sigma_out"),
        _ptr(workspace, torch.uint8, None, "workspace"), workspace.numel(), _stream(stream)),
        "qgalore_refresh_proj")
    return Pq, Ps


def int8_linear_fwd(X: torch.Tensor, Wq: torch.Tensor, Ws: torch.Tensor, out=None,
                    stream=None) -> torch.Tensor:
    """Y = X W~^T (bf16 T x m) for the INT8 weight Wq (m x n) with group scales Ws."""
    T, n = X.shape
    m = Wq.shape[0]
    Y = out if out is not None else torch.empty((T, m), dtype=torch.bfloat16, device=X.device)
    _check(lib().qgalore_int8_linear_fwd(
        _ptr(X, torch.bfloat16, (T, n), "X"), _ptr(Wq, torch.int8, (m, n), "Wq"),
        _ptr(Ws, torch.float32, (n_groups(m * n),), "Ws"), T, m, n,
        _ptr(Y, torch.bfloat16, (T, m), "Y"), _stream(stream)), "qgalore_int8_linear_fwd")
    return Y


def int8_linear_bwd_data(dY: torch.Tensor, Wq: torch.Tensor, Ws: torch.Tensor, out=None,
                         stream=None) -> torch.Tensor:
    """dX = dY W~ (bf16 T x n)."""
    T, m = dY.shape
    n = Wq.shape[1]
    dX = out if out is not None else torch.empty((T, n), dtype=torch.bfloat16, device=dY.device)
    _check(lib().qgalore_int8_linear_bwd_data(
        _ptr(dY, torch.bfloat16, (T, m), "dY"), _ptr(Wq, torch.int8, (m, n), "Wq"),
        _ptr(Ws, torch.float32, (n_groups(m * n),), "Ws"), T, m, n,
        _ptr(dX, torch.bfloat16, (T, n), "dX"), _stream(stream)), "qgalore_int8_linear_bwd_data")
    return dX


def linear_bwd_weight(dY: torch.Tensor, X: torch.Tensor, out=None, stream=None) -> torch.Tensor:
    """G = dY^T X (bf16 m x n): the weight gradient the optimizer step takes."""
    T, m = dY.shape
    n = X.shape[1]
    G = out if out is not None else torch.empty((m, n), dtype=torch.bfloat16, device=dY.device)
    _check(lib().qgalore_linear_bwd_weight(
        _ptr(dY, torch.bfloat16, (T, m), "dY"), _ptr(X, torch.bfloat16, (T, n), "X"), T, m, n,
        _ptr(G, torch.bfloat16, (m, n), "G"), _stream(stream)), "qgalore_linear_bwd_weight")
    return G


class Schedule:
    """Per-layer refresh bookkeeping (host-side, in the library)."""

    def __init__(self, delta0: int, gamma: float = 0.4):
        self._s = Sched()
        _check(lib().qgalore_sched_init(ctypes.byref(self._s), int(delta0), float(gamma)),
               "qgalore_sched_init")

    def due(self, t: int) -> bool:
        return bool(lib().qgalore_sched_due(ctypes.byref(self._s), int(t)))

    def refresh(self, t: int, cs: float | None) -> bool:
        doubled = c_int32(0)
        _check(lib().qgalore_sched_refresh(ctypes.byref(self._s), int(t),
                                           float("nan") if cs is None else float(cs),
                                           ctypes.byref(doubled)), "qgalore_sched_refresh")
        return bool(doubled.value)

    @property
    def delta(self) -> int:
        return int(self._s.delta)

    @property
    def next_refresh(self) -> int:
        return int(self._s.next_refresh)

    @property
    def count(self) -> int:
        return int(self._s.count)

    @property
    def last_cossim(self) -> float:
        v = float(self._s.last_cossim)
        return v if not math.isnan(v) else float("nan")
