"""Python binding of libmuon_hip.so, the batched Muon step for MI355X (gfx950).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in include/muon_hip.h.  PyTorch supplies
device memory (tensors, the cached workspace) and the current stream.  There
is no fallback: if the library is missing or the device is not gfx950 the
calls raise.

Entry points (same names as the C ABI):
    ns_orthogonalize_batched(x, out=None, *, view_blocks=1, ...)
    ns_orthogonalize_batched_noalloc(x, out=None, *, view_blocks=1, ...)
    muon_step_batched(params, grads, momentum_buf, *, lr, weight_decay, momentum, ...)
    muon_step_multi(matrices, *, lr, weight_decay, momentum, ...)
    adamw_step_multi(tensors, *, lr, betas, eps, weight_decay)
    muon_merge_small_dims(shape, threshold, target_ndim=2)
    muon_workspace_bytes(batch, rows, cols, view_blocks=1, cfg=None)
    muon_step_multi_workspace_bytes(matrices, cfg=None)
    muon_workspace_status(workspace, stream=None), last_call_status(device=None)
    muon_debug_set_loop_fault(mode), muon_set_ns_schedule(schedule), muon_set_gemm_tiling(width)
    muon_ns_config_default(), muon_last_error(), muon_abi_version()
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional, Tuple

__all__ = [
    "MuonNSConfig", "MuonError", "LIB_PATH", "EXPORTED_SYMBOLS", "load_library",
    "muon_ns_config_default", "muon_workspace_bytes", "ns_orthogonalize_batched",
    "ns_orthogonalize_batched_noalloc", "NOALLOC_SCRATCH_BYTES", "muon_step_batched", "muon_step_multi", "muon_step_multi_workspace_bytes", "MuonMatrix",
    "adamw_step_multi", "MuonAdamTensor", "muon_merge_small_dims",
    "muon_timing_enable", "muon_timing_collect", "muon_last_error", "muon_abi_version", "make_config",
    "muon_set_ns_schedule", "KERNEL_KINDS", "NS_SCHEDULES", "muon_workspace_status", "last_call_status",
    "muon_debug_set_loop_fault", "muon_set_gemm_tiling", "GEMM_TILINGS",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmuon_hip.so")
EXPORTED_SYMBOLS = ("muon_ns_config_default", "muon_workspace_bytes", "ns_orthogonalize_batched",
                    "ns_orthogonalize_batched_noalloc",
                    "muon_step_batched", "muon_step_multi_workspace_bytes", "muon_step_multi",
                    "adamw_step_multi", "muon_merge_small_dims", "muon_set_ns_schedule", "muon_set_gemm_tiling", "muon_timing_enable",
                    "muon_timing_collect", "muon_workspace_status", "muon_debug_set_loop_fault",
                    "muon_last_error", "muon_abi_version")
NOALLOC_SCRATCH_BYTES = 64 << 20   # MUON_NOALLOC_SCRATCH_BYTES of the header
KERNEL_KINDS = ("prep", "norm_finalize", "gram", "poly", "bx", "finish", "small", "adamw", "ns_loop")
NS_SCHEDULES = {"auto": 0, "per_product": 1, "persistent": 2}
GEMM_TILINGS = (0, 64, 128, 256)

MUON_OK = 0
_STATUS_NAMES = {0: "MUON_OK", 1: "MUON_ERR_INVALID_ARG", 2: "MUON_ERR_SHAPE", 3: "MUON_ERR_ALIGNMENT",
                 4: "MUON_ERR_WORKSPACE", 5: "MUON_ERR_HIP", 6: "MUON_ERR_UNSUPPORTED"}
PRECISIONS = {"fast": 0, "accurate": 1}


class MuonNSConfig(ctypes.Structure):
    _fields_ = [("ns_steps", ctypes.c_int32), ("a", ctypes.c_float), ("b", ctypes.c_float),
                ("c", ctypes.c_float), ("eps", ctypes.c_float), ("precision", ctypes.c_int32)]


class MuonMatrix(ctypes.Structure):
    """muon_matrix of the C ABI: one matrix of a multi-matrix step."""
    _fields_ = [("params", ctypes.c_void_p), ("grads", ctypes.c_void_p), ("momentum_buf", ctypes.c_void_p),
                ("update_out", ctypes.c_void_p), ("rows", ctypes.c_int64), ("cols", ctypes.c_int64),
                ("view_blocks", ctypes.c_int32), ("lr_mul", ctypes.c_float), ("wd_mul", ctypes.c_float)]


class MuonAdamTensor(ctypes.Structure):
    """muon_adam_tensor of the C ABI: one tensor of an AdamW step."""
    _fields_ = [("params", ctypes.c_void_p), ("grads", ctypes.c_void_p), ("exp_avg", ctypes.c_void_p),
                ("exp_avg_sq", ctypes.c_void_p), ("numel", ctypes.c_int64), ("step", ctypes.c_int64),
                ("lr_mul", ctypes.c_float), ("wd_mul", ctypes.c_float)]


class MuonError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


_lib = None
_lib_lock = threading.Lock()


def load_library():
    """Loads libmuon_hip.so (raises if it has not been built)."""
    global _lib
    with _lib_lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing; build it with `python -m newton_schulz_muon_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        vp, i64, i32, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float
        cfgp = ctypes.POINTER(MuonNSConfig)
        lib.muon_ns_config_default.argtypes = [cfgp]
        lib.muon_ns_config_default.restype = None
        lib.muon_workspace_bytes.argtypes = [i64, i64, i64, i32, cfgp]
        lib.muon_workspace_bytes.restype = ctypes.c_size_t
        lib.ns_orthogonalize_batched.argtypes = [vp, vp, i64, i64, i64, i32, cfgp, vp, ctypes.c_size_t, vp]
        lib.ns_orthogonalize_batched.restype = ctypes.c_int
        lib.ns_orthogonalize_batched_noalloc.argtypes = [vp, vp, i64, i64, i64, i32, cfgp, vp]
        lib.ns_orthogonalize_batched_noalloc.restype = ctypes.c_int
        lib.muon_step_batched.argtypes = [vp, vp, vp, i64, i64, i64, i32, f32, f32, f32, i32, f32, f32,
                                          cfgp, vp, vp, ctypes.c_size_t, vp]
        lib.muon_step_batched.restype = ctypes.c_int
        matp = ctypes.POINTER(MuonMatrix)
        lib.muon_step_multi_workspace_bytes.argtypes = [matp, i32, cfgp]
        lib.muon_step_multi_workspace_bytes.restype = ctypes.c_size_t
        lib.muon_step_multi.argtypes = [matp, i32, f32, f32, f32, i32, cfgp, vp, ctypes.c_size_t, vp]
        lib.muon_step_multi.restype = ctypes.c_int
        adamp = ctypes.POINTER(MuonAdamTensor)
        lib.adamw_step_multi.argtypes = [adamp, i32, f32, f32, f32, f32, f32, vp]
        lib.adamw_step_multi.restype = ctypes.c_int
        i64p = ctypes.POINTER(ctypes.c_int64)
        lib.muon_merge_small_dims.argtypes = [i64p, i32, i64, i32, i64p, ctypes.POINTER(ctypes.c_int32)]
        lib.muon_merge_small_dims.restype = ctypes.c_int
        lib.muon_set_ns_schedule.argtypes = [i32]
        lib.muon_set_ns_schedule.restype = ctypes.c_int
        lib.muon_timing_enable.argtypes = [ctypes.c_uint32]
        lib.muon_timing_enable.restype = ctypes.c_int
        lib.muon_timing_collect.argtypes = [ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_double),
                                            ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double)]
        lib.muon_timing_collect.restype = ctypes.c_int
        lib.muon_workspace_status.argtypes = [vp, vp, vp]
        lib.muon_workspace_status.restype = ctypes.c_int
        lib.muon_debug_set_loop_fault.argtypes = [i32]
        lib.muon_debug_set_loop_fault.restype = ctypes.c_int
        lib.muon_set_gemm_tiling.argtypes = [i32]
        lib.muon_set_gemm_tiling.restype = ctypes.c_int
        lib.muon_last_error.argtypes = []
        lib.muon_last_error.restype = ctypes.c_char_p
        lib.muon_abi_version.argtypes = []
        lib.muon_abi_version.restype = ctypes.c_int32
        _lib = lib
        return lib


def muon_ns_config_default() -> MuonNSConfig:
    cfg = MuonNSConfig()
    load_library().muon_ns_config_default(ctypes.byref(cfg))
    return cfg


def make_config(ns_steps: int = 5, coeffs: Optional[Tuple[float, float, float]] = None,
                eps: Optional[float] = None, precision: str = "fast") -> MuonNSConfig:
    cfg = muon_ns_config_default()
    cfg.ns_steps = int(ns_steps)
    if coeffs is not None:
        cfg.a, cfg.b, cfg.c = (float(v) for v in coeffs)
    if eps is not None:
        cfg.eps = float(eps)
    if precision not in PRECISIONS:
        raise ValueError(f"precision must be one of {sorted(PRECISIONS)}")
    cfg.precision = PRECISIONS[precision]
    return cfg


def muon_set_ns_schedule(schedule: str) -> None:
    """Process-wide schedule of the NS iterations of large blocks: "auto" (the
    default: per set of shapes, the faster of the two after a few timed
    calls), "per_product" (three launches per iteration) or "persistent" (one
    launch for all iterations where the shapes allow).  Results are bitwise
    equal."""
    if schedule not in NS_SCHEDULES:
        raise ValueError(f"schedule must be one of {sorted(NS_SCHEDULES)}")
    _check(load_library().muon_set_ns_schedule(NS_SCHEDULES[schedule]))


def muon_set_gemm_tiling(width: int = 0) -> None:
    """Process-wide tile width of the per-product launches: 0 (the default:
    per launch, the lowest estimated time), 64, 128 or 256 (256 where both
    padded block sides are multiples of 256, else 128).  Results are bitwise
    equal."""
    if width not in GEMM_TILINGS:
        raise ValueError(f"tile width must be one of {GEMM_TILINGS}")
    _check(load_library().muon_set_gemm_tiling(int(width)))


def muon_timing_enable(kinds=()) -> None:
    """Records hipEvents around every launch of the named kernel families
    (names from KERNEL_KINDS); an empty list turns recording off."""
    mask = 0
    for k in kinds:
        mask |= 1 << KERNEL_KINDS.index(k)
    _check(load_library().muon_timing_enable(mask))


def muon_timing_collect(with_flops: bool = False) -> dict:
    """{family: (launches, total_ms)} for the launches recorded since the last
    collect; with_flops=True adds the nominal and the executed flops of those
    launches as third and fourth elements."""
    n = len(KERNEL_KINDS)
    launches = (ctypes.c_int64 * n)()
    total = (ctypes.c_double * n)()
    flops = (ctypes.c_double * n)()
    executed = (ctypes.c_double * n)()
    _check(load_library().muon_timing_collect(launches, total, flops, executed))
    if with_flops:
        return {k: (int(launches[i]), float(total[i]), float(flops[i]), float(executed[i]))
                for i, k in enumerate(KERNEL_KINDS) if launches[i]}
    return {k: (int(launches[i]), float(total[i])) for i, k in enumerate(KERNEL_KINDS) if launches[i]}


def muon_workspace_status(workspace, stream=None):
    """(blocks left incomplete, error flags) of the last call that used the
    workspace tensor (see the C ABI's muon_workspace_status); waits for it."""
    import torch
    with torch.cuda.device(workspace.device):
        st = stream if stream is not None else torch.cuda.current_stream(workspace.device).cuda_stream
        out = torch.empty(2, dtype=torch.int32, device=workspace.device)
        _check(load_library().muon_workspace_status(workspace.data_ptr(), out.data_ptr(), st))
        v = out.cpu().tolist()
    return int(v[0]) & 0xffffffff, int(v[1]) & 0xffffffff


def last_call_status(device=None):
    """Status of the last call on `device` (default: current) and its current
    stream that used the binding's cached workspace: (blocks left incomplete,
    error flags); (0, 0) when no call there needed a workspace."""
    import torch
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
    stream = torch.cuda.current_stream(dev).cuda_stream
    with _ws_lock:
        buf = _ws_cache.get((dev.index, stream))
    if buf is None:
        return 0, 0
    return muon_workspace_status(buf, stream)


def muon_debug_set_loop_fault(mode: int) -> None:
    """Diagnostics: 0 normal, 1 every persistent-loop launch stops at its
    first item, 2 every dependency wait not met at once times out."""
    _check(load_library().muon_debug_set_loop_fault(int(mode)))


def muon_last_error() -> str:
    return load_library().muon_last_error().decode()


def muon_abi_version() -> int:
    return int(load_library().muon_abi_version())


def muon_workspace_bytes(batch: int, rows: int, cols: int, view_blocks: int = 1,
                         cfg: Optional[MuonNSConfig] = None) -> int:
    lib = load_library()
    n = lib.muon_workspace_bytes(int(batch), int(rows), int(cols), int(view_blocks),
                                 ctypes.byref(cfg) if cfg is not None else None)
    if n == ctypes.c_size_t(-1).value:
        raise MuonError(2, lib.muon_last_error().decode())
    return int(n)


# ---------------------------------------------------------------- workspace cache
_ws_cache = {}
_ws_lock = threading.Lock()


def _workspace(device, stream_ptr: int, nbytes: int):
    import torch
    if nbytes == 0:
        return None
    key = (device.index, stream_ptr)
    with _ws_lock:
        buf = _ws_cache.get(key)
        if buf is None or buf.numel() < nbytes:
            _ws_cache.pop(key, None)
            buf = torch.empty(nbytes, dtype=torch.uint8, device=device)
            _ws_cache[key] = buf
        return buf


def _check(status: int):
    if status != MUON_OK:
        raise MuonError(status, load_library().muon_last_error().decode())


def _as3d(t, name):
    if t.dim() == 2:
        return t.unsqueeze(0)
    if t.dim() != 3:
        raise ValueError(f"{name} must be [batch, rows, cols] or [rows, cols]")
    return t


def _require(t, name, dtype, device=None):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU device")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def ns_orthogonalize_batched(x, out=None, *, view_blocks: int = 1, ns_steps: int = 5,
                             coeffs: Optional[Tuple[float, float, float]] = None,
                             eps: Optional[float] = None, precision: str = "fast",
                             cfg: Optional[MuonNSConfig] = None):
    """out = NS(x) per NS block of a bf16 [batch, rows, cols] (or [rows, cols]) tensor."""
    import torch
    _require(x, "x", torch.bfloat16)
    if out is None:
        out = torch.empty_like(x)
    _require(out, "out", torch.bfloat16, x.device)
    if out.shape != x.shape:
        raise ValueError("out must have the shape of x")
    x3, o3 = _as3d(x, "x"), _as3d(out, "out")
    cfg = cfg if cfg is not None else make_config(ns_steps, coeffs, eps, precision)
    B, R, C = x3.shape
    lib = load_library()
    with torch.cuda.device(x.device):
        stream = torch.cuda.current_stream(x.device).cuda_stream
        nbytes = muon_workspace_bytes(B, R, C, view_blocks, cfg)
        ws = _workspace(x.device, stream, nbytes)
        _check(lib.ns_orthogonalize_batched(
            x3.data_ptr(), o3.data_ptr(), B, R, C, int(view_blocks), ctypes.byref(cfg),
            ws.data_ptr() if ws is not None else None, nbytes, stream))
    return out


def ns_orthogonalize_batched_noalloc(x, out=None, *, view_blocks: int = 1, ns_steps: int = 5,
                                     coeffs: Optional[Tuple[float, float, float]] = None,
                                     eps: Optional[float] = None, precision: str = "fast",
                                     cfg: Optional[MuonNSConfig] = None):
    """ns_orthogonalize_batched without a workspace: the library's static
    per-GPU scratch (NOALLOC_SCRATCH_BYTES) serves instead, and the C call
    allocates nothing (pass `out` to keep the binding from allocating it)."""
    import torch
    _require(x, "x", torch.bfloat16)
    if out is None:
        out = torch.empty_like(x)
    _require(out, "out", torch.bfloat16, x.device)
    if out.shape != x.shape:
        raise ValueError("out must have the shape of x")
    x3, o3 = _as3d(x, "x"), _as3d(out, "out")
    cfg = cfg if cfg is not None else make_config(ns_steps, coeffs, eps, precision)
    B, R, C = x3.shape
    with torch.cuda.device(x.device):
        stream = torch.cuda.current_stream(x.device).cuda_stream
        _check(load_library().ns_orthogonalize_batched_noalloc(
            x3.data_ptr(), o3.data_ptr(), B, R, C, int(view_blocks), ctypes.byref(cfg), stream))
    return out


def muon_step_batched(params, grads, momentum_buf, *, lr: float, weight_decay: float,
                      momentum: float, nesterov: bool = True, lr_mul: float = 1.0,
                      wd_mul: float = 1.0, view_blocks: int = 1, ns_steps: int = 5,
                      coeffs: Optional[Tuple[float, float, float]] = None,
                      eps: Optional[float] = None, precision: str = "fast",
                      update_out=None, cfg: Optional[MuonNSConfig] = None):
    """One in-place Muon step on fp32 params / bf16 grads / fp32 momentum buffers."""
    import torch
    _require(params, "params", torch.float32)
    _require(grads, "grads", torch.bfloat16, params.device)
    _require(momentum_buf, "momentum_buf", torch.float32, params.device)
    if grads.shape != params.shape or momentum_buf.shape != params.shape:
        raise ValueError("params, grads and momentum_buf must have one shape")
    if update_out is not None:
        _require(update_out, "update_out", torch.bfloat16, params.device)
        if update_out.shape != params.shape:
            raise ValueError("update_out must have the shape of params")
    p3, g3, m3 = _as3d(params, "params"), _as3d(grads, "grads"), _as3d(momentum_buf, "momentum_buf")
    cfg = cfg if cfg is not None else make_config(ns_steps, coeffs, eps, precision)
    B, R, C = p3.shape
    lib = load_library()
    with torch.cuda.device(params.device):
        stream = torch.cuda.current_stream(params.device).cuda_stream
        nbytes = muon_workspace_bytes(B, R, C, view_blocks, cfg)
        ws = _workspace(params.device, stream, nbytes)
        _check(lib.muon_step_batched(
            p3.data_ptr(), g3.data_ptr(), m3.data_ptr(), B, R, C, int(view_blocks),
            float(lr), float(weight_decay), float(momentum), 1 if nesterov else 0,
            float(lr_mul), float(wd_mul), ctypes.byref(cfg),
            update_out.data_ptr() if update_out is not None else None,
            ws.data_ptr() if ws is not None else None, nbytes, stream))
    return params


MERGE_THRESHOLD = 8192   # merge_small_dims threshold for >2-D parameters (the pages' conv example)


def _matrix_array(matrices, device, merge_threshold: int = MERGE_THRESHOLD):
    """ctypes array of MuonMatrix from (params, grads, momentum_buf) tuples or dicts with
    those keys and optional update_out, view_blocks, lr_mul, wd_mul.  A parameter of another
    rank is stepped as the 2-D matrix muon_merge_small_dims(shape, merge_threshold, 2) views it
    as (the same memory); one that does not merge to 2-D is rejected."""
    import torch
    arr = (MuonMatrix * max(1, len(matrices)))()
    keep = []
    for i, m in enumerate(matrices):
        if not isinstance(m, dict):
            m = dict(zip(("params", "grads", "momentum_buf"), m))
        P, G, M = m["params"], m["grads"], m["momentum_buf"]
        _require(P, f"matrices[{i}].params", torch.float32, device)
        _require(G, f"matrices[{i}].grads", torch.bfloat16, device)
        _require(M, f"matrices[{i}].momentum_buf", torch.float32, device)
        if G.shape != P.shape or M.shape != P.shape:
            raise ValueError(f"matrices[{i}]: params, grads and momentum_buf must have one shape")
        if P.dim() == 2:
            rows, cols = P.shape
        else:
            merged = muon_merge_small_dims(tuple(P.shape), merge_threshold, 2)
            if len(merged) != 2:
                raise ValueError(f"matrices[{i}]: shape {tuple(P.shape)} merges to {merged} at threshold "
                                 f"{merge_threshold}, not to a 2-D matrix")
            rows, cols = merged
        out = m.get("update_out")
        if out is not None:
            _require(out, f"matrices[{i}].update_out", torch.bfloat16, device)
            if out.shape != P.shape:
                raise ValueError(f"matrices[{i}].update_out must have the shape of params")
        e = arr[i]
        e.params, e.grads, e.momentum_buf = P.data_ptr(), G.data_ptr(), M.data_ptr()
        e.update_out = out.data_ptr() if out is not None else None
        e.rows, e.cols = rows, cols
        e.view_blocks = int(m.get("view_blocks", 1))
        e.lr_mul = float(m.get("lr_mul", 1.0))
        e.wd_mul = float(m.get("wd_mul", 1.0))
        keep.append(m)
    return arr, keep


def muon_step_multi_workspace_bytes(matrices, cfg: Optional[MuonNSConfig] = None,
                                    merge_threshold: int = MERGE_THRESHOLD) -> int:
    if not matrices:
        return 0
    first = matrices[0] if isinstance(matrices[0], dict) else {"params": matrices[0][0]}
    arr, _ = _matrix_array(matrices, first["params"].device, merge_threshold)
    lib = load_library()
    n = lib.muon_step_multi_workspace_bytes(arr, len(matrices), ctypes.byref(cfg) if cfg is not None else None)
    if n == ctypes.c_size_t(-1).value:
        raise MuonError(2, lib.muon_last_error().decode())
    return int(n)


def muon_step_multi(matrices, *, lr: float, weight_decay: float, momentum: float, nesterov: bool = True,
                    ns_steps: int = 5, coeffs: Optional[Tuple[float, float, float]] = None,
                    eps: Optional[float] = None, precision: str = "fast", cfg: Optional[MuonNSConfig] = None,
                    merge_threshold: int = MERGE_THRESHOLD):
    """One in-place Muon step on a list of matrices, each (params fp32, grads bf16, momentum fp32)
    or a dict with those keys and optional update_out, view_blocks, lr_mul, wd_mul.  Parameters
    that are not 2-D are stepped as their muon_merge_small_dims view (merge_threshold, target 2)."""
    import torch
    if not matrices:
        return
    first = matrices[0] if isinstance(matrices[0], dict) else {"params": matrices[0][0]}
    device = first["params"].device
    arr, _keep = _matrix_array(matrices, device, merge_threshold)
    cfg = cfg if cfg is not None else make_config(ns_steps, coeffs, eps, precision)
    lib = load_library()
    with torch.cuda.device(device):
        stream = torch.cuda.current_stream(device).cuda_stream
        nbytes = lib.muon_step_multi_workspace_bytes(arr, len(matrices), ctypes.byref(cfg))
        if nbytes == ctypes.c_size_t(-1).value:
            raise MuonError(2, lib.muon_last_error().decode())
        ws = _workspace(device, stream, int(nbytes))
        _check(lib.muon_step_multi(arr, len(matrices), float(lr), float(weight_decay), float(momentum),
                                   1 if nesterov else 0, ctypes.byref(cfg),
                                   ws.data_ptr() if ws is not None else None, int(nbytes), stream))


def adamw_step_multi(tensors, *, lr: float, betas: Tuple[float, float], eps: float, weight_decay: float):
    """One in-place AdamW step (DistAdam.step of the pages, decay first) on a list of tensors.

    Each entry is a dict with params (fp32), grads (bf16), exp_avg and exp_avg_sq (fp32), all
    contiguous and of one shape, step (the tensor's step count after the increment, >= 1) and
    optional lr_mul, wd_mul."""
    import torch
    if not tensors:
        return
    device = tensors[0]["params"].device
    arr = (MuonAdamTensor * len(tensors))()
    for i, t in enumerate(tensors):
        P, G, M, V = t["params"], t["grads"], t["exp_avg"], t["exp_avg_sq"]
        _require(P, f"tensors[{i}].params", torch.float32, device)
        _require(G, f"tensors[{i}].grads", torch.bfloat16, device)
        _require(M, f"tensors[{i}].exp_avg", torch.float32, device)
        _require(V, f"tensors[{i}].exp_avg_sq", torch.float32, device)
        if not (G.shape == P.shape and M.shape == P.shape and V.shape == P.shape):
            raise ValueError(f"tensors[{i}]: params, grads, exp_avg and exp_avg_sq must have one shape")
        e = arr[i]
        e.params, e.grads, e.exp_avg, e.exp_avg_sq = P.data_ptr(), G.data_ptr(), M.data_ptr(), V.data_ptr()
        e.numel = P.numel()
        e.step = int(t["step"])
        e.lr_mul = float(t.get("lr_mul", 1.0))
        e.wd_mul = float(t.get("wd_mul", 1.0))
    lib = load_library()
    b1, b2 = betas
    with torch.cuda.device(device):
        stream = torch.cuda.current_stream(device).cuda_stream
        _check(lib.adamw_step_multi(arr, len(tensors), float(lr), float(b1), float(b2), float(eps),
                                    float(weight_decay), stream))


def muon_merge_small_dims(shape, threshold: int, target_ndim: int = 2) -> Tuple[int, ...]:
    """Merged shape of a contiguous tensor (the C ABI's muon_merge_small_dims);
    target_ndim 0 means no target."""
    lib = load_library()
    shape = [int(s) for s in shape]
    arr = (ctypes.c_int64 * max(1, len(shape)))(*shape)
    out = (ctypes.c_int64 * max(1, len(shape)))()
    nd = ctypes.c_int32(0)
    _check(lib.muon_merge_small_dims(arr, len(shape), int(threshold), int(target_ndim), out, ctypes.byref(nd)))
    return tuple(int(out[i]) for i in range(nd.value))
