"""Python binding of libtara.so, the MI355X (gfx950) TARA attention library.

Thin ctypes marshalling over the C ABI in include/tara.h: the functions keep
the C names (tara_attn_fwd, tara_workspace_bytes, ...), take torch tensors for
device buffers and pass their pointers, strides and the current HIP stream.
Every step of the computation runs in the library's kernels; there is no
fallback path. If libtara.so is missing, calls raise TaraLibraryMissing.

What is computed ("TARA: Native Temporal Alignment for MiniMax H3
References", section "The temporal rule"; "BFS H3 Reference Attention Binding
(Experimental)", section "The exact rule"): softmax attention over a packed
sequence where target-query x guide-key logits lose
min(strength*(max(|t_q - t_k| - window, 0)/falloff)^2, cap) and, with binding,
target-query x picture-key logits gain m*ln(gain) (chained bindings add their
terms, section "Common issues").
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

__all__ = [
    "TARA_SEG_TARGET", "TARA_SEG_GUIDE", "TARA_SEG_PICTURE", "TARA_SEG_OTHER",
    "TARA_BF16", "TARA_FP32", "TARA_MODE_FUSED", "TARA_MODE_PARTITIONED", "TARA_MODE_THREE_TERM",
    "TARA_MODE_DENSE_BIAS", "TARA_MODE_FRAME_LOOP", "TARA_PROBE_CONSTANT", "TARA_PROBE_RANDOM",
    "TaraError", "TaraLibraryMissing", "TaraParams", "TaraRunInfo",
    "tara_params_default", "make_params", "tara_workspace_bytes", "tara_attn_fwd", "tara_attn_fwd_noalloc",
    "tara_status_string", "tara_last_error", "tara_get_last_run_info",
    "tara_timing_enable", "tara_timing_read", "tara_probe_mfma_bf16", "attn_fwd", "library_path",
    "load_library",
    "EXPORTED_SYMBOLS",
]

TARA_SEG_TARGET, TARA_SEG_GUIDE, TARA_SEG_PICTURE, TARA_SEG_OTHER = 0, 1, 2, 3
TARA_BF16, TARA_FP32 = 0, 1
TARA_MODE_FUSED, TARA_MODE_PARTITIONED, TARA_MODE_THREE_TERM = 0, 1, 2
TARA_MODE_DENSE_BIAS, TARA_MODE_FRAME_LOOP = 3, 4   # baselines for comparison
TARA_MAX_PICTURES = 16
TARA_MAX_BINDINGS = 4
TARA_MAX_PARTITIONS = 64

EXPORTED_SYMBOLS = (
    "tara_params_default", "tara_workspace_bytes", "tara_attn_fwd", "tara_status_string",
    "tara_last_error", "tara_get_last_run_info", "tara_timing_enable", "tara_timing_read",
    "tara_probe_mfma_bf16", "tara_attn_fwd_noalloc",
)

_PKG = os.path.dirname(os.path.abspath(__file__))


def library_path() -> str:
    return os.environ.get("TARA_LIBRARY", os.path.join(_PKG, "libtara.so"))


class TaraLibraryMissing(RuntimeError):
    pass


class TaraError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        self.detail = detail
        super().__init__(f"tara error {status} ({tara_status_string(status)}): {detail}")


class TaraParams(ctypes.Structure):
    _fields_ = [
        ("window", ctypes.c_float),
        ("falloff", ctypes.c_float),
        ("strength", ctypes.c_float),
        ("cap", ctypes.c_float),
        ("binding_enabled", ctypes.c_int),
        ("num_pictures", ctypes.c_int),
        ("num_bindings", ctypes.c_int),
        ("picture_gain", (ctypes.c_float * TARA_MAX_PICTURES) * TARA_MAX_BINDINGS),
        ("softmax_scale", ctypes.c_float),
        ("mode", ctypes.c_int),
        ("num_partitions", ctypes.c_int),
        ("partition_bounds", ctypes.POINTER(ctypes.c_int32)),
        ("qk8", ctypes.c_int),
    ]


class TaraRunInfo(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in (
        "mode", "dtype", "bias_active", "binding_active", "num_partitions",
        "block_q", "block_k", "grid", "launches", "elem_all", "tile_stats", "tail_parts")] + [
        (n, ctypes.c_longlong) for n in (
            "tiles_plain", "tiles_saturated", "tiles_window", "tiles_picture", "tiles_elem")]

    def as_dict(self):
        return {n: getattr(self, n) for n, _ in self._fields_}


_lib = None


def load_library():
    """Loads libtara.so once and declares the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise TaraLibraryMissing(
            f"{path} is not built; run `python -m temporally_biased_flashattention_amd.build`")
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    I64_3 = ctypes.POINTER(ctypes.c_int64)
    lib.tara_params_default.argtypes = [ctypes.POINTER(TaraParams)]
    lib.tara_params_default.restype = None
    lib.tara_workspace_bytes.argtypes = [ctypes.c_int] * 5 + [ctypes.POINTER(TaraParams)]
    lib.tara_workspace_bytes.restype = ctypes.c_size_t
    lib.tara_attn_fwd.argtypes = ([P, P, P, P, P, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_int, I64_3, I64_3, I64_3, I64_3, P, P, P, P,
                                   ctypes.POINTER(TaraParams), P, ctypes.c_size_t, P])
    lib.tara_attn_fwd.restype = ctypes.c_int
    lib.tara_attn_fwd_noalloc.argtypes = ([P, P, P, P, P, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                           ctypes.c_int, I64_3, I64_3, I64_3, I64_3, P, P, P, P,
                                           ctypes.POINTER(TaraParams), P])
    lib.tara_attn_fwd_noalloc.restype = ctypes.c_int
    lib.tara_status_string.argtypes = [ctypes.c_int]
    lib.tara_status_string.restype = ctypes.c_char_p
    lib.tara_last_error.argtypes = []
    lib.tara_last_error.restype = ctypes.c_char_p
    lib.tara_get_last_run_info.argtypes = [ctypes.POINTER(TaraRunInfo)]
    lib.tara_get_last_run_info.restype = ctypes.c_int
    lib.tara_timing_enable.argtypes = [ctypes.c_int]
    lib.tara_timing_enable.restype = ctypes.c_int
    lib.tara_timing_read.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_int, ctypes.POINTER(ctypes.c_int)]
    lib.tara_timing_read.restype = ctypes.c_int
    lib.tara_probe_mfma_bf16.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_float), ctypes.c_void_p]
    lib.tara_probe_mfma_bf16.restype = ctypes.c_int
    _lib = lib
    return lib


# ----------------------------------------------------------------- params
def tara_params_default() -> TaraParams:
    p = TaraParams()
    load_library().tara_params_default(ctypes.byref(p))
    return p


def make_params(window: float = 0.20, falloff: float = 0.25, strength: float = 2.0, cap: float = 6.0,
                binding: bool = False, gains: Sequence[float] = (), softmax_scale: float = 0.0,
                mode: str = "fused", partitions: int = 1,
                bounds: Optional[Sequence[int]] = None,
                chained: Sequence[Sequence[float]] = (), qk8: bool = False) -> TaraParams:
    """Builds tara_params_t. gains[i] is the gain of 0-based picture id i
    under the first binding; chained[j][i] that under binding j + 1; qk8
    selects the 8-bit Q.K product (bf16, fused mode)."""
    p = tara_params_default()
    p.window, p.falloff, p.strength, p.cap = window, falloff, strength, cap
    p.binding_enabled = int(bool(binding))
    p.num_pictures = len(gains)
    if len(gains) > TARA_MAX_PICTURES:
        raise ValueError("at most 16 pictures")
    if 1 + len(chained) > TARA_MAX_BINDINGS:
        raise ValueError("at most 4 bindings")
    p.num_bindings = 1 + len(chained)
    for j, gs in enumerate((tuple(gains),) + tuple(tuple(c) for c in chained)):
        if len(gs) != len(gains):
            raise ValueError("every binding gives one gain per picture")
        for i, g in enumerate(gs):
            p.picture_gain[j][i] = g
    p.softmax_scale = softmax_scale
    p.mode = {"fused": TARA_MODE_FUSED, "partitioned": TARA_MODE_PARTITIONED,
              "three-term": TARA_MODE_THREE_TERM, "dense-bias": TARA_MODE_DENSE_BIAS,
              "frame-loop": TARA_MODE_FRAME_LOOP}[mode]
    p.num_partitions = int(partitions)
    if bounds is not None:
        arr = (ctypes.c_int32 * len(bounds))(*[int(x) for x in bounds])
        p._bounds_keepalive = arr  # noqa: SLF001 (keeps the host array alive)
        p.partition_bounds = ctypes.cast(arr, ctypes.POINTER(ctypes.c_int32))
    p.qk8 = int(bool(qk8))
    return p


# ----------------------------------------------------------------- calls
def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return TARA_BF16
    if t.dtype == torch.float32:
        return TARA_FP32
    return 99  # rejected by the library as TARA_ERR_UNSUPPORTED_DTYPE


def _strides(t):
    if t.dim() != 4:
        raise ValueError("q, k, v and o must be 4-D [B, H, N, D] tensors (views allowed)")
    if t.shape[-1] > 1 and t.stride(-1) != 1:
        raise ValueError("the head dimension must be contiguous (stride 1)")
    return (ctypes.c_int64 * 3)(t.stride(0), t.stride(1), t.stride(2))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check(status: int):
    if status != 0:
        raise TaraError(status, tara_last_error())


def tara_workspace_bytes(dtype: int, B: int, H: int, N: int, D: int, params: TaraParams) -> int:
    n = load_library().tara_workspace_bytes(dtype, B, H, N, D, ctypes.byref(params))
    if n == ctypes.c_size_t(-1).value:
        raise TaraError(-6, "tara_workspace_bytes rejected the arguments")
    return int(n)


def _check_call_args(q, k, v, o, lse, seg_type, token_time, picture_id, mask_weight, params, workspace):
    """Raises ValueError unless every buffer has the device, dtype, shape and
    layout tara_attn_fwd reads or writes, so that no kernel is launched on a
    buffer too small for it. Shapes and dtypes are checked before devices."""
    import torch

    def need(cond, msg):
        if not cond:
            raise ValueError(msg)

    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("lse", lse), ("seg_type", seg_type),
                    ("token_time", token_time)):
        need(isinstance(t, torch.Tensor), f"{name} must be a torch tensor")
    need(q.dim() == 4, "q must be 4-D [B, H, N, D] (views allowed)")
    B, H, N, D = q.shape
    for name, t in (("k", k), ("v", v), ("o", o)):
        need(t.shape == q.shape, f"{name} has shape {tuple(t.shape)}, q has {tuple(q.shape)}")
        need(t.dtype == q.dtype, f"{name} is {t.dtype}, q is {q.dtype}")
    need(lse.dtype == torch.float32 and tuple(lse.shape) == (B, H, N) and lse.is_contiguous(),
         f"lse must be contiguous float32 [{B}, {H}, {N}]")
    need(seg_type.dtype == torch.uint8 and tuple(seg_type.shape) == (B, N) and seg_type.is_contiguous(),
         f"seg_type must be contiguous uint8 [{B}, {N}]")
    need(token_time.dtype == torch.float32 and tuple(token_time.shape) == (B, N) and token_time.is_contiguous(),
         f"token_time must be contiguous float32 [{B}, {N}]")
    if picture_id is not None:
        need(isinstance(picture_id, torch.Tensor) and picture_id.dtype == torch.int16
             and tuple(picture_id.shape) == (B, N) and picture_id.is_contiguous(),
             f"picture_id must be contiguous int16 [{B}, {N}] or None")
    if mask_weight is not None:
        need(isinstance(mask_weight, torch.Tensor) and mask_weight.dtype == torch.float32
             and mask_weight.is_contiguous(), "mask_weight must be a contiguous float32 tensor or None")
        if params.binding_enabled:
            # planes [J, B, N]; the library reads the first num_bindings of them
            nb = max(int(params.num_bindings), 1)
            want = (B, N) if nb == 1 else (nb, B, N)
            need(mask_weight.dim() >= 2 and tuple(mask_weight.shape[-2:]) == (B, N)
                 and mask_weight.numel() >= nb * B * N,
                 f"mask_weight must hold {list(want)} (one [B, N] plane per binding), got {tuple(mask_weight.shape)}")
    if workspace is not None:
        need(isinstance(workspace, torch.Tensor) and workspace.is_contiguous(),
             "workspace must be a contiguous tensor")
    dev = q.device
    need(dev.type == "cuda", f"q is on {dev}; tara_attn_fwd needs HIP device tensors")
    for name, t in (("k", k), ("v", v), ("o", o), ("lse", lse), ("seg_type", seg_type),
                    ("token_time", token_time), ("picture_id", picture_id), ("mask_weight", mask_weight),
                    ("workspace", workspace)):
        if t is not None:
            need(t.device == dev, f"{name} is on {t.device}, q is on {dev}")


def tara_attn_fwd(q, k, v, o, lse, seg_type, token_time, picture_id, mask_weight,
                  params: TaraParams, workspace, stream=None) -> None:
    """Calls tara_attn_fwd on torch device tensors.

    q, k, v, o: [B, H, N, D] (any strides with a contiguous last dim);
    lse: fp32 [B, H, N] contiguous; seg_type uint8 [B, N]; token_time fp32
    [B, N]; picture_id int16 [B, N] or None; mask_weight fp32 [B, N] (one
    binding), [J, B, N] (J chained bindings, contiguous) or None;
    workspace: a byte tensor of at least tara_workspace_bytes(...) bytes.
    stream: a torch.cuda.Stream (default: the current stream).
    Buffers of the wrong device, dtype, shape or layout raise ValueError
    before the library is called.
    """
    import torch
    _check_call_args(q, k, v, o, lse, seg_type, token_time, picture_id, mask_weight, params, workspace)
    lib = load_library()
    B, H, N, D = q.shape
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    elif stream.device != q.device:
        raise ValueError(f"stream is on {stream.device}, q is on {q.device}")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.tara_attn_fwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _dtype_code(q), B, H, N, D,
        _strides(q), _strides(k), _strides(v), _strides(o),
        _ptr(seg_type), _ptr(token_time), _ptr(picture_id), _ptr(mask_weight),
        ctypes.byref(params), _ptr(workspace), ws_bytes, ctypes.c_void_p(stream.cuda_stream))
    _check(st)


def tara_attn_fwd_noalloc(q, k, v, o, lse, seg_type, token_time, picture_id, mask_weight,
                          params: TaraParams, stream=None) -> None:
    """Calls tara_attn_fwd_noalloc: tara_attn_fwd without a workspace (the
    library's fixed device array serves as one; see include/tara.h). Same
    tensor rules as tara_attn_fwd."""
    import torch
    _check_call_args(q, k, v, o, lse, seg_type, token_time, picture_id, mask_weight, params, None)
    lib = load_library()
    B, H, N, D = q.shape
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    elif stream.device != q.device:
        raise ValueError(f"stream is on {stream.device}, q is on {q.device}")
    st = lib.tara_attn_fwd_noalloc(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _dtype_code(q), B, H, N, D,
        _strides(q), _strides(k), _strides(v), _strides(o),
        _ptr(seg_type), _ptr(token_time), _ptr(picture_id), _ptr(mask_weight),
        ctypes.byref(params), ctypes.c_void_p(stream.cuda_stream))
    _check(st)


def tara_status_string(status: int) -> str:
    return load_library().tara_status_string(status).decode()


def tara_last_error() -> str:
    return load_library().tara_last_error().decode()


def tara_get_last_run_info() -> dict:
    info = TaraRunInfo()
    _check(load_library().tara_get_last_run_info(ctypes.byref(info)))
    return info.as_dict()


def tara_timing_enable(on: bool) -> None:
    _check(load_library().tara_timing_enable(int(bool(on))))


def tara_timing_read(max_count: int = 4096):
    buf = (ctypes.c_float * max(max_count, 1))()
    n = ctypes.c_int(0)
    _check(load_library().tara_timing_read(buf, max_count, ctypes.byref(n)))
    return [float(buf[i]) for i in range(n.value)]


TARA_PROBE_CONSTANT = 0
TARA_PROBE_RANDOM = 1


def tara_probe_mfma_bf16(iterations: int = 20000, operands: int = TARA_PROBE_RANDOM, stream=None) -> float:
    """Rate (TFLOP/s) of a kernel of back-to-back bf16 MFMAs on the current
    device, on constant (TARA_PROBE_CONSTANT) or varied (TARA_PROBE_RANDOM)
    register operands."""
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    out = ctypes.c_float(0.0)
    _check(load_library().tara_probe_mfma_bf16(int(iterations), int(operands), ctypes.byref(out),
                                               ctypes.c_void_p(stream.cuda_stream)))
    return float(out.value)


def attn_fwd(q, k, v, seg_type, token_time, picture_id=None, mask_weight=None,
             params: Optional[TaraParams] = None, out=None, lse=None, workspace=None):
    """Allocates O, LSE and the workspace with torch, then calls tara_attn_fwd.

    Returns (O, LSE): O like q (contiguous [B, H, N, D]), LSE fp32 [B, H, N].
    """
    import torch
    if params is None:
        params = tara_params_default()
    B, H, N, D = q.shape
    if out is None:
        out = torch.empty((B, H, N, D), dtype=q.dtype, device=q.device)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    if workspace is None:
        nbytes = tara_workspace_bytes(_dtype_code(q), B, H, N, D, params)
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    tara_attn_fwd(q, k, v, out, lse, seg_type, token_time, picture_id, mask_weight, params, workspace)
    return out, lse
