"""Python binding of libwsg.so: argument marshalling only.

Every step of the hot path runs in the HIP kernels of libwsg.so (built by
warp_specialized_gemm_amd/build.py); this module only checks tensor
dtypes/shapes, passes device pointers and the current torch stream through the
C ABI declared in include/wsg.h, and turns nonzero return codes into
exceptions. There is no fallback: if libwsg.so is missing or fails to load,
importing this package raises.

Names follow the C ABI: gemm_bias_relu, gemm_bias_relu_bf16,
gemm_bias_relu_ex, gemm_bias_relu_ex_noalloc, grouped_gemm_bias_relu_ex, attention_fwd, staged_copy,
staged_copy_ex, resolve_config, check_device_status, set_stream, get_stream, last_error, version.
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "WsgError", "Config", "lib", "library_path", "EXPORTS",
    "gemm_bias_relu", "gemm_bias_relu_bf16", "gemm_bias_relu_ex", "gemm_bias_relu_ex_noalloc",
    "grouped_gemm_bias_relu_ex", "attention_fwd", "resolve_config",
    "staged_copy", "staged_copy_ex", "check_device_status", "set_wait_stats", "read_wait_stats",
    "set_stream", "get_stream", "status_message",
    "last_error", "version", "WSG_FP32", "WSG_BF16", "WSG_FLAG_GENERAL_PRODUCER", "WSG_FLAG_NONTEMPORAL",
    "WSG_FLAG_HOMOGENEOUS", "WSG_FLAG_DIRECT_COPY", "WSG_FLAG_STREAM_K", "WSG_FLAG_NO_STREAM_K",
    "WSG_MAX_GROUPS", "WSG_NOALLOC_SCRATCH_BYTES",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libwsg.so")

WSG_OK = 0
WSG_EINVAL = -1
WSG_EUNSUPPORTED = -2
WSG_ELAUNCH = -3
WSG_ETIMEOUT = -4
WSG_FP32 = 0
WSG_BF16 = 1
WSG_FLAG_GENERAL_PRODUCER = 1
WSG_FLAG_NONTEMPORAL = 2
WSG_FLAG_HOMOGENEOUS = 4
WSG_FLAG_DIRECT_COPY = 8
WSG_FLAG_STREAM_K = 16
WSG_FLAG_NO_STREAM_K = 32
WSG_MAX_GROUPS = 64
WSG_NOALLOC_SCRATCH_BYTES = 75497472  # 72 MiB
WSG_STATUS_TIMEOUT = 1
WSG_STATUS_COPY = 2
WSG_STATUS_GEMM = 4
WSG_STATUS_ATTENTION = 8

# every function include/wsg.h declares
EXPORTS = (
    "gemm_bias_relu", "gemm_bias_relu_bf16", "gemm_bias_relu_ex", "gemm_bias_relu_ex_noalloc",
    "grouped_gemm_bias_relu_ex", "attention_fwd", "wsg_gemm_resolve_config", "staged_copy", "staged_copy_ex", "wsg_set_stream", "wsg_get_stream", "wsg_last_error",
    "wsg_check_device_status", "wsg_status_message", "wsg_set_wait_stats", "wsg_read_wait_stats", "wsg_version",
)


class WsgError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__("libwsg error %d: %s" % (code, message))
        self.code = code


class Config(ctypes.Structure):
    """struct wsg_config; zero fields mean "default"."""
    _fields_ = [("BM", ctypes.c_int), ("BN", ctypes.c_int), ("BK", ctypes.c_int),
                ("producer_waves", ctypes.c_int), ("consumer_waves", ctypes.c_int),
                ("copy_tile_bytes", ctypes.c_int), ("flags", ctypes.c_int), ("group_k", ctypes.c_int),
                ("copy_workgroups", ctypes.c_int)]

    def as_dict(self) -> dict:
        return {f: getattr(self, f) for f, _ in self._fields_}


def library_path() -> str:
    return _LIB_PATH


def _load() -> ctypes.CDLL:
    if not os.path.exists(_LIB_PATH):
        raise ImportError("libwsg.so is not built (%s); run __graft_entry__.build() or "
                          "python warp_specialized_gemm_amd/build.py" % _LIB_PATH)
    L = ctypes.CDLL(_LIB_PATH)
    i64, vp, ci = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
    cfgp = ctypes.POINTER(Config)
    sig = {
        "gemm_bias_relu": ([i64, i64, i64, vp, vp, vp, vp, ci], ci),
        "gemm_bias_relu_bf16": ([i64, i64, i64, vp, vp, vp, vp, ci], ci),
        "gemm_bias_relu_ex": ([ci, i64, i64, i64, vp, vp, vp, vp, ci, cfgp], ci),
        "gemm_bias_relu_ex_noalloc": ([ci, i64, i64, i64, vp, vp, vp, vp, ci, cfgp], ci),
        "grouped_gemm_bias_relu_ex": ([ci, ci, ctypes.POINTER(i64), i64, i64, vp, vp, vp, vp, ci, cfgp], ci),
        "attention_fwd": ([i64, i64, i64, i64, i64, vp, vp, vp, vp, ctypes.c_float, ci, ci, cfgp], ci),
        "wsg_gemm_resolve_config": ([ci, i64, i64, i64, ci, cfgp, cfgp], ci),
        "staged_copy": ([vp, vp, ctypes.c_size_t, ci], ci),
        "staged_copy_ex": ([vp, vp, ctypes.c_size_t, ci, cfgp], ci),
        "wsg_set_stream": ([vp], ci),
        "wsg_get_stream": ([], vp),
        "wsg_last_error": ([], ctypes.c_char_p),
        "wsg_check_device_status": ([], ci),
        "wsg_status_message": ([ctypes.c_uint], ctypes.c_char_p),
        "wsg_set_wait_stats": ([ci], ci),
        "wsg_read_wait_stats": ([ctypes.POINTER(ctypes.c_uint64)], ci),
        "wsg_version": ([], ctypes.c_char_p),
    }
    for name, (args, res) in sig.items():
        f = getattr(L, name)
        f.argtypes = args
        f.restype = res
    return L


lib = _load()


def _raise_on(rc: int) -> None:
    if rc != WSG_OK:
        raise WsgError(rc, lib.wsg_last_error().decode(errors="replace"))


def last_error() -> str:
    return lib.wsg_last_error().decode(errors="replace")


def version() -> str:
    return lib.wsg_version().decode()


def set_stream(stream) -> None:
    """Stream for this thread's later launches: a torch.cuda.Stream, an int handle or None."""
    handle = getattr(stream, "cuda_stream", stream)
    lib.wsg_set_stream(ctypes.c_void_p(handle or 0))


def get_stream() -> int:
    return lib.wsg_get_stream() or 0


def _use_current_stream() -> None:
    import torch
    lib.wsg_set_stream(ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


def _config(config) -> "ctypes.POINTER(Config) | None":
    if config is None:
        return None
    if isinstance(config, dict):
        c = Config()
        for k, v in config.items():
            setattr(c, k, int(v))
        config = c
    return ctypes.pointer(config)


def _gemm_operands(A, B, bias, C, want_dtype):
    import torch
    for name, t in (("A", A), ("B", B), ("bias", bias)):
        if not isinstance(t, torch.Tensor) or not t.is_cuda:
            raise TypeError("%s must be a CUDA (HIP) tensor" % name)
        if t.dtype not in want_dtype:
            raise TypeError("%s must have dtype in %s, got %s" % (name, want_dtype, t.dtype))
        if not t.is_contiguous():
            raise ValueError("%s must be contiguous (row-major)" % name)
    if A.dim() != 2 or B.dim() != 2 or bias.dim() != 1:
        raise ValueError("A must be MxK, B KxN and bias N")
    M, K = A.shape
    K2, N = B.shape
    if K2 != K or bias.shape[0] != N:
        raise ValueError("shape mismatch: A %s, B %s, bias %s" % (tuple(A.shape), tuple(B.shape),
                                                                  tuple(bias.shape)))
    if C is None:
        C = torch.empty((M, N), dtype=torch.float32, device=A.device)
    elif C.dtype != torch.float32 or tuple(C.shape) != (M, N) or not C.is_contiguous() or not C.is_cuda:
        raise ValueError("C must be a contiguous float32 CUDA tensor of shape (%d, %d)" % (M, N))
    return M, N, K, C


def gemm_bias_relu(A, B, bias, C=None, stages: int = 2):
    """C = relu(A @ B + bias) for float32 tensors; returns C. `stages` is the
    LDS ring depth; the GEMM calls default to 2, the fastest depth measured on
    MI355X for the default tiles (a deeper ring forces shallower k tiles)."""
    import torch
    M, N, K, C = _gemm_operands(A, B, bias, C, (torch.float32,))
    _use_current_stream()
    _raise_on(lib.gemm_bias_relu(M, N, K, A.data_ptr(), B.data_ptr(), bias.data_ptr(), C.data_ptr(), stages))
    return C


def _bf16_ok():
    import torch
    return (torch.bfloat16, torch.int16, torch.uint16)


def gemm_bias_relu_bf16(A, B, bias, C=None, stages: int = 2):
    """C = relu(A @ B + bias) for bf16 tensors (or their 16-bit patterns); fp32 C."""
    M, N, K, C = _gemm_operands(A, B, bias, C, _bf16_ok())
    _use_current_stream()
    _raise_on(lib.gemm_bias_relu_bf16(M, N, K, A.data_ptr(), B.data_ptr(), bias.data_ptr(), C.data_ptr(),
                                      stages))
    return C


def gemm_bias_relu_ex(A, B, bias, C=None, stages: int = 2, config=None):
    """Either GEMM with an explicit launch configuration (Config or dict)."""
    import torch
    if A.dtype == torch.float32:
        dtype, ok = WSG_FP32, (torch.float32,)
    else:
        dtype, ok = WSG_BF16, _bf16_ok()
    M, N, K, C = _gemm_operands(A, B, bias, C, ok)
    _use_current_stream()
    _raise_on(lib.gemm_bias_relu_ex(dtype, M, N, K, A.data_ptr(), B.data_ptr(), bias.data_ptr(), C.data_ptr(),
                                    stages, _config(config)))
    return C


def gemm_bias_relu_ex_noalloc(A, B, bias, C, stages: int = 2, config=None):
    """gemm_bias_relu_ex without any device allocation, by the library or
    here: C must be given; the stream-K workspace is the library's static
    per-device scratch array (calls that may overlap on one GPU race)."""
    import torch
    if C is None:
        raise ValueError("gemm_bias_relu_ex_noalloc allocates nothing: pass the output C")
    if A.dtype == torch.float32:
        dtype, ok = WSG_FP32, (torch.float32,)
    else:
        dtype, ok = WSG_BF16, _bf16_ok()
    M, N, K, C = _gemm_operands(A, B, bias, C, ok)
    _use_current_stream()
    _raise_on(lib.gemm_bias_relu_ex_noalloc(dtype, M, N, K, A.data_ptr(), B.data_ptr(), bias.data_ptr(),
                                            C.data_ptr(), stages, _config(config)))
    return C


def grouped_gemm_bias_relu_ex(A, B, bias, group_rows, C=None, stages: int = 2, config=None):
    """Mixture-of-experts GEMM: A's rows sorted by expert, group_rows[e] of them
    for expert e; B is (experts, K, N), bias (experts, N). Returns C (rows, N)
    with C[rows of e] = relu(A[rows of e] @ B[e] + bias[e])."""
    import torch
    if not isinstance(A, torch.Tensor):
        raise TypeError("A must be a CUDA (HIP) tensor")
    if A.dtype == torch.float32:
        dtype, ok = WSG_FP32, (torch.float32,)
    else:
        dtype, ok = WSG_BF16, _bf16_ok()
    for name, t in (("A", A), ("B", B), ("bias", bias)):
        if not isinstance(t, torch.Tensor) or not t.is_cuda:
            raise TypeError("%s must be a CUDA (HIP) tensor" % name)
        if t.dtype not in ok:
            raise TypeError("%s must have dtype in %s, got %s" % (name, ok, t.dtype))
        if not t.is_contiguous():
            raise ValueError("%s must be contiguous (row-major)" % name)
    rows = [int(r) for r in group_rows]
    G = len(rows)
    if A.dim() != 2 or B.dim() != 3 or bias.dim() != 2:
        raise ValueError("A must be rows x K, B experts x K x N and bias experts x N")
    M, K = A.shape
    if tuple(B.shape[:2]) != (G, K) or tuple(bias.shape) != (G, B.shape[2]) or sum(rows) != M:
        raise ValueError("shape mismatch: A %s, B %s, bias %s, %d experts with %d rows" % (
            tuple(A.shape), tuple(B.shape), tuple(bias.shape), G, sum(rows)))
    N = B.shape[2]
    if C is None:
        C = torch.empty((M, N), dtype=torch.float32, device=A.device)
    elif C.dtype != torch.float32 or tuple(C.shape) != (M, N) or not C.is_contiguous() or not C.is_cuda:
        raise ValueError("C must be a contiguous float32 CUDA tensor of shape (%d, %d)" % (M, N))
    counts = (ctypes.c_int64 * max(G, 1))(*rows)
    _use_current_stream()
    _raise_on(lib.grouped_gemm_bias_relu_ex(dtype, G, counts, N, K, A.data_ptr(), B.data_ptr(), bias.data_ptr(),
                                            C.data_ptr(), stages, _config(config)))
    return C


def attention_fwd(Q, K, V, O=None, scale=None, causal: bool = False, stages: int = 2, config=None):
    """O = softmax(scale * Q K^T [causal]) V; Q (batch, heads, Sq, D), K and V
    (batch, heads, Skv, D) as bf16 tensors or their 16-bit patterns; fp32 O.
    scale defaults to 1 / sqrt(D); it must be finite and at least 2^-126."""
    import math
    import torch
    ok = _bf16_ok()
    for name, t in (("Q", Q), ("K", K), ("V", V)):
        if not isinstance(t, torch.Tensor) or not t.is_cuda:
            raise TypeError("%s must be a CUDA (HIP) tensor" % name)
        if t.dtype not in ok:
            raise TypeError("%s must have dtype in %s, got %s" % (name, ok, t.dtype))
        if not t.is_contiguous() or t.dim() != 4:
            raise ValueError("%s must be a contiguous 4-d tensor (batch, heads, S, D)" % name)
    Bn, H, Sq, D = Q.shape
    if tuple(K.shape) != tuple(V.shape) or tuple(K.shape[:2]) != (Bn, H) or K.shape[3] != D:
        raise ValueError("shape mismatch: Q %s, K %s, V %s" % (tuple(Q.shape), tuple(K.shape), tuple(V.shape)))
    Skv = K.shape[2]
    if O is None:
        O = torch.empty((Bn, H, Sq, D), dtype=torch.float32, device=Q.device)
    elif O.dtype != torch.float32 or tuple(O.shape) != (Bn, H, Sq, D) or not O.is_contiguous() or not O.is_cuda:
        raise ValueError("O must be a contiguous float32 CUDA tensor of shape %s" % ((Bn, H, Sq, D),))
    if scale is None:
        scale = 1.0 / math.sqrt(D) if D else 1.0
    _use_current_stream()
    _raise_on(lib.attention_fwd(Bn, H, Sq, Skv, D, Q.data_ptr(), K.data_ptr(), V.data_ptr(), O.data_ptr(),
                                float(scale), 1 if causal else 0, stages, _config(config)))
    return O


def resolve_config(dtype: int, M: int, N: int, K: int, stages: int = 2, config=None) -> dict:
    """The launch configuration gemm_bias_relu_ex would use (no device work)."""
    out = Config()
    _raise_on(lib.wsg_gemm_resolve_config(dtype, M, N, K, stages, _config(config), ctypes.pointer(out)))
    return out.as_dict()


def _copy_operands(src, dst):
    import torch
    if not isinstance(src, torch.Tensor) or not src.is_cuda or not src.is_contiguous():
        raise TypeError("src must be a contiguous CUDA tensor")
    if dst is None:
        dst = torch.empty_like(src)
    if not dst.is_cuda or not dst.is_contiguous():
        raise TypeError("dst must be a contiguous CUDA tensor")
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() < nbytes:
        raise ValueError("dst is smaller than src")
    return dst, nbytes


def staged_copy(src, dst=None, stages: int = 2):
    """dst = src byte for byte through the LDS ring; returns dst."""
    dst, nbytes = _copy_operands(src, dst)
    _use_current_stream()
    _raise_on(lib.staged_copy(src.data_ptr(), dst.data_ptr(), nbytes, stages))
    return dst


def staged_copy_ex(src, dst=None, stages: int = 2, config=None):
    dst, nbytes = _copy_operands(src, dst)
    _use_current_stream()
    _raise_on(lib.staged_copy_ex(src.data_ptr(), dst.data_ptr(), nbytes, stages, _config(config)))
    return dst


def set_wait_stats(enable: bool) -> None:
    """Count flag waits per role in this thread's later launches (a diagnostic)."""
    _raise_on(lib.wsg_set_wait_stats(1 if enable else 0))


def read_wait_stats() -> dict:
    """Synchronize, read and clear the wait counters of the current device."""
    _use_current_stream()
    buf = (ctypes.c_uint64 * 16)()
    _raise_on(lib.wsg_read_wait_stats(buf))
    v = list(buf)
    names = ("gemm_consumer_full", "gemm_producer_empty", "copy_consumer_full", "copy_producer_empty",
             "attention_consumer_full")
    return {n: {"waits": v[3 * i], "blocked": v[3 * i + 1], "polls": v[3 * i + 2]} for i, n in enumerate(names)}


def status_message(word: int) -> str:
    """The text check_device_status reports for a device status word (host only)."""
    return lib.wsg_status_message(int(word) & 0xFFFFFFFF).decode()


def check_device_status() -> None:
    """Synchronize the current stream and raise WsgError if a ring wait gave up."""
    _use_current_stream()
    _raise_on(lib.wsg_check_device_status())
