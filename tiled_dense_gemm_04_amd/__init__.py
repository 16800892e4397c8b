"""tiled_dense_gemm_04_amd -- Python binding of libtgemm (fp16 GEMM + fused ReLU on MI355X).

Argument marshalling only: every step of C = ReLU(A @ B) runs in the library's HIP
kernels (``csrc/``), reached through the C ABI declared in ``include/tgemm.h``. PyTorch
is used for device memory and streams. There is no CPU fallback: if ``libtgemm.so`` is
missing or cannot be loaded, every call raises.

The names mirror the C ABI: ``gemm_f16``, ``gemm_f16_cfg``, ``tgemm_strerror``,
``tgemm_version``, ``tgemm_num_configs``, ``tgemm_config_desc``, ``tgemm_select_config``,
``tgemm_tile_of``, ``tgemm_num_workgroups`` and ``tgemm_mfma_probe``; the instrumented
twin ``libtgemm_stamps.so`` (``stamps_lib()``, measurement tools only) adds
``tgemm_stamps_capacity``, ``tgemm_stamps_read`` and ``tgemm_stamps_clear``
(``include/tgemm_stamps.h``).
"""
from __future__ import annotations

import ctypes
import os

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(PKG_DIR, "libtgemm.so")
STAMPS_LIBRARY = os.path.join(PKG_DIR, "libtgemm_stamps.so")

TGEMM_OK = 0
TGEMM_EINVAL_DIM = -1
TGEMM_EINVAL_LD = -2
TGEMM_ENULL = -3
TGEMM_EDEVICE = -4
TGEMM_ELAUNCH = -5
TGEMM_EINVAL_CFG = -6
TGEMM_EALIGN = -7
SELECT_NOOP = -100
SELECT_ZERO_FILL = -101

# Every symbol include/tgemm.h declares.
EXPORTS = ("gemm_f16", "gemm_f16_cfg", "tgemm_strerror", "tgemm_version", "tgemm_num_configs",
           "tgemm_config_desc", "tgemm_select_config", "tgemm_tile_of", "tgemm_num_workgroups",
           "tgemm_mfma_probe")
# The extra symbols include/tgemm_stamps.h declares (instrumented build only).
STAMPS_EXPORTS = ("tgemm_stamps_capacity", "tgemm_stamps_read", "tgemm_stamps_clear")
PROBE_THREADS = 512          # TGEMM_PROBE_THREADS
PROBE_MFMA_PER_ITER = 16     # TGEMM_PROBE_MFMA_PER_ITER
PROBE_FLOP_PER_MFMA = 2 * 16 * 16 * 32


class TgemmError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {tgemm_strerror(code)} (code {code})")


class ConfigInfo(ctypes.Structure):
    _fields_ = [("block_m", ctypes.c_int32), ("block_n", ctypes.c_int32),
                ("block_k", ctypes.c_int32), ("stages", ctypes.c_int32),
                ("waves_m", ctypes.c_int32), ("waves_n", ctypes.c_int32),
                ("panel", ctypes.c_int32), ("xcd_remap", ctypes.c_int32),
                ("generic", ctypes.c_int32), ("lds_bytes", ctypes.c_int32),
                ("name", ctypes.c_char * 48)]

    def as_dict(self) -> dict:
        d = {f: getattr(self, f) for f, _ in self._fields_ if f != "name"}
        d["name"] = self.name.decode()
        return d


_lib = None
_stamps_lib = None


def _load(path: str, stamps: bool) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run `python -m tiled_dense_gemm_04_amd.build` "
                          "or __graft_entry__.build()")
    L = ctypes.CDLL(path)
    i64, p, i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
    L.gemm_f16.restype = i32
    L.gemm_f16.argtypes = [i64, i64, i64, p, i64, p, i64, p, i64, i32, p]
    L.gemm_f16_cfg.restype = i32
    L.gemm_f16_cfg.argtypes = [i32, i64, i64, i64, p, i64, p, i64, p, i64, i32, p]
    L.tgemm_strerror.restype = ctypes.c_char_p
    L.tgemm_strerror.argtypes = [i32]
    L.tgemm_version.restype = ctypes.c_char_p
    L.tgemm_version.argtypes = []
    L.tgemm_num_configs.restype = i32
    L.tgemm_num_configs.argtypes = []
    L.tgemm_config_desc.restype = i32
    L.tgemm_config_desc.argtypes = [i32, ctypes.POINTER(ConfigInfo)]
    L.tgemm_select_config.restype = i32
    L.tgemm_select_config.argtypes = [i64, i64, i64, p, i64, p, i64, p, i64]
    L.tgemm_tile_of.restype = i32
    L.tgemm_tile_of.argtypes = [i32, i64, i64, i64, ctypes.POINTER(i64), ctypes.POINTER(i64)]
    L.tgemm_num_workgroups.restype = i64
    L.tgemm_num_workgroups.argtypes = [i32, i64, i64]
    L.tgemm_mfma_probe.restype = i32
    L.tgemm_mfma_probe.argtypes = [i32, i32, p, p]
    if stamps:
        L.tgemm_stamps_capacity.restype = i32
        L.tgemm_stamps_capacity.argtypes = [ctypes.POINTER(i32), ctypes.POINTER(i32)]
        L.tgemm_stamps_read.restype = i32
        L.tgemm_stamps_read.argtypes = [ctypes.POINTER(ctypes.c_uint64), i64]
        L.tgemm_stamps_clear.restype = i32
        L.tgemm_stamps_clear.argtypes = []
    return L


def lib() -> ctypes.CDLL:
    """The loaded libtgemm.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        _lib = _load(LIBRARY, stamps=False)
    return _lib


def stamps_lib() -> ctypes.CDLL:
    """The instrumented libtgemm_stamps.so (measurement tools only)."""
    global _stamps_lib
    if _stamps_lib is None:
        _stamps_lib = _load(STAMPS_LIBRARY, stamps=True)
    return _stamps_lib


# ---------------------------------------------------------------- raw C-ABI calls
def gemm_f16_raw(M, N, K, A, lda, B, ldb, C, ldc, relu, stream, library=None) -> int:
    """The C call with integer pointers; returns the library's code."""
    return (library or lib()).gemm_f16(M, N, K, A, lda, B, ldb, C, ldc, int(relu), stream)


def gemm_f16_cfg_raw(idx, M, N, K, A, lda, B, ldb, C, ldc, relu, stream, library=None) -> int:
    return (library or lib()).gemm_f16_cfg(idx, M, N, K, A, lda, B, ldb, C, ldc, int(relu), stream)


def tgemm_strerror(code: int) -> str:
    return lib().tgemm_strerror(int(code)).decode()


def tgemm_version() -> str:
    return lib().tgemm_version().decode()


def tgemm_num_configs() -> int:
    return int(lib().tgemm_num_configs())


def tgemm_config_desc(idx: int) -> dict:
    info = ConfigInfo()
    rc = lib().tgemm_config_desc(int(idx), ctypes.byref(info))
    if rc != TGEMM_OK:
        raise TgemmError(rc, "tgemm_config_desc")
    return info.as_dict()


def tgemm_select_config(M, N, K, A=0, lda=None, B=0, ldb=None, C=0, ldc=None) -> int:
    lda = max(1, K) if lda is None else lda
    ldb = max(1, N) if ldb is None else ldb
    ldc = max(1, N) if ldc is None else ldc
    return int(lib().tgemm_select_config(M, N, K, A, lda, B, ldb, C, ldc))


def tgemm_tile_of(idx: int, M: int, N: int, wg: int):
    tm, tn = ctypes.c_int64(), ctypes.c_int64()
    rc = lib().tgemm_tile_of(idx, M, N, wg, ctypes.byref(tm), ctypes.byref(tn))
    if rc != TGEMM_OK:
        raise TgemmError(rc, "tgemm_tile_of")
    return tm.value, tn.value


def tgemm_num_workgroups(idx: int, M: int, N: int) -> int:
    return int(lib().tgemm_num_workgroups(idx, M, N))


def tgemm_mfma_probe(blocks: int, iters: int, out, stream=None, library=None) -> int:
    """Enqueue the MFMA throughput probe; out is a float32 device tensor of at least
    blocks * PROBE_THREADS elements. Returns the FLOP the launch performs."""
    import torch
    if out.dtype != torch.float32 or not out.is_cuda or out.numel() < blocks * PROBE_THREADS:
        raise ValueError("out must be a float32 device tensor of blocks * PROBE_THREADS elements")
    handle = torch.cuda.current_stream(out.device).cuda_stream if stream is None else (
        stream if isinstance(stream, int) else stream.cuda_stream)
    with torch.cuda.device(out.device):
        rc = (library or lib()).tgemm_mfma_probe(int(blocks), int(iters), out.data_ptr(), handle)
    if rc != TGEMM_OK:
        raise TgemmError(rc, "tgemm_mfma_probe")
    return blocks * (PROBE_THREADS // 64) * iters * PROBE_MFMA_PER_ITER * PROBE_FLOP_PER_MFMA


def tgemm_stamps_read(workgroups: int):
    """Rows [0, workgroups) of the instrumented build's stamp table, as a numpy uint64
    array of shape (workgroups, words) (synchronous)."""
    import numpy as np
    L = stamps_lib()
    nwg, words = ctypes.c_int(), ctypes.c_int()
    rc = L.tgemm_stamps_capacity(ctypes.byref(nwg), ctypes.byref(words))
    if rc != TGEMM_OK:
        raise TgemmError(rc, "tgemm_stamps_capacity")
    n = min(int(workgroups), nwg.value)
    buf = np.zeros((n, words.value), dtype=np.uint64)
    rc = L.tgemm_stamps_read(buf.ctypes.data_as(ctypes.POINTER(ctypes.c_uint64)), buf.size)
    if rc != TGEMM_OK:
        raise TgemmError(rc, "tgemm_stamps_read")
    return buf


def tgemm_stamps_clear() -> None:
    rc = stamps_lib().tgemm_stamps_clear()
    if rc != TGEMM_OK:
        raise TgemmError(rc, "tgemm_stamps_clear")


# ---------------------------------------------------------------- torch-tensor front end
def _operand(t, name):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != torch.float16:
        raise TypeError(f"{name} must be float16, got {t.dtype}")
    if t.dim() != 2:
        raise ValueError(f"{name} must be 2-D")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    rows, cols = t.shape
    if cols > 1 and t.stride(1) != 1:
        raise ValueError(f"{name} must be row-major (stride(1) == 1)")
    ld = t.stride(0) if rows > 1 else max(1, cols)
    return rows, cols, ld


def gemm_f16(a, b, c=None, relu: bool = True, stream=None, cfg: int | None = None, library=None):
    """C = ReLU(a @ b) (relu=True) or a @ b, through the library. a: (M, K) fp16,
    b: (K, N) fp16, c: (M, N) fp16 output (allocated if None). Row-major views with
    any row stride are accepted. ``stream`` is a torch.cuda.Stream or raw handle; by
    default the current stream of a's device. ``cfg`` forces a table config.
    ``library`` selects another loaded build (``stamps_lib()``); default libtgemm.so."""
    import torch
    M, K, lda = _operand(a, "a")
    K2, N, ldb = _operand(b, "b")
    if K2 != K:
        raise ValueError(f"inner dimensions differ: {tuple(a.shape)} @ {tuple(b.shape)}")
    if c is None:
        c = torch.empty((M, N), dtype=torch.float16, device=a.device)
    Mc, Nc, ldc = _operand(c, "c")
    if (Mc, Nc) != (M, N):
        raise ValueError(f"c has shape {tuple(c.shape)}, expected {(M, N)}")
    if not (a.device == b.device == c.device):
        raise ValueError("a, b and c must be on the same device")
    if stream is None:
        handle = torch.cuda.current_stream(a.device).cuda_stream
    elif isinstance(stream, int):
        handle = stream
    else:
        handle = stream.cuda_stream
    with torch.cuda.device(a.device):
        if cfg is None:
            rc = gemm_f16_raw(M, N, K, a.data_ptr(), lda, b.data_ptr(), ldb, c.data_ptr(), ldc,
                              relu, handle, library)
        else:
            rc = gemm_f16_cfg_raw(cfg, M, N, K, a.data_ptr(), lda, b.data_ptr(), ldb, c.data_ptr(),
                                  ldc, relu, handle, library)
    if rc != TGEMM_OK:
        raise TgemmError(rc, "gemm_f16" if cfg is None else f"gemm_f16_cfg[{cfg}]")
    return c


def configs() -> list:
    return [tgemm_config_desc(i) for i in range(tgemm_num_configs())]
