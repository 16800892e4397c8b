"""tiled_dense_gemm_04_amd -- Python binding of libtgemm (fp16 GEMM + fused ReLU on MI355X).

Argument marshalling only: every step of C = ReLU(A @ B) runs in the library's HIP
kernels (``csrc/``), reached through the C ABI declared in ``include/tgemm.h``. PyTorch
is used for device memory and streams. There is no CPU fallback: if ``libtgemm.so`` is
missing or cannot be loaded, every call raises.

The names mirror the C ABI: ``gemm_f16``, ``gemm_f16_ex`` (transposed operands),
``gemm_f16_cfg``, ``gemm_f16_ex_cfg`` (as ``cfg=``), ``tgemm_strerror``, ``tgemm_version``,
``tgemm_num_configs``, ``tgemm_config_desc``, ``tgemm_select_config``,
``tgemm_select_config_ex``, ``tgemm_tile_of``, ``tgemm_split_tile_of``, ``tgemm_num_workgroups``, and split-K: ``gemm_f16_ws`` (workspace managed here per device and
stream unless given), ``gemm_f16_ws_cfg`` (as ``cfg=``/``splits=``),
``tgemm_workspace_bytes``, ``tgemm_workspace_bytes_cfg`` and ``tgemm_split_plan``, and
``gemm_f16_ws_static`` (split-K scratch in a static device array: allocates nothing); grouped
GEMMs: ``gemm_f16_grouped``;
the fp8 (E4M3) block-scaled path: ``gemm_fp8_block`` (``gemm_fp8_block_cfg`` as
``cfg=``), ``quant_fp8_block``, ``tgemm_fp8_num_configs``, ``tgemm_fp8_config_desc``,
``tgemm_fp8_select_config``, and ``fp8_block_scaled_linear`` (quantize x per 1 x 128
block, then the block-scaled GEMM against an fp8 weight). ``matmul`` takes row- or
column-major operand views and picks the layout; ``GemmFunction`` is the autograd wrapper (backward: dA = dC B^T, dB = A^T dC
through gemm_f16_ex). The tooling
twin ``libtgemm_stamps.so`` (``stamps_lib()``, measurement tools only) compiles every config
row (the sweep-only variants too; ``built`` in a config description says whether the
library at hand has the row) and adds ``tgemm_stamps_capacity``, ``tgemm_stamps_read``,
``tgemm_stamps_clear``, the MFMA throughput probe ``tgemm_mfma_probe`` and the LDS access
probe ``tgemm_lds_probe`` (``include/tgemm_stamps.h``).
"""
from __future__ import annotations

import ctypes
import os

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(PKG_DIR, "libtgemm.so")
STAMPS_LIBRARY = os.path.join(PKG_DIR, "libtgemm_stamps.so")
DEBUGFILL_LIBRARY = os.path.join(PKG_DIR, "libtgemm_debugfill.so")

TGEMM_OK = 0
TGEMM_EINVAL_DIM = -1
TGEMM_EINVAL_LD = -2
TGEMM_ENULL = -3
TGEMM_EDEVICE = -4
TGEMM_ELAUNCH = -5
TGEMM_EINVAL_CFG = -6
TGEMM_EALIGN = -7
TGEMM_EWORKSPACE = -8
SELECT_NOOP = -100
SELECT_ZERO_FILL = -101
FP8_GENERIC = -102           # TGEMM_FP8_GENERIC
FP8_BLOCK = 128

# Every symbol include/tgemm.h declares.
EXPORTS = ("gemm_f16", "gemm_f16_ex", "gemm_f16_cfg", "gemm_f16_ex_cfg", "tgemm_strerror",
           "tgemm_version", "tgemm_num_configs", "tgemm_config_desc", "tgemm_select_config",
           "tgemm_select_config_ex", "tgemm_tile_of", "tgemm_split_tile_of", "tgemm_num_workgroups",
           "gemm_f16_ws", "gemm_f16_ws_cfg", "tgemm_workspace_bytes", "tgemm_split_plan",
           "gemm_f16_grouped", "gemm_fp8_block", "gemm_fp8_block_cfg", "quant_fp8_block",
           "tgemm_fp8_num_configs", "tgemm_fp8_config_desc", "tgemm_fp8_select_config",
           "tgemm_workspace_bytes_cfg", "gemm_f16_ws_static")
# The extra symbols include/tgemm_stamps.h declares (tooling build only).
STAMPS_EXPORTS = ("tgemm_stamps_capacity", "tgemm_stamps_read", "tgemm_stamps_clear", "tgemm_mfma_probe",
                  "tgemm_mfma_probe_ex", "tgemm_lds_probe")
# LDS probe instruction kinds (TGEMM_LDS_*) and their access widths in bytes.
LDS_OPS = {"read_b32": (0, 4), "read_b64": (1, 8), "read_b128": (2, 16), "write_b32": (3, 4),
           "write_b64": (4, 8), "write_b128": (5, 16), "read_tr16_b64": (6, 8)}
STATIC_SCRATCH_BYTES = 4096 + (64 << 20)   # TGEMM_STATIC_SCRATCH_BYTES
FAST_MAX_LD = 1 << 22        # TGEMM_FAST_MAX_LD
PROBE_THREADS = 512          # TGEMM_PROBE_THREADS
PROBE_MFMA_PER_ITER = 16     # TGEMM_PROBE_MFMA_PER_ITER
PROBE_FLOP_PER_MFMA = 2 * 16 * 16 * 32
# MFMA probe modes (TGEMM_PROBE_*): operand source and MFMA shape.
PROBE_MODES = {"synthetic": 0, "operands": 1, "operands_32x32": 2, "lds_reads": 3}


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
                ("layouts", ctypes.c_int32), ("built", ctypes.c_int32), ("name", ctypes.c_char * 48)]

    def as_dict(self) -> dict:
        d = {f: getattr(self, f) for f, _ in self._fields_ if f != "name"}
        d["name"] = self.name.decode()
        return d


class GemmDesc(ctypes.Structure):
    """tgemm_gemm_desc"""
    _fields_ = [("M", ctypes.c_int64), ("N", ctypes.c_int64), ("K", ctypes.c_int64),
                ("A", ctypes.c_void_p), ("lda", ctypes.c_int64), ("B", ctypes.c_void_p),
                ("ldb", ctypes.c_int64), ("C", ctypes.c_void_p), ("ldc", ctypes.c_int64)]


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
    L.gemm_f16_ex.restype = i32
    L.gemm_f16_ex.argtypes = [i32, i32, i64, i64, i64, p, i64, p, i64, p, i64, i32, p]
    L.gemm_f16_ex_cfg.restype = i32
    L.gemm_f16_ex_cfg.argtypes = [i32, i32, i32, i64, i64, i64, p, i64, p, i64, p, i64, i32, p]
    L.tgemm_select_config_ex.restype = i32
    L.tgemm_select_config_ex.argtypes = [i32, i32, i64, i64, i64, p, i64, p, i64, p, i64]
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
    L.tgemm_split_tile_of.restype = i32
    L.tgemm_split_tile_of.argtypes = [i32, i64, i64, i32, i64, ctypes.POINTER(i64), ctypes.POINTER(i64),
                                      ctypes.POINTER(i32)]
    L.tgemm_num_workgroups.restype = i64
    L.tgemm_num_workgroups.argtypes = [i32, i64, i64]
    L.gemm_f16_ws.restype = i32
    L.gemm_f16_ws.argtypes = [i32, i32, i64, i64, i64, p, i64, p, i64, p, i64, i32, p, i64, p]
    L.gemm_f16_ws_cfg.restype = i32
    L.gemm_f16_ws_cfg.argtypes = [i32, i32, i32, i32, i64, i64, i64, p, i64, p, i64, p, i64, i32, p, i64, p]
    L.tgemm_workspace_bytes.restype = i64
    L.tgemm_workspace_bytes.argtypes = [i32, i32, i64, i64, i64]
    L.tgemm_workspace_bytes_cfg.restype = i64
    L.tgemm_workspace_bytes_cfg.argtypes = [i32, i32, i64, i64]
    L.gemm_f16_ws_static.restype = i32
    L.gemm_f16_ws_static.argtypes = [i32, i32, i64, i64, i64, p, i64, p, i64, p, i64, i32, p]
    L.gemm_f16_grouped.restype = i32
    L.gemm_f16_grouped.argtypes = [i32, i32, i32, ctypes.POINTER(GemmDesc), i32, p]
    L.tgemm_split_plan.restype = i32
    L.tgemm_split_plan.argtypes = [i32, i32, i64, i64, i64, p, i64, p, i64, p, i64, ctypes.POINTER(i32),
                                   ctypes.POINTER(i32), ctypes.POINTER(i64)]
    L.gemm_fp8_block.restype = i32
    L.gemm_fp8_block.argtypes = [i64, i64, i64, p, i64, p, p, i64, p, p, i64, i32, p]
    L.gemm_fp8_block_cfg.restype = i32
    L.gemm_fp8_block_cfg.argtypes = [i32, i64, i64, i64, p, i64, p, p, i64, p, p, i64, i32, p]
    L.quant_fp8_block.restype = i32
    L.quant_fp8_block.argtypes = [i64, i64, p, i64, i32, p, i64, p, p]
    L.tgemm_fp8_num_configs.restype = i32
    L.tgemm_fp8_num_configs.argtypes = []
    L.tgemm_fp8_config_desc.restype = i32
    L.tgemm_fp8_config_desc.argtypes = [i32, ctypes.POINTER(ConfigInfo)]
    L.tgemm_fp8_select_config.restype = i32
    L.tgemm_fp8_select_config.argtypes = [i64, i64, i64, p, i64, p, i64, p, i64]
    if stamps:
        L.tgemm_stamps_capacity.restype = i32
        L.tgemm_stamps_capacity.argtypes = [ctypes.POINTER(i32), ctypes.POINTER(i32)]
        L.tgemm_stamps_read.restype = i32
        L.tgemm_stamps_read.argtypes = [ctypes.POINTER(ctypes.c_uint64), i64]
        L.tgemm_stamps_clear.restype = i32
        L.tgemm_stamps_clear.argtypes = []
        L.tgemm_mfma_probe.restype = i32
        L.tgemm_mfma_probe.argtypes = [i32, i32, p, p]
        L.tgemm_mfma_probe_ex.restype = i32
        L.tgemm_mfma_probe_ex.argtypes = [i32, i32, i32, p, p, p]
        L.tgemm_lds_probe.restype = i32
        L.tgemm_lds_probe.argtypes = [i32, ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_uint64), i32, i32,
                                      i32, p, p]
    return L


def lib() -> ctypes.CDLL:
    """The loaded libtgemm.so (raises if it has not been built). The environment variable
    TGEMM_LIBRARY names another build with the same ABI to load instead (for instance
    libtgemm_debugfill.so, to run a whole test suite on the NaN-poisoning build)."""
    global _lib
    if _lib is None:
        _lib = _load(os.environ.get("TGEMM_LIBRARY") or LIBRARY, stamps=False)
    return _lib


_debugfill_lib = None


def debugfill_lib() -> ctypes.CDLL:
    """The debugging build libtgemm_debugfill.so (TGEMM_DEBUG_FILL: LDS copy destinations
    are NaN-poisoned before every copy); same ABI as libtgemm.so."""
    global _debugfill_lib
    if _debugfill_lib is None:
        _debugfill_lib = _load(DEBUGFILL_LIBRARY, stamps=False)
    return _debugfill_lib


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


def gemm_f16_ex_raw(ta, tb, M, N, K, A, lda, B, ldb, C, ldc, relu, stream, library=None) -> int:
    return (library or lib()).gemm_f16_ex(int(ta), int(tb), M, N, K, A, lda, B, ldb, C, ldc, int(relu),
                                          stream)


def gemm_f16_ex_cfg_raw(idx, ta, tb, M, N, K, A, lda, B, ldb, C, ldc, relu, stream, library=None) -> int:
    return (library or lib()).gemm_f16_ex_cfg(idx, int(ta), int(tb), M, N, K, A, lda, B, ldb, C, ldc,
                                              int(relu), stream)


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


def tgemm_select_config(M, N, K, A=256, lda=None, B=256, ldb=None, C=256, ldc=None) -> int:
    """Config index gemm_f16 would use for these arguments (the pointers are only checked
    for null and alignment, never dereferenced: the defaults stand for aligned buffers)."""
    lda = max(1, K) if lda is None else lda
    ldb = max(1, N) if ldb is None else ldb
    ldc = max(1, N) if ldc is None else ldc
    return int(lib().tgemm_select_config(M, N, K, A, lda, B, ldb, C, ldc))


def tgemm_select_config_ex(trans_a, trans_b, M, N, K, A=256, lda=None, B=256, ldb=None, C=256, ldc=None) -> int:
    lda = max(1, M if trans_a else K) if lda is None else lda
    ldb = max(1, K if trans_b else N) if ldb is None else ldb
    ldc = max(1, N) if ldc is None else ldc
    return int(lib().tgemm_select_config_ex(int(trans_a), int(trans_b), M, N, K, A, lda, B, ldb, C, ldc))


def tgemm_workspace_bytes(trans_a, trans_b, M, N, K) -> int:
    return int(lib().tgemm_workspace_bytes(int(trans_a), int(trans_b), M, N, K))


def tgemm_workspace_bytes_cfg(idx, splits, M, N) -> int:
    """Workspace bytes gemm_f16_ws_cfg needs for config idx with `splits` splits over an
    M x N output (raises for a combination the library would reject)."""
    n = int(lib().tgemm_workspace_bytes_cfg(int(idx), int(splits), M, N))
    if n < 0:
        raise TgemmError(n, f"tgemm_workspace_bytes_cfg[{idx}, {splits}]")
    return n


def tgemm_split_plan(trans_a, trans_b, M, N, K, A=256, lda=None, B=256, ldb=None, C=256, ldc=None):
    """(config index, splits, workspace bytes) gemm_f16_ws would use (pure host logic)."""
    lda = max(1, M if trans_a else K) if lda is None else lda
    ldb = max(1, K if trans_b else N) if ldb is None else ldb
    ldc = max(1, N) if ldc is None else ldc
    cfg, sp, wb = ctypes.c_int(), ctypes.c_int(), ctypes.c_int64()
    rc = lib().tgemm_split_plan(int(trans_a), int(trans_b), M, N, K, A, lda, B, ldb, C, ldc,
                                ctypes.byref(cfg), ctypes.byref(sp), ctypes.byref(wb))
    if rc != TGEMM_OK:
        raise TgemmError(rc, "tgemm_split_plan")
    return cfg.value, sp.value, wb.value


def tgemm_tile_of(idx: int, M: int, N: int, wg: int):
    tm, tn = ctypes.c_int64(), ctypes.c_int64()
    rc = lib().tgemm_tile_of(idx, M, N, wg, ctypes.byref(tm), ctypes.byref(tn))
    if rc != TGEMM_OK:
        raise TgemmError(rc, "tgemm_tile_of")
    return tm.value, tn.value


def tgemm_split_tile_of(idx: int, M: int, N: int, splits: int, wg: int):
    tm, tn, sp = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int32()
    rc = lib().tgemm_split_tile_of(idx, M, N, splits, wg, ctypes.byref(tm), ctypes.byref(tn), ctypes.byref(sp))
    if rc != TGEMM_OK:
        raise TgemmError(rc, "tgemm_split_tile_of")
    return tm.value, tn.value, sp.value


def tgemm_num_workgroups(idx: int, M: int, N: int) -> int:
    return int(lib().tgemm_num_workgroups(idx, M, N))


def tgemm_mfma_probe(blocks: int, iters: int, out, stream=None, library=None) -> int:
    """Enqueue the MFMA throughput probe of the tooling build (libtgemm_stamps.so); out is a
    float32 device tensor of at least blocks * PROBE_THREADS elements. Returns the FLOP the
    launch performs."""
    import torch
    if out.dtype != torch.float32 or not out.is_cuda or out.numel() < blocks * PROBE_THREADS:
        raise ValueError("out must be a float32 device tensor of blocks * PROBE_THREADS elements")
    handle = torch.cuda.current_stream(out.device).cuda_stream if stream is None else (
        stream if isinstance(stream, int) else stream.cuda_stream)
    with torch.cuda.device(out.device):
        rc = (library or stamps_lib()).tgemm_mfma_probe(int(blocks), int(iters), out.data_ptr(), handle)
    if rc != TGEMM_OK:
        raise TgemmError(rc, "tgemm_mfma_probe")
    return blocks * (PROBE_THREADS // 64) * iters * PROBE_MFMA_PER_ITER * PROBE_FLOP_PER_MFMA


def tgemm_mfma_probe_ex(mode: str, blocks: int, iters: int, out, operands=None, stream=None, library=None) -> int:
    """The MFMA probe with a choice of operands and MFMA shape (PROBE_MODES); operands is a
    binary16 device tensor of PROBE_THREADS * 64 values for every mode but "synthetic".
    Returns the FLOP the launch performs (the same for every mode)."""
    import torch
    if out.dtype != torch.float32 or not out.is_cuda or out.numel() < blocks * PROBE_THREADS:
        raise ValueError("out must be a float32 device tensor of blocks * PROBE_THREADS elements")
    if operands is not None and (operands.dtype != torch.float16 or not operands.is_cuda or
                                 operands.numel() < PROBE_THREADS * 64 or not operands.is_contiguous()):
        raise ValueError("operands must be a contiguous float16 device tensor of PROBE_THREADS * 64 values")
    handle = torch.cuda.current_stream(out.device).cuda_stream if stream is None else (
        stream if isinstance(stream, int) else stream.cuda_stream)
    with torch.cuda.device(out.device):
        rc = (library or stamps_lib()).tgemm_mfma_probe_ex(PROBE_MODES[mode], int(blocks), int(iters),
                                                           None if operands is None else operands.data_ptr(),
                                                           out.data_ptr(), handle)
    if rc != TGEMM_OK:
        raise TgemmError(rc, "tgemm_mfma_probe_ex")
    return blocks * (PROBE_THREADS // 64) * iters * PROBE_MFMA_PER_ITER * PROBE_FLOP_PER_MFMA


def tgemm_lds_probe(op: str, addrs, active=None, iters: int = 1000, blocks: int = 256, out=None, stream=None):
    """Enqueue the tooling build's LDS access probe: instruction kind ``op`` (a key of
    LDS_OPS), addrs an (ni, 64) array of byte addresses (ni <= 8), active an optional list
    of ni 64-bit lane masks (default: all lanes). Returns the float32 device tensor the
    workgroups write."""
    import numpy as np
    import torch
    a = np.ascontiguousarray(np.asarray(addrs, dtype=np.int32).reshape(-1, 64))
    ni = a.shape[0]
    m = np.asarray(active if active is not None else [(1 << 64) - 1] * ni, dtype=np.uint64)
    if out is None:
        out = torch.empty(blocks, dtype=torch.float32, device="cuda")
    handle = torch.cuda.current_stream(out.device).cuda_stream if stream is None else (
        stream if isinstance(stream, int) else stream.cuda_stream)
    with torch.cuda.device(out.device):
        rc = stamps_lib().tgemm_lds_probe(LDS_OPS[op][0], a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                          m.ctypes.data_as(ctypes.POINTER(ctypes.c_uint64)), ni, int(iters),
                                          int(blocks), out.data_ptr(), handle)
    if rc != TGEMM_OK:
        raise TgemmError(rc, "tgemm_lds_probe")
    return out


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
    if t.numel() == 0:  # an empty operand has no meaningful strides
        return rows, cols, max(1, cols)
    if cols > 1 and t.stride(1) != 1:
        raise ValueError(f"{name} must be row-major (stride(1) == 1)")
    ld = t.stride(0) if rows > 1 else max(1, cols)
    return rows, cols, ld


def _stream_handle(stream, device):
    import torch
    if stream is None:
        return torch.cuda.current_stream(device).cuda_stream
    return stream if isinstance(stream, int) else stream.cuda_stream


def gemm_f16_ex(a, b, c=None, trans_a: bool = False, trans_b: bool = False, relu: bool = True,
                stream=None, cfg: int | None = None, library=None):
    """C = ReLU(op(a) @ op(b)) (relu=True) or op(a) @ op(b), through the library. ``a`` is
    the stored matrix: (M, K) fp16, or (K, M) when trans_a; ``b`` is (K, N), or (N, K) when
    trans_b; both row-major views with any row stride. ``c``: (M, N) fp16 output (allocated
    if None). ``stream``: a torch.cuda.Stream or raw handle, by default the current stream
    of a's device. ``cfg`` forces a table config. ``library`` selects another loaded build
    (``stamps_lib()``); default libtgemm.so."""
    import torch
    ra, ca, lda = _operand(a, "a")
    rb, cb, ldb = _operand(b, "b")
    M, K = (ca, ra) if trans_a else (ra, ca)
    K2, N = (cb, rb) if trans_b else (rb, cb)
    if K2 != K:
        raise ValueError(f"inner dimensions differ: op(a) is {M}x{K}, op(b) is {K2}x{N}")
    if c is None:
        c = torch.empty((M, N), dtype=torch.float16, device=a.device)
    Mc, Nc, ldc = _operand(c, "c")
    if (Mc, Nc) != (M, N):
        raise ValueError(f"c has shape {tuple(c.shape)}, expected {(M, N)}")
    if not (a.device == b.device == c.device):
        raise ValueError("a, b and c must be on the same device")
    handle = _stream_handle(stream, a.device)
    args = (M, N, K, a.data_ptr(), lda, b.data_ptr(), ldb, c.data_ptr(), ldc, relu, handle, library)
    with torch.cuda.device(a.device):
        if not trans_a and not trans_b:
            rc = gemm_f16_raw(*args) if cfg is None else gemm_f16_cfg_raw(cfg, *args)
        else:
            rc = (gemm_f16_ex_raw(trans_a, trans_b, *args) if cfg is None
                  else gemm_f16_ex_cfg_raw(cfg, trans_a, trans_b, *args))
    if rc != TGEMM_OK:
        where = "gemm_f16" if not (trans_a or trans_b) else "gemm_f16_ex"
        raise TgemmError(rc, where if cfg is None else f"{where}_cfg[{cfg}]")
    return c


_workspaces = {}


def workspace_for(nbytes: int, device, stream_handle: int):
    """A zero-filled device workspace of at least nbytes for calls on this stream (grown on
    demand; the library keeps its counter region zero between calls in stream order)."""
    import torch
    key = (torch.device(device).index, int(stream_handle or 0))
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.zeros(max(nbytes, 1 << 20), dtype=torch.uint8, device=device)
        torch.cuda.synchronize(device)  # the fill is complete before any stream uses it
        _workspaces[key] = ws
    return ws


def gemm_f16_ws(a, b, c=None, trans_a: bool = False, trans_b: bool = False, relu: bool = True,
                stream=None, workspace=None, cfg: int | None = None, splits: int | None = None,
                library=None):
    """gemm_f16_ex with split-K for small output grids (gemm_f16_ws / gemm_f16_ws_cfg).
    ``workspace``: a uint8 device tensor (zero-filled before its first use, 256-byte
    aligned); by default one is kept per device and stream. ``cfg`` and ``splits`` force
    the plan (both or neither)."""
    import torch
    ra, ca, lda = _operand(a, "a")
    rb, cb, ldb = _operand(b, "b")
    M, K = (ca, ra) if trans_a else (ra, ca)
    K2, N = (cb, rb) if trans_b else (rb, cb)
    if K2 != K:
        raise ValueError(f"inner dimensions differ: op(a) is {M}x{K}, op(b) is {K2}x{N}")
    if c is None:
        c = torch.empty((M, N), dtype=torch.float16, device=a.device)
    Mc, Nc, ldc = _operand(c, "c")
    if (Mc, Nc) != (M, N):
        raise ValueError(f"c has shape {tuple(c.shape)}, expected {(M, N)}")
    if not (a.device == b.device == c.device):
        raise ValueError("a, b and c must be on the same device")
    if (cfg is None) != (splits is None):
        raise ValueError("give both cfg and splits, or neither")
    handle = _stream_handle(stream, a.device)
    L = library or lib()
    if workspace is None:
        if cfg is None:
            need = tgemm_split_plan(trans_a, trans_b, M, N, K, a.data_ptr(), lda, b.data_ptr(), ldb,
                                    c.data_ptr(), ldc)[2]
        else:
            need = tgemm_workspace_bytes_cfg(cfg, splits, M, N)
        workspace = workspace_for(need, a.device, handle) if need else None
    wptr = workspace.data_ptr() if workspace is not None else None
    wbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    with torch.cuda.device(a.device):
        if cfg is None:
            rc = L.gemm_f16_ws(int(trans_a), int(trans_b), M, N, K, a.data_ptr(), lda, b.data_ptr(), ldb,
                               c.data_ptr(), ldc, int(relu), wptr, wbytes, handle)
        else:
            rc = L.gemm_f16_ws_cfg(cfg, splits, int(trans_a), int(trans_b), M, N, K, a.data_ptr(), lda,
                                   b.data_ptr(), ldb, c.data_ptr(), ldc, int(relu), wptr, wbytes, handle)
    if rc != TGEMM_OK:
        raise TgemmError(rc, "gemm_f16_ws" if cfg is None else f"gemm_f16_ws_cfg[{cfg}, {splits}]")
    return c


def gemm_f16_ws_static_raw(ta, tb, M, N, K, A, lda, B, ldb, C, ldc, relu, stream, library=None) -> int:
    return (library or lib()).gemm_f16_ws_static(int(ta), int(tb), M, N, K, A, lda, B, ldb, C, ldc, int(relu),
                                                 stream)


def gemm_f16_ws_static(a, b, c=None, trans_a: bool = False, trans_b: bool = False, relu: bool = True,
                       stream=None, library=None):
    """gemm_f16_ws without a workspace (gemm_f16_ws_static): the split-K scratch is the
    library's static device array, so the library allocates nothing. Calls on one device
    must not overlap in time. ``c`` is allocated here only if not given."""
    import torch
    ra, ca, lda = _operand(a, "a")
    rb, cb, ldb = _operand(b, "b")
    M, K = (ca, ra) if trans_a else (ra, ca)
    K2, N = (cb, rb) if trans_b else (rb, cb)
    if K2 != K:
        raise ValueError(f"inner dimensions differ: op(a) is {M}x{K}, op(b) is {K2}x{N}")
    if c is None:
        c = torch.empty((M, N), dtype=torch.float16, device=a.device)
    Mc, Nc, ldc = _operand(c, "c")
    if (Mc, Nc) != (M, N):
        raise ValueError(f"c has shape {tuple(c.shape)}, expected {(M, N)}")
    if not (a.device == b.device == c.device):
        raise ValueError("a, b and c must be on the same device")
    with torch.cuda.device(a.device):
        rc = gemm_f16_ws_static_raw(trans_a, trans_b, M, N, K, a.data_ptr(), lda, b.data_ptr(), ldb,
                                    c.data_ptr(), ldc, relu, _stream_handle(stream, a.device), library)
    if rc != TGEMM_OK:
        raise TgemmError(rc, "gemm_f16_ws_static")
    return c


def gemm_f16_grouped(problems, trans_a: bool = False, trans_b: bool = False, relu: bool = True,
                     stream=None, library=None):
    """Independent GEMMs in as few launches as possible: ``problems`` is a list of (a, b) or
    (a, b, c) with a, b stored as in gemm_f16_ex (same trans_a / trans_b for all) and c
    allocated when missing. Returns the list of outputs."""
    import torch
    if not problems:
        return []
    descs = (GemmDesc * len(problems))()
    outs = []
    dev = problems[0][0].device
    for i, pr in enumerate(problems):
        a, b = pr[0], pr[1]
        c = pr[2] if len(pr) > 2 else None
        ra, ca, lda = _operand(a, f"problems[{i}].a")
        rb, cb, ldb = _operand(b, f"problems[{i}].b")
        M, K = (ca, ra) if trans_a else (ra, ca)
        K2, N = (cb, rb) if trans_b else (rb, cb)
        if K2 != K:
            raise ValueError(f"problems[{i}]: op(a) is {M}x{K}, op(b) is {K2}x{N}")
        if c is None:
            c = torch.empty((M, N), dtype=torch.float16, device=a.device)
        Mc, Nc, ldc = _operand(c, f"problems[{i}].c")
        if (Mc, Nc) != (M, N):
            raise ValueError(f"problems[{i}]: c has shape {tuple(c.shape)}, expected {(M, N)}")
        if not (a.device == b.device == c.device == dev):
            raise ValueError("all operands must be on one device")
        descs[i] = GemmDesc(M, N, K, a.data_ptr(), lda, b.data_ptr(), ldb, c.data_ptr(), ldc)
        outs.append(c)
    with torch.cuda.device(dev):
        rc = (library or lib()).gemm_f16_grouped(int(trans_a), int(trans_b), len(problems), descs, int(relu),
                                                 _stream_handle(stream, dev))
    if rc != TGEMM_OK:
        raise TgemmError(rc, "gemm_f16_grouped")
    return outs


def gemm_f16(a, b, c=None, relu: bool = True, stream=None, cfg: int | None = None, library=None):
    """C = ReLU(a @ b) (relu=True) or a @ b, through the library. a: (M, K) fp16,
    b: (K, N) fp16, c: (M, N) fp16 output (allocated if None). Row-major views with
    any row stride are accepted. ``stream`` is a torch.cuda.Stream or raw handle; by
    default the current stream of a's device. ``cfg`` forces a table config.
    ``library`` selects another loaded build (``stamps_lib()``); default libtgemm.so."""
    return gemm_f16_ex(a, b, c, False, False, relu, stream, cfg, library)


def _as_stored(x, name):
    """(stored tensor, transposed?) for a logical 2-D operand view: row-major views are
    used as they are; a column-major view (e.g. ``t.t()`` of a row-major t) is passed as
    its row-major transpose with the trans flag set. Anything else is rejected (no hidden
    copies)."""
    rows, cols = x.shape
    if cols <= 1 or x.stride(1) == 1:
        return x, False
    if rows <= 1 or x.stride(0) == 1:
        return x.t(), True
    raise ValueError(f"{name} must be row-major or column-major (strides {tuple(x.stride())})")


def matmul(a, b, relu: bool = False, out=None, stream=None):
    """op(a) @ op(b) (+ ReLU) for logical (M, K) and (K, N) fp16 views, each row- or
    column-major: transposed views such as ``w.t()`` go to the library as transposed
    operands, with no copy. Runs through gemm_f16_ws, so small output grids with a long K
    (weight gradients) are split over the GPU with a workspace kept per device and stream."""
    sa, ta = _as_stored(a, "a")
    sb, tb = _as_stored(b, "b")
    return gemm_f16_ws(sa, sb, out, ta, tb, relu, stream)


def _dense_2d(x):
    """x itself if it is a row- or column-major view the library can take (strides at
    least the row or column length), else a contiguous copy: an upstream gradient may be
    a broadcast view with stride 0 (e.g. from C.sum(0))."""
    rows, cols = x.shape
    row_major = (cols <= 1 or x.stride(1) == 1) and (rows <= 1 or x.stride(0) >= cols)
    col_major = (rows <= 1 or x.stride(0) == 1) and (cols <= 1 or x.stride(1) >= rows)
    return x if (row_major or col_major) else x.contiguous()


def _autograd_function():
    import torch

    class GemmFunction(torch.autograd.Function):
        """C = A @ B with the backward of the pages' autograd wrapper: dA = dC @ B^T and
        dB = A^T @ dC, both as transposed-operand GEMMs in the library (no ReLU: the
        wrapper's forward is the plain GEMM)."""

        @staticmethod
        def forward(ctx, A, B):
            ctx.save_for_backward(A, B)
            return matmul(A, B, relu=False)

        @staticmethod
        def backward(ctx, dC):
            A, B = ctx.saved_tensors
            dC = _dense_2d(dC)
            dA = matmul(dC, B.t()) if ctx.needs_input_grad[0] else None
            dB = matmul(A.t(), dC) if ctx.needs_input_grad[1] else None
            return dA, dB

    return GemmFunction


def __getattr__(name):
    if name == "GemmFunction":
        fn = _autograd_function()
        globals()["GemmFunction"] = fn
        return fn
    raise AttributeError(name)


def configs() -> list:
    return [tgemm_config_desc(i) for i in range(tgemm_num_configs())]


# ---------------------------------------------------------------- fp8 block-scaled path
def gemm_fp8_block_raw(M, N, K, A, lda, SA, B, ldb, SB, C, ldc, relu, stream, library=None) -> int:
    return (library or lib()).gemm_fp8_block(M, N, K, A, lda, SA, B, ldb, SB, C, ldc, int(relu), stream)


def gemm_fp8_block_cfg_raw(idx, M, N, K, A, lda, SA, B, ldb, SB, C, ldc, relu, stream, library=None) -> int:
    return (library or lib()).gemm_fp8_block_cfg(idx, M, N, K, A, lda, SA, B, ldb, SB, C, ldc, int(relu), stream)


def quant_fp8_block_raw(R, K, X, ldx, block_rows, Q, ldq, S, stream, library=None) -> int:
    return (library or lib()).quant_fp8_block(R, K, X, ldx, int(block_rows), Q, ldq, S, stream)


def tgemm_fp8_num_configs() -> int:
    return int(lib().tgemm_fp8_num_configs())


def tgemm_fp8_config_desc(idx: int) -> dict:
    info = ConfigInfo()
    rc = lib().tgemm_fp8_config_desc(idx, ctypes.byref(info))
    if rc != TGEMM_OK:
        raise TgemmError(rc, f"tgemm_fp8_config_desc({idx})")
    return info.as_dict()


def fp8_configs() -> list:
    return [tgemm_fp8_config_desc(i) for i in range(tgemm_fp8_num_configs())]


def tgemm_fp8_select_config(M, N, K, A=256, lda=None, B=256, ldb=None, C=256, ldc=None) -> int:
    """Config index gemm_fp8_block would use (FP8_GENERIC for the generic kernel)."""
    lda = max(1, K) if lda is None else lda
    ldb = max(1, K) if ldb is None else ldb
    ldc = max(1, N) if ldc is None else ldc
    return int(lib().tgemm_fp8_select_config(M, N, K, A, lda, B, ldb, C, ldc))


def _operand8(t, name):
    """A 2-D row-major device tensor of E4M3 codes (uint8 or torch.float8_e4m3fn)."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype not in (torch.uint8, getattr(torch, "float8_e4m3fn", torch.uint8)):
        raise TypeError(f"{name} must hold E4M3 codes (uint8 or float8_e4m3fn), got {t.dtype}")
    if t.dim() != 2:
        raise ValueError(f"{name} must be 2-D")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    rows, cols = t.shape
    if t.numel() == 0:
        return rows, cols, max(1, cols)
    if cols > 1 and t.stride(1) != 1:
        raise ValueError(f"{name} must be row-major (stride(1) == 1)")
    return rows, cols, (t.stride(0) if rows > 1 else max(1, cols))


def _scale_operand(t, shape, name):
    import torch
    if not isinstance(t, torch.Tensor) or t.dtype != torch.float32 or not t.is_cuda:
        raise TypeError(f"{name} must be a float32 device tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.numel() and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def gemm_fp8_block(a, scale_a, b, scale_b, c=None, relu: bool = False, stream=None, cfg: int | None = None,
                   library=None):
    """C = ReLU?(sum_kb scale_a[i,kb] scale_b[j/128,kb] sum_k a[i,k] b[j,k]) through the
    library. a: (M, K) E4M3 codes, b: (N, K) codes (a linear layer's weight), scale_a:
    (M, ceil(K/128)) float32, scale_b: (ceil(N/128), ceil(K/128)) float32; c: (M, N) fp16
    (allocated if None). ``cfg`` forces an fp8 config (or FP8_GENERIC)."""
    import torch
    M, K, lda = _operand8(a, "a")
    N, K2, ldb = _operand8(b, "b")
    if K2 != K:
        raise ValueError(f"inner dimensions differ: a is {M}x{K}, b (N x K) is {N}x{K2}")
    KB = -(-K // FP8_BLOCK)
    _scale_operand(scale_a, (M, KB), "scale_a")
    _scale_operand(scale_b, (-(-N // FP8_BLOCK), KB), "scale_b")
    if c is None:
        c = torch.empty((M, N), dtype=torch.float16, device=a.device)
    Mc, Nc, ldc = _operand(c, "c")
    if (Mc, Nc) != (M, N):
        raise ValueError(f"c has shape {tuple(c.shape)}, expected {(M, N)}")
    if not (a.device == b.device == c.device == scale_a.device == scale_b.device):
        raise ValueError("all operands must be on the same device")
    handle = _stream_handle(stream, a.device)
    args = (M, N, K, a.data_ptr(), lda, scale_a.data_ptr(), b.data_ptr(), ldb, scale_b.data_ptr(), c.data_ptr(),
            ldc, relu, handle, library)
    with torch.cuda.device(a.device):
        rc = gemm_fp8_block_raw(*args) if cfg is None else gemm_fp8_block_cfg_raw(cfg, *args)
    if rc != TGEMM_OK:
        raise TgemmError(rc, "gemm_fp8_block" if cfg is None else f"gemm_fp8_block_cfg[{cfg}]")
    return c


def quant_fp8_block(x, block_rows: int = 1, q=None, scale=None, stream=None, library=None):
    """E4M3 codes and float32 block scales of fp16 x (R, K): blocks of block_rows x 128
    (1: activations, 128: weights). Returns (q (R, K) uint8, scale (ceil(R/block_rows),
    ceil(K/128)) float32)."""
    import torch
    R, K, ldx = _operand(x, "x")
    KB = -(-K // FP8_BLOCK)
    if q is None:
        q = torch.empty((R, K), dtype=torch.uint8, device=x.device)
    if scale is None:
        scale = torch.empty((-(-R // max(1, block_rows)), KB), dtype=torch.float32, device=x.device)
    Rq, Kq, ldq = _operand8(q, "q")
    if (Rq, Kq) != (R, K):
        raise ValueError(f"q has shape {tuple(q.shape)}, expected {(R, K)}")
    _scale_operand(scale, (-(-R // max(1, block_rows)), KB), "scale")
    handle = _stream_handle(stream, x.device)
    with torch.cuda.device(x.device):
        rc = quant_fp8_block_raw(R, K, x.data_ptr(), ldx, block_rows, q.data_ptr(), ldq, scale.data_ptr(), handle,
                                 library)
    if rc != TGEMM_OK:
        raise TgemmError(rc, "quant_fp8_block")
    return q, scale


def fp8_block_scaled_linear(x, w_fp8, scale_w, block: int = 128, relu: bool = False, out=None, stream=None):
    """y = x W^T with W = w_fp8 (N x K E4M3 codes) scaled per 128 x 128 block by scale_w:
    x (M x K fp16) is quantized per 1 x 128 block (quant_fp8_block), then multiplied with
    gemm_fp8_block. Both steps run in the library on the same stream."""
    if block != FP8_BLOCK:
        raise ValueError(f"only block = {FP8_BLOCK} is supported")
    xq, sx = quant_fp8_block(x, 1, stream=stream)
    return gemm_fp8_block(xq, sx, w_fp8, scale_w, c=out, relu=relu, stream=stream)
