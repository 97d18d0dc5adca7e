"""Python binding of libspectra (ctypes).  Argument marshalling only: every
step of packing and of the product runs in the library's gfx950 kernels.

Names mirror the C ABI in include/spectra.h.  PyTorch supplies device memory
and streams; tensors cross the boundary as raw pointers.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libspectra.so")

SPECTRA_OK = 0
SPECTRA_E_INVAL = -1
SPECTRA_E_NONFINITE = -2
SPECTRA_E_NOMEM = -3
SPECTRA_E_HIP = -4
SPECTRA_E_UNSUPPORTED = -5
SPECTRA_E_IO = -6
SPECTRA_E_TIMEOUT = -7

KERNELS = {"auto": 0, "gemv": 1, "mfma": 2, "mfma_tiled": 3, "mfma_strip": 4, "mfma_splitk": 5}

EXPORTED = ["spectra_pack", "spectra_pack_device", "spectra_gemm", "spectra_gemm_ex", "spectra_gemm_noalloc",
            "spectra_gemm_plan",
            "spectra_gemm_grouped", "spectra_embed", "spectra_free", "spectra_info",
            "spectra_export", "spectra_validate_image", "spectra_import", "spectra_save",
            "spectra_load", "spectra_kv_create", "spectra_kv_append", "spectra_kv_attend",
            "spectra_kv_length", "spectra_kv_reset", "spectra_kv_export", "spectra_kv_free",
            "spectra_step_create", "spectra_step_run", "spectra_step_status", "spectra_step_test_hooks",
            "spectra_step_free", "spectra_release_workspaces", "spectra_test_fail_allocations", "spectra_last_error", "spectra_last_status",
            "spectra_version"]


class SpectraError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"spectra status {status}: {msg}")
        self.status = status


STEP_MAX_TASKS = 4


class spectra_step_phase(ctypes.Structure):
    _fields_ = [("ntasks", ctypes.c_int32), ("c", ctypes.c_void_p * STEP_MAX_TASKS),
                ("y", ctypes.c_void_p * STEP_MAX_TASKS), ("input", ctypes.c_int32),
                ("x", ctypes.c_void_p), ("x_scale", ctypes.c_float)]


class spectra_info_t(ctypes.Structure):
    _fields_ = [("K", ctypes.c_int64), ("N", ctypes.c_int64), ("K_b", ctypes.c_int64),
                ("G", ctypes.c_int64), ("n_out", ctypes.c_int64),
                ("bytes_codes", ctypes.c_uint64), ("bytes_scales", ctypes.c_uint64),
                ("bytes_zeros", ctypes.c_uint64), ("bytes_outliers", ctypes.c_uint64),
                ("bytes_payload", ctypes.c_uint64), ("bytes_meta", ctypes.c_uint64),
                ("bytes_total", ctypes.c_uint64)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load the in-tree libspectra.so; fail loudly when it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m dequant_gemv_spectra_amd.build` (needs ROCm hipcc)")
    L = ctypes.CDLL(LIB_PATH)
    vp, i64, u64, c_int = ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint64, ctypes.c_int
    L.spectra_pack.argtypes = [vp, vp, i64, i64]
    L.spectra_pack.restype = vp
    L.spectra_pack_device.argtypes = [vp, vp, i64, i64, vp]
    L.spectra_pack_device.restype = vp
    L.spectra_gemm.argtypes = [vp, vp, vp, i64]
    L.spectra_gemm.restype = c_int
    L.spectra_gemm_ex.argtypes = [vp, vp, vp, i64, vp, c_int]
    L.spectra_gemm_ex.restype = c_int
    L.spectra_gemm_noalloc.argtypes = [vp, vp, vp, i64, vp, c_int]
    L.spectra_gemm_noalloc.restype = c_int
    L.spectra_gemm_plan.argtypes = [vp, i64, c_int]
    L.spectra_gemm_plan.restype = c_int
    L.spectra_gemm_grouped.argtypes = [ctypes.POINTER(vp), c_int, vp, ctypes.POINTER(vp), i64, vp]
    L.spectra_gemm_grouped.restype = c_int
    L.spectra_embed.argtypes = [vp, vp, i64, vp, vp]
    L.spectra_embed.restype = c_int
    L.spectra_validate_image.argtypes = [vp, u64]
    L.spectra_validate_image.restype = c_int
    L.spectra_import.argtypes = [vp, u64]
    L.spectra_import.restype = vp
    L.spectra_save.argtypes = [vp, ctypes.c_char_p, u64]
    L.spectra_save.restype = c_int
    L.spectra_load.argtypes = [ctypes.c_char_p, u64]
    L.spectra_load.restype = vp
    L.spectra_kv_create.argtypes = [i64, ctypes.c_int32, ctypes.c_int32]
    L.spectra_kv_create.restype = vp
    L.spectra_kv_append.argtypes = [vp, vp, vp, i64, vp]
    L.spectra_kv_append.restype = c_int
    L.spectra_kv_attend.argtypes = [vp, vp, ctypes.c_int32, vp, vp]
    L.spectra_kv_attend.restype = c_int
    L.spectra_kv_length.argtypes = [vp]
    L.spectra_kv_length.restype = i64
    L.spectra_kv_reset.argtypes = [vp]
    L.spectra_kv_reset.restype = c_int
    L.spectra_kv_export.argtypes = [vp, vp, u64]
    L.spectra_kv_export.restype = c_int
    L.spectra_kv_free.argtypes = [vp]
    L.spectra_kv_free.restype = None
    L.spectra_free.argtypes = [vp]
    L.spectra_free.restype = None
    L.spectra_info.argtypes = [vp, ctypes.POINTER(spectra_info_t)]
    L.spectra_info.restype = c_int
    L.spectra_export.argtypes = [vp, vp, u64]
    L.spectra_export.restype = c_int
    L.spectra_step_create.argtypes = [ctypes.POINTER(spectra_step_phase), ctypes.c_int32]
    L.spectra_step_create.restype = vp
    L.spectra_step_run.argtypes = [vp, vp]
    L.spectra_step_run.restype = c_int
    L.spectra_step_status.argtypes = [vp, vp]
    L.spectra_step_status.restype = c_int
    L.spectra_step_test_hooks.argtypes = [vp, ctypes.c_uint32, ctypes.c_uint32]
    L.spectra_step_test_hooks.restype = c_int
    L.spectra_step_free.argtypes = [vp]
    L.spectra_step_free.restype = None
    L.spectra_last_error.argtypes = []
    L.spectra_last_error.restype = ctypes.c_char_p
    L.spectra_release_workspaces.argtypes = []
    L.spectra_release_workspaces.restype = c_int
    L.spectra_test_fail_allocations.argtypes = [ctypes.c_int64, ctypes.c_int64]
    L.spectra_test_fail_allocations.restype = c_int
    L.spectra_last_status.argtypes = []
    L.spectra_last_status.restype = c_int
    L.spectra_version.argtypes = []
    L.spectra_version.restype = c_int
    _lib = L
    return L


def spectra_last_error() -> str:
    return lib().spectra_last_error().decode()


def spectra_last_status() -> int:
    return lib().spectra_last_status()


def _null_handle_error() -> "SpectraError":
    """The error behind a NULL handle, classified by the library's status code."""
    st = spectra_last_status()
    return SpectraError(st if st < 0 else SPECTRA_E_INVAL, spectra_last_error())


def _check(status: int):
    if status != SPECTRA_OK:
        raise SpectraError(status, spectra_last_error())


class Container:
    """Owning handle of a packed container (freed on close / garbage collection)."""

    def __init__(self, ptr: int):
        self.ptr = ptr
        self._info = None

    @property
    def handle(self):
        if not self.ptr:
            raise SpectraError(SPECTRA_E_INVAL, "container already freed")
        return ctypes.c_void_p(self.ptr)

    def info(self) -> dict:
        if self._info is None:
            self._info = spectra_info(self)
        return self._info

    def close(self):
        if self.ptr:
            lib().spectra_free(ctypes.c_void_p(self.ptr))
            self.ptr = 0

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()


def _stream_ptr(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def spectra_pack(W, gamma, stream=None) -> Container:
    """Pack fp16 W [N][K] with gain fp16 gamma [K].

    numpy arrays and CPU tensors go through the host entry point; CUDA tensors
    through the device entry point (on `stream`, default the current stream).
    """
    if isinstance(W, np.ndarray) or (hasattr(W, "is_cuda") and not W.is_cuda):
        Wn = np.ascontiguousarray(np.asarray(W), dtype=np.float16)
        gn = np.ascontiguousarray(np.asarray(gamma), dtype=np.float16)
        if Wn.ndim != 2 or gn.shape != (Wn.shape[1],):
            raise ValueError("W must be [N][K] and gamma [K]")
        N, K = Wn.shape
        p = lib().spectra_pack(Wn.ctypes.data_as(ctypes.c_void_p), gn.ctypes.data_as(ctypes.c_void_p),
                               K, N)
    else:
        import torch
        if W.dtype != torch.float16 or gamma.dtype != torch.float16:
            raise ValueError("W and gamma must be float16")
        W = W.contiguous()
        gamma = gamma.contiguous()
        N, K = W.shape
        if gamma.shape != (K,) or not gamma.is_cuda:
            raise ValueError("gamma must be a CUDA tensor of shape [K]")
        p = lib().spectra_pack_device(ctypes.c_void_p(W.data_ptr()), ctypes.c_void_p(gamma.data_ptr()),
                                      K, N, _stream_ptr(stream))
    if not p:
        raise _null_handle_error()
    return Container(p)


def spectra_gemm(c: Container, x, y=None, stream=None, kernel: str = "auto"):
    """y = x W_hat^T for CUDA fp16 x [M][K]; returns y (fp16 [M][N], allocated if None)."""
    import torch
    info = c.info()
    if x.dtype != torch.float16 or not x.is_cuda or x.dim() != 2 or x.shape[1] != info["K"]:
        raise ValueError("x must be a CUDA float16 tensor of shape [M][K]")
    x = x.contiguous()
    M = x.shape[0]
    if y is None:
        y = torch.empty((M, info["N"]), dtype=torch.float16, device=x.device)
    elif y.dtype != torch.float16 or not y.is_contiguous() or tuple(y.shape) != (M, info["N"]):
        raise ValueError("y must be a contiguous float16 tensor of shape [M][N]")
    _check(lib().spectra_gemm_ex(c.handle, ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(y.data_ptr()),
                                 M, _stream_ptr(stream), KERNELS[kernel]))
    return y


def spectra_gemm_noalloc(c: Container, x, y, stream=None, kernel: str = "auto"):
    """As spectra_gemm into a given y, through the entry point that allocates
    no device memory (the MFMA path uses the library's static scratch)."""
    import torch
    info = c.info()
    if x.dtype != torch.float16 or not x.is_cuda or x.dim() != 2 or x.shape[1] != info["K"]:
        raise ValueError("x must be a CUDA float16 tensor of shape [M][K]")
    M = x.shape[0]
    if y.dtype != torch.float16 or not y.is_contiguous() or tuple(y.shape) != (M, info["N"]):
        raise ValueError("y must be a contiguous float16 tensor of shape [M][N]")
    _check(lib().spectra_gemm_noalloc(c.handle, ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(y.data_ptr()),
                                      M, _stream_ptr(stream), KERNELS[kernel]))
    return y


PLANS = {1: "k_gemv_m1", 2: "k_mfma_ks", 3: "k_mfma", 4: "k_mfma_sk"}


def spectra_gemm_plan(c: Container, M: int, kernel: str = "auto") -> str:
    """Name of the kernel spectra_gemm would run for M rows of x (no device work)."""
    st = lib().spectra_gemm_plan(c.handle, M, KERNELS[kernel])
    if st < 0:
        _check(st)
    return PLANS[st]


def spectra_gemm_grouped(cs, x, ys=None, stream=None):
    """ys[i] = x W_i^T for containers sharing K, one launch; x is CUDA fp16 [1][K]."""
    import torch
    n = len(cs)
    if ys is None:
        ys = [torch.empty((x.shape[0], c.info()["N"]), dtype=torch.float16, device=x.device) for c in cs]
    arr_c = (ctypes.c_void_p * n)(*[c.handle.value for c in cs])
    arr_y = (ctypes.c_void_p * n)(*[y.data_ptr() for y in ys])
    x = x.contiguous()
    _check(lib().spectra_gemm_grouped(arr_c, n, ctypes.c_void_p(x.data_ptr()), arr_y, x.shape[0],
                                      _stream_ptr(stream)))
    return ys


def spectra_embed(c: Container, ids, out=None, stream=None):
    """Rows of the packed table for CUDA int32 ids [T]: fp16 [T][K] (allocated if None)."""
    import torch
    info = c.info()
    if ids.dtype != torch.int32 or not ids.is_cuda or ids.dim() != 1:
        raise ValueError("ids must be a 1-D CUDA int32 tensor")
    ids = ids.contiguous()
    T = ids.shape[0]
    if out is None:
        out = torch.empty((T, info["K"]), dtype=torch.float16, device=ids.device)
    elif out.dtype != torch.float16 or not out.is_contiguous() or tuple(out.shape) != (T, info["K"]):
        raise ValueError("out must be a contiguous float16 tensor of shape [T][K]")
    _check(lib().spectra_embed(c.handle, ctypes.c_void_p(ids.data_ptr()), T,
                               ctypes.c_void_p(out.data_ptr()), _stream_ptr(stream)))
    return out


def spectra_validate_image(image: bytes) -> None:
    """Raise SpectraError unless `image` is a well-formed container image."""
    buf = (ctypes.c_ubyte * len(image)).from_buffer_copy(image) if image else None
    _check(lib().spectra_validate_image(buf, len(image)))


def spectra_import(image: bytes) -> Container:
    """A new container on the current device from a host image."""
    buf = (ctypes.c_ubyte * len(image)).from_buffer_copy(image) if image else None
    p = lib().spectra_import(buf, len(image))
    if not p:
        raise _null_handle_error()
    return Container(p)


def spectra_save(c: Container, path: str, chunk_bytes: int = 0) -> None:
    _check(lib().spectra_save(c.handle, os.fsencode(path), chunk_bytes))


def spectra_load(path: str, chunk_bytes: int = 0) -> Container:
    """Stream a container file into a new container on the current device."""
    p = lib().spectra_load(os.fsencode(path), chunk_bytes)
    if not p:
        raise _null_handle_error()
    return Container(p)


class KvCache:
    """Owning handle of a Group-32 4-bit KV cache (one attention layer)."""

    def __init__(self, capacity: int, heads: int, head_dim: int):
        p = lib().spectra_kv_create(capacity, heads, head_dim)
        if not p:
            raise _null_handle_error()
        self.handle = ctypes.c_void_p(p)
        self.heads, self.head_dim = heads, head_dim

    def append(self, k, v, stream=None) -> None:
        """k, v: CUDA fp16 [T][heads][head_dim]."""
        import torch
        for t in (k, v):
            if t.dtype != torch.float16 or not t.is_cuda or t.dim() != 3 or tuple(t.shape[1:]) != (self.heads, self.head_dim):
                raise ValueError("k and v must be CUDA float16 tensors of shape [T][heads][head_dim]")
        k, v = k.contiguous(), v.contiguous()
        _check(lib().spectra_kv_append(self.handle, ctypes.c_void_p(k.data_ptr()), ctypes.c_void_p(v.data_ptr()),
                                       k.shape[0], _stream_ptr(stream)))

    def attend(self, q, out=None, stream=None):
        """q: CUDA fp16 [q_heads][head_dim] -> out fp16 [q_heads][head_dim]."""
        import torch
        if q.dtype != torch.float16 or not q.is_cuda or q.dim() != 2 or q.shape[1] != self.head_dim:
            raise ValueError("q must be a CUDA float16 tensor of shape [q_heads][head_dim]")
        q = q.contiguous()
        if out is None:
            out = torch.empty_like(q)
        _check(lib().spectra_kv_attend(self.handle, ctypes.c_void_p(q.data_ptr()), q.shape[0],
                                       ctypes.c_void_p(out.data_ptr()), _stream_ptr(stream)))
        return out

    @property
    def length(self) -> int:
        return int(lib().spectra_kv_length(self.handle))

    def reset(self) -> None:
        _check(lib().spectra_kv_reset(self.handle))

    def export(self) -> bytes:
        n = self.length * self.heads * (self.head_dim // 32)
        total = 2 * (16 * n + 2 * n + n // 2)
        buf = (ctypes.c_ubyte * max(1, total))()
        _check(lib().spectra_kv_export(self.handle, buf, total))
        return bytes(buf)[:total]

    def close(self) -> None:
        if self.handle:
            lib().spectra_kv_free(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class StepPlan:
    """Owning handle of a decode step: a chain of dependent M = 1 products run
    by one persistent launch (spectra_step_create).

    phases: sequence of dicts with keys
      "containers": 1 .. 4 Containers sharing K,
      "ys": matching CUDA fp16 output tensors [N_i] (or [1][N_i]),
      "input": -1 for an external x, else the index of an earlier phase whose
               first container's output is the input,
      "x": CUDA fp16 [K] tensor when input == -1,
      "x_scale": power of two applied to the staged input (default 1.0).
    The plan borrows the containers and tensors; keep them alive while it is used.
    """

    def __init__(self, phases):
        n = len(phases)
        arr = (spectra_step_phase * n)()
        self._keep = []
        for i, ph in enumerate(phases):
            cs, ys = list(ph["containers"]), list(ph["ys"])
            if not 1 <= len(cs) <= STEP_MAX_TASKS or len(ys) != len(cs):
                raise ValueError("each phase needs 1 .. 4 containers and as many outputs")
            arr[i].ntasks = len(cs)
            for j, (c, y) in enumerate(zip(cs, ys)):
                arr[i].c[j] = c.handle.value
                arr[i].y[j] = y.data_ptr()
            arr[i].input = int(ph.get("input", -1))
            x = ph.get("x")
            arr[i].x = x.data_ptr() if x is not None else None
            arr[i].x_scale = float(ph.get("x_scale", 1.0))
            self._keep.append((cs, ys, x))
        p = lib().spectra_step_create(arr, n)
        if not p:
            raise _null_handle_error()
        self.handle = ctypes.c_void_p(p)

    def run(self, stream=None) -> None:
        _check(lib().spectra_step_run(self.handle, _stream_ptr(stream)))

    def status(self, stream=None) -> int:
        """SPECTRA_OK, or SPECTRA_E_TIMEOUT when a wait of an earlier run gave up."""
        st = lib().spectra_step_status(self.handle, _stream_ptr(stream))
        if st not in (SPECTRA_OK, SPECTRA_E_TIMEOUT):
            _check(st)
        return st

    def test_hooks(self, poll_limit: int = 0, tag_skew: int = 0) -> None:
        _check(lib().spectra_step_test_hooks(self.handle, poll_limit, tag_skew))

    def close(self) -> None:
        if self.handle:
            lib().spectra_step_free(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def spectra_free(c: Container):
    c.close()


def spectra_info(c: Container) -> dict:
    out = spectra_info_t()
    _check(lib().spectra_info(c.handle, ctypes.byref(out)))
    return {name: getattr(out, name) for name, _ in spectra_info_t._fields_}


def spectra_export(c: Container) -> bytes:
    total = c.info()["bytes_total"]
    buf = (ctypes.c_ubyte * total)()
    _check(lib().spectra_export(c.handle, buf, total))
    return bytes(buf)


def spectra_release_workspaces() -> None:
    """Free the workspaces earlier growth retired (no graph captured before a
    growth may be replayed afterwards)."""
    _check(lib().spectra_release_workspaces())


def spectra_test_fail_allocations(skip: int, count: int) -> None:
    """Testing hook: of the library's next device / pinned-host allocations,
    `skip` succeed and `count` fail as out of memory; (0, 0) turns it off."""
    _check(lib().spectra_test_fail_allocations(skip, count))


def spectra_version() -> int:
    return lib().spectra_version()
