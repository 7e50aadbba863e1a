"""dense_tiled_gemm_fp16_amd: C = A.B for fp16 matrices on MI355X (gfx950).

The computation runs in libgemmf16.so (hand-written HIP, C-ABI in
include/gemm_f16.h).  This package only marshals arguments: torch supplies
device memory and the current stream.

    gemm(a, b, out=None, ...)      -> C ([M, N], float16 or bfloat16 like a and b;
                                      float16 for float8_e4m3fn / float8_e5m2 inputs)
    gemm_grouped(a, b, offsets)    -> C, group g: C[off[g]:off[g+1]] = A[...] @ b[g]
    pack_b(b) / gemm_packed(a, p)  -> a static fp16 B packed once, then C = a @ B
    plan(a, b, out=None, ...)      -> dict describing the kernel that would run
    workspace_bytes(M, N, K, ...)  -> bytes of split-K workspace needed
    gemm_noalloc(a, b, out)        -> C = a @ b (float16) with no device allocation by the
                                      library (its workspace in a fixed per-GPU array)
"""
import ctypes

import torch

from ._lib import (GEMM_OK, LIB_PATH, PATHS, STATUS, VARIANTS, Opts, PlanInfo, lib, make_opts,
                   status_string)

__all__ = ["gemm", "gemm_raw", "gemm_noalloc", "gemm_grouped", "pack_b", "gemm_packed", "PackedB", "plan",
           "workspace_bytes", "GemmError", "LIB_PATH",
           "VARIANTS"]


class GemmError(RuntimeError):
    def __init__(self, rc):
        super().__init__(f"{STATUS.get(rc, rc)}: {status_string(rc)}")
        self.status = rc


def _check(a, b, out):
    # Argument checks in the spirit of the Triton article's wrapper (section
    # "addresses and bounds in one short kernel"); the library re-validates.
    if a.ndim != 2 or b.ndim != 2:
        raise ValueError("expected two matrices")
    if not a.is_cuda or not b.is_cuda or a.device != b.device:
        raise ValueError("inputs must share one GPU device")
    if a.dtype in F8_FORMATS or b.dtype in F8_FORMATS:
        if a.dtype not in F8_FORMATS or b.dtype not in F8_FORMATS:
            raise TypeError("FP8 inputs must both be float8_e4m3fn or float8_e5m2")
        out_dtype = torch.float16
    elif a.dtype not in (torch.float16, torch.bfloat16) or b.dtype != a.dtype:
        raise TypeError("inputs must both be float16, both bfloat16, or both FP8")
    else:
        out_dtype = a.dtype
    m, k = a.shape
    kb, n = b.shape
    if k != kb or min(m, n, k) <= 0:
        raise ValueError("incompatible or empty shape")
    if min(a.stride() + b.stride()) <= 0:
        raise ValueError("strides must be positive")
    if out is None:
        out = torch.empty((m, n), device=a.device, dtype=out_dtype)
    else:
        if out.dtype != out_dtype or out.device != a.device or out.shape != (m, n):
            raise ValueError("out must be an [M, N] tensor of the output dtype on the inputs' device")
        if out.stride(1) != 1 or out.stride(0) < n:
            raise ValueError("out must be row-major with unit column stride")
    return m, n, k, out


def gemm_raw(A, lda_m, lda_k, B, ldb_k, ldb_n, C, ldc, M, N, K, stream=0, workspace=0,
             workspace_bytes=0, opts=None):
    """Direct call of gemm_f16_ex with integer device addresses; returns the status."""
    o = opts if opts is not None else None
    return lib.gemm_f16_ex(A, lda_m, lda_k, B, ldb_k, ldb_n, C, ldc, M, N, K, stream,
                           workspace, workspace_bytes, ctypes.byref(o) if o is not None else None)


# OCP FP8 formats of the inputs -> format codes of gemm_f8* (0 E4M3, 1 E5M2).
F8_FORMATS = {torch.float8_e4m3fn: 0, torch.float8_e5m2: 1}


def _fn(a, name, b=None):
    """The entry point for the inputs' format.  For FP8 inputs the returned
    callable appends the two format codes after K (the gemm_f8* layout)."""
    if a.dtype in F8_FORMATS:
        f = getattr(lib, name.replace("gemm_f16", "gemm_f8"))
        fa, fb = F8_FORMATS[a.dtype], F8_FORMATS[(b if b is not None else a).dtype]

        def call(*args):
            return f(*args[:11], fa, fb, *args[11:])
        return call
    return getattr(lib, name if a.dtype == torch.float16 else name.replace("gemm_f16", "gemm_bf16"))


def gemm(a, b, out=None, workspace=None, variant="auto", split_k=0, panel=0, tile=0,
         stream=None):
    """C = a @ b with fp32 accumulation, output in the inputs' format (float16
    or bfloat16), computed by libgemmf16."""
    m, n, k, out = _check(a, b, out)
    opts = make_opts(variant, split_k, panel, tile)
    if stream is None:
        stream = torch.cuda.current_stream(a.device)
    ws_ptr, ws_bytes = 0, 0
    if workspace is not None:
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    with torch.cuda.device(a.device):
        rc = _fn(a, "gemm_f16_ex", b)(a.data_ptr(), a.stride(0), a.stride(1), b.data_ptr(),
                                   b.stride(0), b.stride(1), out.data_ptr(), out.stride(0), m, n,
                                   k, stream.cuda_stream, ws_ptr, ws_bytes, ctypes.byref(opts))
    if rc != GEMM_OK:
        raise GemmError(rc)
    return out


def gemm_noalloc(a, b, out, stream=None):
    """C = a @ b for float16 a and b into the caller's float16 `out`, through
    gemm_f16_noalloc: the library allocates nothing (see that entry point for
    the size limit and for calls that overlap on one GPU)."""
    if a.dtype != torch.float16 or b.dtype != torch.float16 or out is None:
        raise TypeError("gemm_noalloc takes float16 a, b and a float16 out")
    m, n, k, out = _check(a, b, out)
    if stream is None:
        stream = torch.cuda.current_stream(a.device)
    with torch.cuda.device(a.device):
        rc = lib.gemm_f16_noalloc(a.data_ptr(), a.stride(0), a.stride(1), b.data_ptr(), b.stride(0),
                                  b.stride(1), out.data_ptr(), out.stride(0), m, n, k,
                                  stream.cuda_stream)
    if rc != GEMM_OK:
        raise GemmError(rc)
    return out


def gemm_grouped(a, b, offsets, out=None, workspace=None, stream=None):
    """Grouped product: for each g, C[offsets[g]:offsets[g+1]] = a[same rows] @ b[g].

    a [M_total, K] and b [G, K, N] on one GPU, both float16 or both bfloat16
    (out in the same format) or both FP8 (float8_e4m3fn / float8_e5m2, out
    float16), offsets a device int64 tensor of G + 1 row offsets (read by
    the kernels, never by the host).  Rows of out outside every group are
    left as they were."""
    if a.ndim != 2 or b.ndim != 3:
        raise ValueError("expected a [M, K] matrix and a [G, K, N] stack")
    if not (a.is_cuda and b.is_cuda and offsets.is_cuda) or len({a.device, b.device, offsets.device}) != 1:
        raise ValueError("inputs must share one GPU device")
    f8 = a.dtype in F8_FORMATS and b.dtype in F8_FORMATS
    if not (f8 or (a.dtype in (torch.float16, torch.bfloat16) and b.dtype == a.dtype)) or \
            offsets.dtype != torch.int64:
        raise TypeError("a and b must be both float16, both bfloat16 or both FP8, offsets int64")
    c_dtype = torch.float16 if f8 else a.dtype
    m, k = a.shape
    g, kb, n = b.shape
    if kb != k or min(m, n, k, g) <= 0 or offsets.shape != (g + 1,) or offsets.stride(0) != 1:
        raise ValueError("incompatible or empty shape, or offsets not a contiguous [G + 1] vector")
    if out is None:
        out = torch.empty((m, n), device=a.device, dtype=c_dtype)
    elif out.dtype != c_dtype or out.device != a.device or out.shape != (m, n) or out.stride(1) != 1:
        raise ValueError("out must be a row-major [M, N] tensor of the output format (float16 for FP8 "
                         "inputs) on the inputs' device")
    if stream is None:
        stream = torch.cuda.current_stream(a.device)
    ws_ptr, ws_bytes = 0, 0
    if workspace is not None:
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    with torch.cuda.device(a.device):
        args = (a.data_ptr(), a.stride(0), a.stride(1), b.data_ptr(), b.stride(0), b.stride(1),
                b.stride(2), out.data_ptr(), out.stride(0), offsets.data_ptr(), g, m, n, k)
        if f8:
            rc = lib.gemm_f8_grouped(*args, F8_FORMATS[a.dtype], F8_FORMATS[b.dtype],
                                     stream.cuda_stream, ws_ptr, ws_bytes)
        else:
            fn = lib.gemm_f16_grouped if a.dtype == torch.float16 else lib.gemm_bf16_grouped
            rc = fn(*args, stream.cuda_stream, ws_ptr, ws_bytes)
    if rc != GEMM_OK:
        raise GemmError(rc)
    return out


def plan(a, b, out=None, variant="auto", split_k=0, panel=0, tile=0):
    """The plan (kernel family, tile, split, raster panel, load paths, grid,
    workspace) that gemm would execute for these tensors."""
    m, n, k, out = _check(a, b, out)
    opts = make_opts(variant, split_k, panel, tile)
    info = PlanInfo()
    with torch.cuda.device(a.device):
        rc = _fn(a, "gemm_f16_plan", b)(a.data_ptr(), a.stride(0), a.stride(1), b.data_ptr(),
                                     b.stride(0), b.stride(1), out.data_ptr(), out.stride(0), m, n,
                                     k, ctypes.byref(opts), ctypes.byref(info))
    if rc != GEMM_OK:
        raise GemmError(rc)
    d = info.as_dict()
    d["a_path"], d["b_path"] = PATHS[d["a_path"]], PATHS[d["b_path"]]
    d["variant"] = {v: k for k, v in VARIANTS.items()}[d["variant"]]
    return d


def workspace_bytes(M, N, K, variant="auto", split_k=0, panel=0, tile=0):
    opts = make_opts(variant, split_k, panel, tile)
    return int(lib.gemm_f16_workspace_bytes(M, N, K, ctypes.byref(opts)))


class PackedB:
    """A float16 B [K, N] packed by gemm_f16_pack_b (opaque bytes on its GPU)."""

    def __init__(self, data, K, N):
        self.data, self.K, self.N = data, K, N


def pack_b(b, stream=None):
    """Pack a static float16 B [K, N] (any positive strides) for gemm_packed."""
    if b.ndim != 2 or not b.is_cuda or b.dtype != torch.float16:
        raise ValueError("expected a float16 [K, N] matrix on a GPU")
    K, N = b.shape
    nbytes = int(lib.gemm_f16_packed_b_bytes(K, N))
    if nbytes == 0:
        raise ValueError("empty or oversized shape")
    data = torch.empty(nbytes, dtype=torch.uint8, device=b.device)
    if stream is None:
        stream = torch.cuda.current_stream(b.device)
    with torch.cuda.device(b.device):
        rc = lib.gemm_f16_pack_b(b.data_ptr(), b.stride(0), b.stride(1), K, N, data.data_ptr(),
                                 stream.cuda_stream)
    if rc != GEMM_OK:
        raise GemmError(rc)
    return PackedB(data, K, N)


def gemm_packed(a, packed, out=None, stream=None):
    """C = a @ B for a float16 a [M, K] (K-contiguous rows) and B packed by pack_b."""
    if a.ndim != 2 or not a.is_cuda or a.dtype != torch.float16:
        raise ValueError("expected a float16 [M, K] matrix on a GPU")
    if packed.data.device != a.device or a.shape[1] != packed.K:
        raise ValueError("a and the packed B must share the GPU and K")
    m, n = a.shape[0], packed.N
    if out is None:
        out = torch.empty((m, n), device=a.device, dtype=torch.float16)
    elif out.dtype != torch.float16 or out.shape != (m, n) or out.stride(1) != 1:
        raise ValueError("out must be a row-major float16 [M, N] tensor")
    if stream is None:
        stream = torch.cuda.current_stream(a.device)
    with torch.cuda.device(a.device):
        rc = lib.gemm_f16_packed(a.data_ptr(), a.stride(0), a.stride(1), packed.data.data_ptr(),
                                 out.data_ptr(), out.stride(0), m, n, packed.K, stream.cuda_stream)
    if rc != GEMM_OK:
        raise GemmError(rc)
    return out
