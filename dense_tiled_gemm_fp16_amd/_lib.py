"""ctypes view of libgemmf16.so (the C-ABI in include/gemm_f16.h).

Argument marshalling only: every step of the computation runs in the HIP
library.  There is no fallback: if the library cannot be loaded, importing
this module raises."""
import ctypes
import os

from . import build as _build

i32, i64, vp, sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t

GEMM_OK = 0
STATUS = {0: "GEMM_OK", -1: "GEMM_ERR_NULL", -2: "GEMM_ERR_SHAPE", -3: "GEMM_ERR_STRIDE",
          -4: "GEMM_ERR_LDC", -5: "GEMM_ERR_ALIAS", -6: "GEMM_ERR_WORKSPACE",
          -7: "GEMM_ERR_OPTS", -8: "GEMM_ERR_HIP", -9: "GEMM_ERR_LAYOUT", -10: "GEMM_ERR_SCRATCH"}
SCRATCH_BYTES = 32 << 20   # GEMM_F16_SCRATCH_BYTES
VARIANT_AUTO, VARIANT_MAIN, VARIANT_SKINNY, VARIANT_SPLITK, VARIANT_TILE64X32, VARIANT_STREAMK = \
    0, 1, 2, 3, 4, 5
VARIANTS = {"auto": 0, "main": 1, "skinny": 2, "splitk": 3, "tile64x32": 4, "streamk": 5}
PATHS = {0: "gather", 1: "kvec", 2: "rvec", 3: "packed"}

EXPORTS = ["gemm_f16", "gemm_f16_ex", "gemm_f16_plan", "gemm_f16_plan_cus", "gemm_f16_workspace_bytes",
           "gemm_bf16", "gemm_bf16_ex", "gemm_bf16_plan", "gemm_bf16_workspace_bytes",
           "gemm_f8", "gemm_f8_ex", "gemm_f8_plan", "gemm_f8_plan_cus", "gemm_f8_workspace_bytes",
           "gemm_f16_packed_b_bytes", "gemm_f16_pack_b", "gemm_f16_packed",
           "gemm_f16_grouped", "gemm_bf16_grouped", "gemm_f8_grouped", "gemm_f16_grouped_workspace_bytes",
           "gemm_f16_noalloc", "gemm_f16_status_string", "gemm_f16_version"]


class Opts(ctypes.Structure):
    _fields_ = [("variant", i32), ("split_k", i32), ("panel", i32), ("tile", i32)]


class PlanInfo(ctypes.Structure):
    _fields_ = [("variant", i32), ("tile_m", i32), ("tile_n", i32), ("tile_k", i32),
                ("split_k", i32), ("panel", i32), ("a_path", i32), ("b_path", i32),
                ("tile_id", i32), ("grid", i64), ("grid2", i64),
                ("workspace_bytes", ctypes.c_uint64), ("sk_tiles", i64)]

    def as_dict(self):
        return {f: getattr(self, f) for f, _ in self._fields_}


def _load():
    if not os.path.exists(_build.LIB):
        _build.build()
    lib = ctypes.CDLL(_build.LIB)
    args12 = [vp, i64, i64, vp, i64, i64, vp, i64, i64, i64, i64, vp]
    lib.gemm_f16.argtypes = args12
    lib.gemm_f16.restype = ctypes.c_int
    lib.gemm_f16_noalloc.argtypes = args12
    lib.gemm_f16_noalloc.restype = ctypes.c_int
    lib.gemm_f16_ex.argtypes = args12 + [vp, sz, ctypes.POINTER(Opts)]
    lib.gemm_f16_ex.restype = ctypes.c_int
    lib.gemm_f16_plan.argtypes = [vp, i64, i64, vp, i64, i64, vp, i64, i64, i64, i64,
                                  ctypes.POINTER(Opts), ctypes.POINTER(PlanInfo)]
    lib.gemm_f16_plan.restype = ctypes.c_int
    lib.gemm_f16_plan_cus.argtypes = [vp, i64, i64, vp, i64, i64, vp, i64, i64, i64, i64, i32,
                                      ctypes.POINTER(Opts), ctypes.POINTER(PlanInfo)]
    lib.gemm_f16_plan_cus.restype = ctypes.c_int
    lib.gemm_f16_workspace_bytes.argtypes = [i64, i64, i64, ctypes.POINTER(Opts)]
    lib.gemm_f16_workspace_bytes.restype = sz
    for pre in ("gemm_bf16",):
        getattr(lib, pre).argtypes = args12
        getattr(lib, pre).restype = ctypes.c_int
        getattr(lib, pre + "_ex").argtypes = lib.gemm_f16_ex.argtypes
        getattr(lib, pre + "_ex").restype = ctypes.c_int
        getattr(lib, pre + "_plan").argtypes = lib.gemm_f16_plan.argtypes
        getattr(lib, pre + "_plan").restype = ctypes.c_int
        getattr(lib, pre + "_workspace_bytes").argtypes = lib.gemm_f16_workspace_bytes.argtypes
        getattr(lib, pre + "_workspace_bytes").restype = sz
    args14 = [vp, i64, i64, vp, i64, i64, vp, i64, i64, i64, i64, i32, i32, vp]
    lib.gemm_f8.argtypes = args14
    lib.gemm_f8.restype = ctypes.c_int
    lib.gemm_f8_ex.argtypes = args14 + [vp, sz, ctypes.POINTER(Opts)]
    lib.gemm_f8_ex.restype = ctypes.c_int
    lib.gemm_f8_plan.argtypes = [vp, i64, i64, vp, i64, i64, vp, i64, i64, i64, i64, i32, i32,
                                 ctypes.POINTER(Opts), ctypes.POINTER(PlanInfo)]
    lib.gemm_f8_plan.restype = ctypes.c_int
    lib.gemm_f8_plan_cus.argtypes = [vp, i64, i64, vp, i64, i64, vp, i64, i64, i64, i64, i32, i32, i32,
                                     ctypes.POINTER(Opts), ctypes.POINTER(PlanInfo)]
    lib.gemm_f8_plan_cus.restype = ctypes.c_int
    lib.gemm_f8_workspace_bytes.argtypes = [i64, i64, i64, ctypes.POINTER(Opts)]
    lib.gemm_f8_workspace_bytes.restype = sz
    lib.gemm_f16_packed_b_bytes.argtypes = [i64, i64]
    lib.gemm_f16_packed_b_bytes.restype = sz
    lib.gemm_f16_pack_b.argtypes = [vp, i64, i64, i64, i64, vp, vp]
    lib.gemm_f16_pack_b.restype = ctypes.c_int
    lib.gemm_f16_packed.argtypes = [vp, i64, i64, vp, vp, i64, i64, i64, i64, vp]
    lib.gemm_f16_packed.restype = ctypes.c_int
    lib.gemm_f16_grouped.argtypes = [vp, i64, i64, vp, i64, i64, i64, vp, i64, vp, i32,
                                     i64, i64, i64, vp, vp, sz]
    lib.gemm_f16_grouped.restype = ctypes.c_int
    lib.gemm_bf16_grouped.argtypes = lib.gemm_f16_grouped.argtypes
    lib.gemm_bf16_grouped.restype = ctypes.c_int
    lib.gemm_f8_grouped.argtypes = [vp, i64, i64, vp, i64, i64, i64, vp, i64, vp, i32, i64, i64, i64,
                                    i32, i32, vp, vp, sz]
    lib.gemm_f8_grouped.restype = ctypes.c_int
    lib.gemm_f16_grouped_workspace_bytes.argtypes = [i32]
    lib.gemm_f16_grouped_workspace_bytes.restype = sz
    lib.gemm_f16_status_string.argtypes = [ctypes.c_int]
    lib.gemm_f16_status_string.restype = ctypes.c_char_p
    lib.gemm_f16_version.argtypes = []
    lib.gemm_f16_version.restype = ctypes.c_int
    return lib


lib = _load()
LIB_PATH = _build.LIB


def status_string(rc):
    return lib.gemm_f16_status_string(rc).decode()


def make_opts(variant=0, split_k=0, panel=0, tile=0):
    if isinstance(variant, str):
        variant = VARIANTS[variant]
    return Opts(variant, split_k, panel, tile)
