"""ctypes mirror of include/qv.h and the loader of libqv.so.

torch is imported before the library is opened so that libqv.so binds to the
HIP runtime torch has already loaded (both carry the SONAME
libamdhip64.so.7); device pointers and streams from torch are then valid in
the library.  A missing library is an error: there is no fallback path."""
from __future__ import annotations

import ctypes
import os
import re
from ctypes import POINTER, Structure, c_char_p, c_float, c_int32, c_int64, c_size_t, c_uint64, c_void_p

HERE = os.path.dirname(os.path.abspath(__file__))
# QV_LIBRARY names another build of the same ABI (the host-only sanitizer build
# of the test suite); by default the library next to this file.
LIB_PATH = os.environ.get("QV_LIBRARY") or os.path.join(HERE, "libqv.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "qv.h")

QV_OK, QV_ERR_NULL, QV_ERR_SHAPE, QV_ERR_BUDGET, QV_ERR_WORKSPACE, QV_ERR_UNSUPPORTED, QV_ERR_HIP = range(7)
QV_F32, QV_BF16, QV_I8 = 0, 1, 2
QV_SCRATCH_BYTES = 64 << 20   # static workspace of qv_vision_forward_noalloc
STATUS_NAMES = {0: "QV_OK", 1: "QV_ERR_NULL", 2: "QV_ERR_SHAPE", 3: "QV_ERR_BUDGET", 4: "QV_ERR_WORKSPACE",
                5: "QV_ERR_UNSUPPORTED", 6: "QV_ERR_HIP"}


class QvError(RuntimeError):
    def __init__(self, status: int, text: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {text}")
        self.status = status


class GridParams(Structure):
    _fields_ = [("patch", c_int32), ("merge", c_int32), ("temporal", c_int32), ("reserved", c_int32),
                ("min_pixels", c_int64), ("max_pixels", c_int64)]


class Image(Structure):
    _fields_ = [("offset", c_int64), ("frames", c_int32), ("channels", c_int32), ("height", c_int32),
                ("width", c_int32), ("reserved", c_int32)]


class PatchOpts(Structure):
    _fields_ = [("fold", c_int32), ("normalize", c_int32), ("mean", c_float * 4), ("std", c_float * 4)]


CLIP_MEAN = (0.48145466, 0.4578275, 0.40821073, 0.0)
CLIP_STD = (0.26862954, 0.26130258, 0.27577711, 1.0)


BLOCK_FIELDS = ("ln1_w", "ln1_b", "qkv_w", "qkv_b", "proj_w", "proj_b",
                "ln2_w", "ln2_b", "fc1_w", "fc1_b", "fc2_w", "fc2_b")


# float32 row scales of the int8 block matrices (qv_vision_cfg.weights = QV_I8)
BLOCK_SCALE_FIELDS = ("qkv_s", "proj_s", "fc1_s", "fc2_s")
QUANT_FIELDS = ("qkv_w", "proj_w", "fc1_w", "fc2_w")


class BlockW(Structure):
    _fields_ = [(k, c_void_p) for k in BLOCK_FIELDS + BLOCK_SCALE_FIELDS]


class VisionW(Structure):
    _fields_ = [("patch_w", c_void_p), ("patch_b", c_void_p), ("blocks", POINTER(BlockW))]


class VisionCfg(Structure):
    _fields_ = [("depth", c_int32), ("dim", c_int32), ("heads", c_int32), ("mlp", c_int32),
                ("patch_dim", c_int32), ("ld", c_int32), ("merge", c_int32), ("dtype", c_int32),
                ("ln_eps", c_float), ("rope_theta", c_float), ("window", c_int32), ("weights", c_int32),
                ("full_blocks", c_uint64)]


class MergerCfg(Structure):
    _fields_ = [("dim", c_int32), ("merge", c_int32), ("hidden", c_int32), ("out_dim", c_int32),
                ("dtype", c_int32), ("ln_eps", c_float)]


KERNEL_CLASSES = ("patchify", "patch_embed", "layernorm", "qkv", "attention", "proj", "fc1", "fc2",
                  "merge_fc1", "merge_fc2")

MERGER_FIELDS = ("ln_w", "ln_b", "fc1_w", "fc1_b", "fc2_w", "fc2_b")


class MergerW(Structure):
    _fields_ = [(k, c_void_p) for k in MERGER_FIELDS]


_lib = None


def header_functions() -> list:
    """Names of the functions include/qv.h declares."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qv_[a-z_0-9]+)\s*\(", text)))


def lib() -> ctypes.CDLL:
    """Open libqv.so once (after torch), with argument types declared."""
    global _lib
    if _lib is not None:
        return _lib
    import torch  # noqa: F401  (binds libqv.so to torch's HIP runtime)
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it first (python -c 'import __graft_entry__ as g; g.build()')")
    L = ctypes.CDLL(LIB_PATH)
    L.qv_last_error.restype = c_char_p
    L.qv_last_error.argtypes = []
    L.qv_abi_version.restype = c_int32
    L.qv_grid_params_default.restype = None
    L.qv_grid_params_default.argtypes = [POINTER(GridParams)]
    L.qv_smart_resize_grid.restype = c_int32
    L.qv_smart_resize_grid.argtypes = [c_int64, c_int64, c_int32, POINTER(GridParams), POINTER(c_int64),
                                       POINTER(c_int64), POINTER(c_int32)]
    L.qv_seq_meta.restype = c_int32
    L.qv_seq_meta.argtypes = [c_void_p, c_int32, c_int32, c_void_p, c_void_p, c_void_p]
    L.qv_patchify.restype = c_int32
    L.qv_patchify.argtypes = [c_void_p, POINTER(Image), c_int32, c_void_p, POINTER(GridParams), c_void_p, c_int32,
                              c_int32, c_void_p]
    L.qv_patchify_ex.restype = c_int32
    L.qv_patchify_ex.argtypes = [c_void_p, POINTER(Image), c_int32, c_void_p, POINTER(GridParams),
                                 POINTER(PatchOpts), c_void_p, c_int32, c_int32, c_void_p]
    L.qv_fold_patch_weight.restype = c_int32
    L.qv_fold_patch_weight.argtypes = [c_void_p, c_int32, c_int32, c_int32, c_int32, c_int32, c_void_p, c_int32,
                                       c_int32, c_void_p]
    L.qv_quantize_i8.restype = c_int32
    L.qv_quantize_i8.argtypes = [c_void_p, c_int32, c_int32, c_int32, c_int32, c_void_p, c_void_p, c_void_p]
    L.qv_vision_workspace_size.restype = c_int32
    L.qv_vision_workspace_size.argtypes = [POINTER(VisionCfg), c_void_p, c_int32, POINTER(c_size_t)]
    L.qv_vision_forward.restype = c_int32
    L.qv_vision_forward.argtypes = [POINTER(VisionCfg), POINTER(VisionW), c_void_p, c_void_p, c_int32, c_void_p,
                                    c_void_p, c_void_p, c_size_t, c_void_p]
    L.qv_vision_forward_noalloc.restype = c_int32
    L.qv_vision_forward_noalloc.argtypes = [POINTER(VisionCfg), POINTER(VisionW), c_void_p, c_void_p, c_int32,
                                            c_void_p, c_void_p, c_void_p]
    L.qv_merge_workspace_size.restype = c_int32
    L.qv_merge_workspace_size.argtypes = [POINTER(MergerCfg), c_int64, POINTER(c_size_t)]
    L.qv_patch_merge.restype = c_int32
    L.qv_patch_merge.argtypes = [POINTER(MergerCfg), POINTER(MergerW), c_void_p, c_int64, c_void_p, c_void_p,
                                 c_size_t, c_void_p]
    L.qv_timing_start.restype = c_int32
    L.qv_timing_start.argtypes = [c_int32]
    L.qv_timing_stop.restype = c_int32
    L.qv_timing_stop.argtypes = [POINTER(ctypes.c_double), POINTER(c_int64)]
    _lib = L
    return L


def check(status: int) -> None:
    if status != QV_OK:
        raise QvError(status, lib().qv_last_error().decode())
