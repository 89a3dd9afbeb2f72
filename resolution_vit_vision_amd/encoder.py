"""Thin torch-facing binding of the qv C ABI.

Everything here marshals arguments: torch tensors become device pointers,
the current torch stream becomes the hipStream_t, Python lists become host
arrays.  Every step of the encoder runs inside libqv.so."""
from __future__ import annotations

import ctypes
from dataclasses import dataclass
from typing import Dict, List, Sequence, Tuple

import numpy as np
import torch

from . import _abi
from ._abi import check, lib

DTYPES = {"bf16": _abi.QV_BF16, "f32": _abi.QV_F32}
TORCH_DTYPES = {"bf16": torch.bfloat16, "f32": torch.float32}


def _stream(stream=None) -> ctypes.c_void_p:
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t) -> ctypes.c_void_p:
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def grid_params(patch=14, merge=2, temporal=2, min_pixels=3136, max_pixels=12845056) -> _abi.GridParams:
    return _abi.GridParams(patch, merge, temporal, 0, min_pixels, max_pixels)


# ------------------------------------------------------------------ host calls
def smart_resize_grid(height: int, width: int, frames: int = 1, **kw) -> Tuple[int, int, Tuple[int, int, int]]:
    p = grid_params(**kw)
    oh, ow = ctypes.c_int64(), ctypes.c_int64()
    g = (ctypes.c_int32 * 3)()
    check(lib().qv_smart_resize_grid(height, width, frames, ctypes.byref(p), ctypes.byref(oh), ctypes.byref(ow), g))
    return oh.value, ow.value, (g[0], g[1], g[2])


def _grid_array(grids) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(grids, dtype=np.int32).reshape(-1, 3))


def seq_meta(grids, merge: int = 2):
    """(cu_seqlens [n+1], pos_hw [N][2], perm [N]) as int32 numpy arrays."""
    g = _grid_array(grids)
    n = int((g[:, 0].astype(np.int64) * g[:, 1] * g[:, 2]).sum())
    cu = np.zeros(len(g) + 1, np.int32)
    pos = np.zeros((n, 2), np.int32)
    perm = np.zeros(n, np.int32)
    check(lib().qv_seq_meta(g.ctypes.data, len(g), merge, cu.ctypes.data, pos.ctypes.data, perm.ctypes.data))
    return cu, pos, perm


# -------------------------------------------------------------------- patchify
def pack_images(images: Sequence[np.ndarray]):
    """Concatenate host images [F][C][H][W] into one flat float32 array and
    return it with the per-image (offset, frames, channels, height, width)."""
    descs, off = [], 0
    for im in images:
        f, c, h, w = im.shape
        descs.append((off, f, c, h, w))
        off += im.size
    flat = np.concatenate([np.ascontiguousarray(im, dtype=np.float32).ravel() for im in images])
    return flat, descs


def patch_opts(fold: bool = False, normalize=None) -> _abi.PatchOpts:
    """normalize: None/False (off), True (CLIP mean/std) or a (mean, std) pair."""
    o = _abi.PatchOpts()
    o.fold = 1 if fold else 0
    if normalize:
        mean, std = (_abi.CLIP_MEAN, _abi.CLIP_STD) if normalize is True else normalize
        o.normalize = 1
        for i in range(4):
            o.mean[i] = float(mean[i]) if i < len(mean) else 0.0
            o.std[i] = float(std[i]) if i < len(std) else 1.0
    return o


def patch_width(channels: int, fold: bool = False, patch: int = 14, temporal: int = 2) -> int:
    """Row width of the patch matrix: C*T*p*p, or C*p*p rounded up to 8 with the fold."""
    return (channels * patch * patch + 7) // 8 * 8 if fold else channels * temporal * patch * patch


def patchify(pixels: torch.Tensor, descs, grids, dtype: str = "bf16", ld: int | None = None,
             out: torch.Tensor | None = None, stream=None, fold: bool = False, normalize=None,
             **grid_kw) -> torch.Tensor:
    p = grid_params(**grid_kw)
    g = _grid_array(grids)
    arr = (_abi.Image * len(descs))(*[_abi.Image(o, f, c, h, w, 0) for (o, f, c, h, w) in descs])
    n = int((g[:, 0].astype(np.int64) * g[:, 1] * g[:, 2]).sum())
    pd = patch_width(descs[0][2], fold, p.patch, p.temporal)
    ld = pd if ld is None else ld
    if out is None:
        out = torch.empty((n, ld), dtype=TORCH_DTYPES[dtype], device=pixels.device)
    opts = patch_opts(fold, normalize)
    check(lib().qv_patchify_ex(_ptr(pixels), arr, len(descs), g.ctypes.data, ctypes.byref(p), ctypes.byref(opts),
                               _ptr(out), DTYPES[dtype], ld, _stream(stream)))
    return out


def fold_patch_weight(w: torch.Tensor, channels: int = 3, patch: int = 14, temporal: int = 2,
                      ld_out: int | None = None, stream=None) -> torch.Tensor:
    """Conv3d patch-embed weight [dim][C*T*p*p] (device, bf16 or f32) -> the
    Conv2d weight [dim][ld_out] of still images (temporal taps summed)."""
    dim = w.shape[0]
    ld_out = patch_width(channels, True, patch, temporal) if ld_out is None else ld_out
    out = torch.empty((dim, ld_out), dtype=w.dtype, device=w.device)
    dt = "bf16" if w.dtype == torch.bfloat16 else "f32"
    check(lib().qv_fold_patch_weight(_ptr(w), dim, channels, patch, temporal, w.stride(0), _ptr(out), ld_out,
                                     DTYPES[dt], _stream(stream)))
    return out


def quantize_i8(w: torch.Tensor, stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Device matrix [rows][cols] (f32 or bf16) -> (int8 codes [rows][cols],
    float32 row scales [rows]) by qv_quantize_i8."""
    rows, cols = w.shape
    q = torch.empty((rows, cols), dtype=torch.int8, device=w.device)
    sc = torch.empty(rows, dtype=torch.float32, device=w.device)
    dt = "bf16" if w.dtype == torch.bfloat16 else "f32"
    check(lib().qv_quantize_i8(_ptr(w), rows, cols, w.stride(0), DTYPES[dt], _ptr(q), _ptr(sc), _stream(stream)))
    return q, sc


# --------------------------------------------------------------------- weights
WEIGHT_FORMATS = {"dtype": 0, "int8": _abi.QV_I8}


@dataclass
class VisionConfig:
    depth: int
    dim: int = 1280
    heads: int = 16
    mlp: int = 5120
    patch_dim: int = 1176
    ld: int = 1176
    merge: int = 2
    dtype: str = "bf16"
    ln_eps: float = 1e-6
    rope_theta: float = 1e4
    window: int = 0                 # window side in patches (0: full attention in every block)
    full_blocks: Tuple[int, ...] = ()  # blocks that keep full attention when window > 0
    weights: str = "dtype"          # block matrices: "dtype" (as the tower) or "int8"

    def c(self) -> _abi.VisionCfg:
        mask = 0
        for b in self.full_blocks:
            if not 0 <= b < 64:
                raise ValueError(f"full-attention block {b} outside 0..63")
            mask |= 1 << b
        return _abi.VisionCfg(self.depth, self.dim, self.heads, self.mlp, self.patch_dim, self.ld, self.merge,
                              DTYPES[self.dtype], self.ln_eps, self.rope_theta, self.window,
                              WEIGHT_FORMATS[self.weights], mask)


@dataclass
class MergerConfig:
    dim: int = 1280
    merge: int = 2
    out_dim: int = 1536
    dtype: str = "bf16"
    ln_eps: float = 1e-6

    def c(self) -> _abi.MergerCfg:
        return _abi.MergerCfg(self.dim, self.merge, self.dim * self.merge ** 2, self.out_dim, DTYPES[self.dtype],
                              self.ln_eps)


def _dev(a: np.ndarray, dtype: str, device, matrix: bool) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    if matrix and dtype == "bf16":
        t = t.to(torch.bfloat16)
    return t.to(device)


class VisionWeights:
    """Device copies of the tower parameters and the ctypes struct pointing at
    them.  fold: the Conv3d patch-embed weight is folded on the device into
    the Conv2d weight of still images (qv_fold_patch_weight).  weights="int8":
    the four block matrices are quantized on the device from their float32
    values (qv_quantize_i8) and kept only as int8 codes and row scales."""

    def __init__(self, params: Dict[str, np.ndarray], depth: int, dtype: str = "bf16", device="cuda",
                 fold: bool = False, weights: str = "dtype"):
        if weights not in WEIGHT_FORMATS:
            raise ValueError(f"weights must be one of {sorted(WEIGHT_FORMATS)}")
        self.tensors: Dict[str, torch.Tensor] = {}
        pw = params["patch_w"]
        self.tensors["patch_w"] = _dev(pw.reshape(pw.shape[0], -1), dtype, device, True)
        if fold:
            _, c, t, p, _ = pw.shape
            self.tensors["patch_w_conv3d"] = self.tensors["patch_w"]
            self.tensors["patch_w"] = fold_patch_weight(self.tensors["patch_w"], c, p, t)
        self.patch_b = None
        if "patch_b" in params:
            self.patch_b = _dev(params["patch_b"], dtype, device, False)
        blocks = (_abi.BlockW * max(depth, 1))()
        for l in range(depth):
            vals, scales = [], {}
            for k in _abi.BLOCK_FIELDS:
                a = params[f"blocks.{l}.{k}"]
                if weights == "int8" and k in _abi.QUANT_FIELDS:
                    t, sc = quantize_i8(_dev(a, "f32", device, True))
                    self.tensors[f"blocks.{l}.{k[:-2]}_s"] = sc
                    scales[k[:-2] + "_s"] = sc.data_ptr()
                else:
                    t = _dev(a, dtype, device, a.ndim == 2)
                self.tensors[f"blocks.{l}.{k}"] = t
                vals.append(t.data_ptr())
            vals += [scales.get(k, 0) for k in _abi.BLOCK_SCALE_FIELDS]
            blocks[l] = _abi.BlockW(*vals)
        self._blocks = blocks
        self.struct = _abi.VisionW(self.tensors["patch_w"].data_ptr(),
                                   0 if self.patch_b is None else self.patch_b.data_ptr(), blocks)


class MergerWeights:
    def __init__(self, params: Dict[str, np.ndarray], dtype: str = "bf16", device="cuda"):
        self.tensors = {}
        vals = []
        for k in _abi.MERGER_FIELDS:
            a = params[f"merger.{k}"]
            t = _dev(a, dtype, device, a.ndim == 2)
            self.tensors[k] = t
            vals.append(t.data_ptr())
        self.struct = _abi.MergerW(*vals)


# ------------------------------------------------------------------ forward
def vision_workspace_size(cfg: VisionConfig, grids) -> int:
    g = _grid_array(grids)
    n = ctypes.c_size_t()
    check(lib().qv_vision_workspace_size(ctypes.byref(cfg.c()), g.ctypes.data, len(g), ctypes.byref(n)))
    return n.value


def vision_forward(cfg: VisionConfig, w: VisionWeights, patches: torch.Tensor, grids, cu_seqlens: torch.Tensor,
                   hidden: torch.Tensor | None = None, ws: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    g = _grid_array(grids)
    n = int((g[:, 0].astype(np.int64) * g[:, 1] * g[:, 2]).sum())
    if hidden is None:
        hidden = torch.empty((n, cfg.dim), dtype=torch.float32, device=patches.device)
    if ws is None:
        ws = torch.empty(vision_workspace_size(cfg, g), dtype=torch.uint8, device=patches.device)
    c = cfg.c()
    check(lib().qv_vision_forward(ctypes.byref(c), ctypes.byref(w.struct), _ptr(patches), g.ctypes.data, len(g),
                                  _ptr(cu_seqlens), _ptr(hidden), _ptr(ws), ws.numel(), _stream(stream)))
    return hidden


def vision_forward_noalloc(cfg: VisionConfig, w: VisionWeights, patches: torch.Tensor, grids,
                           cu_seqlens: torch.Tensor, hidden: torch.Tensor, stream=None) -> torch.Tensor:
    """qv_vision_forward_noalloc: the same forward with the library's static
    device workspace (no allocation by the library or here; `hidden` is the
    caller's)."""
    g = _grid_array(grids)
    c = cfg.c()
    check(lib().qv_vision_forward_noalloc(ctypes.byref(c), ctypes.byref(w.struct), _ptr(patches), g.ctypes.data,
                                          len(g), _ptr(cu_seqlens), _ptr(hidden), _stream(stream)))
    return hidden


def merge_workspace_size(cfg: MergerConfig, n_tokens: int) -> int:
    n = ctypes.c_size_t()
    check(lib().qv_merge_workspace_size(ctypes.byref(cfg.c()), n_tokens, ctypes.byref(n)))
    return n.value


def patch_merge(cfg: MergerConfig, w: MergerWeights, hidden: torch.Tensor, out: torch.Tensor | None = None,
                ws: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    n = hidden.shape[0]
    g = cfg.merge ** 2
    if out is None:
        out = torch.empty((n // g, cfg.out_dim), dtype=TORCH_DTYPES[cfg.dtype], device=hidden.device)
    if ws is None:
        ws = torch.empty(merge_workspace_size(cfg, n), dtype=torch.uint8, device=hidden.device)
    c = cfg.c()
    check(lib().qv_patch_merge(ctypes.byref(c), ctypes.byref(w.struct), _ptr(hidden), n, _ptr(out), _ptr(ws),
                               ws.numel(), _stream(stream)))
    return out


class Encoder:
    """One configured encoder with device weights and preallocated buffers for a
    fixed image list: run() enqueues patchify -> tower -> merger."""

    def __init__(self, params: Dict[str, np.ndarray], images: Sequence[np.ndarray], depth: int, out_dim: int,
                 dtype: str = "bf16", dim: int = 1280, heads: int = 16, mlp: int = 5120, ln_eps: float = 1e-6,
                 rope_theta: float = 1e4, window: int = 0, full_blocks=(), device="cuda", grids=None,
                 fold: bool = False, normalize=None, weights: str = "dtype", **grid_kw):
        self.dtype = dtype
        self.grid_kw = grid_kw
        if grids is None:
            grids = [smart_resize_grid(im.shape[2], im.shape[3], im.shape[0], **grid_kw)[2] for im in images]
        self.grids = [tuple(int(x) for x in g) for g in grids]
        for im, (t, gh, gw) in zip(images, self.grids):
            if im.shape[2] != 14 * gh or im.shape[3] != 14 * gw:
                raise ValueError("image sides must already sit on the 28-pixel lattice inside the budget")
        flat, self.descs = pack_images(images)
        self.pixels = torch.from_numpy(flat).to(device)
        cu, _, _ = seq_meta(self.grids)
        self.cu_host = cu
        self.cu = torch.from_numpy(cu).to(device)
        self.n = int(cu[-1])
        self.fold, self.normalize = fold, normalize
        pd = patch_width(images[0].shape[1], fold)
        self.vcfg = VisionConfig(depth=depth, dim=dim, heads=heads, mlp=mlp, patch_dim=pd, ld=pd, dtype=dtype,
                                 ln_eps=ln_eps, rope_theta=rope_theta, window=window,
                                 full_blocks=tuple(full_blocks), weights=weights)
        self.mcfg = MergerConfig(dim=dim, out_dim=out_dim, dtype=dtype, ln_eps=ln_eps)
        self.vw = VisionWeights(params, depth, dtype, device, fold=fold, weights=weights)
        self.mw = MergerWeights(params, dtype, device)
        self.patches = torch.empty((self.n, pd), dtype=TORCH_DTYPES[dtype], device=device)
        self.hidden = torch.empty((self.n, dim), dtype=torch.float32, device=device)
        self.out = torch.empty((self.n // 4, out_dim), dtype=TORCH_DTYPES[dtype], device=device)
        self.ws = torch.empty(max(vision_workspace_size(self.vcfg, self.grids),
                                  merge_workspace_size(self.mcfg, self.n)), dtype=torch.uint8, device=device)

    def run(self, stream=None):
        patchify(self.pixels, self.descs, self.grids, self.dtype, out=self.patches, stream=stream, fold=self.fold,
                 normalize=self.normalize, **self.grid_kw)
        vision_forward(self.vcfg, self.vw, self.patches, self.grids, self.cu, hidden=self.hidden, ws=self.ws,
                       stream=stream)
        patch_merge(self.mcfg, self.mw, self.hidden, out=self.out, ws=self.ws, stream=stream)
        return self.out


class KernelTimer:
    """Sum of device time over every launch of one kernel class between
    start() and stop(), from hipEvent pairs the library records on the launch
    stream."""

    def __init__(self, kernel_class: str):
        self.cls = _abi.KERNEL_CLASSES.index(kernel_class)

    def start(self):
        check(lib().qv_timing_start(self.cls))

    def stop(self):
        ms = ctypes.c_double()
        n = ctypes.c_int64()
        check(lib().qv_timing_stop(ctypes.byref(ms), ctypes.byref(n)))
        return ms.value, n.value
