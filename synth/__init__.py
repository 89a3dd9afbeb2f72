"""Seeded synthetic inputs for the native-resolution ViT encoder workloads.

This module only *draws numbers*: workload shapes, parameter tensors and
pixels.  It computes no step of the encoder (no grid selection, no patch
order, no rotary angles, no layer arithmetic), so the oracle and the HIP
path can both take their inputs from here without sharing any of the
method.

Recipe (every workload):
  * parameter tensor #i (fixed enumeration order below) is drawn from
    ``numpy.random.default_rng((seed, 0, i))`` as float32 N(0, 0.02);
    LayerNorm gains are 1 + N(0, 0.02).  In bf16 workloads every
    parameter is rounded once to bf16 (round-to-nearest-even), so both
    sides see exactly the same values.
  * image k's pixels are ``default_rng((seed, 1, k)).uniform(-1, 1,
    (frames, 3, H, W))`` float32, channel-major per frame.
  * the mixed-resolution batch draws its 16 (H, W) pairs as
    ``28 * default_rng((seed, 2)).integers(8, 49, size=(16, 2))``:
    each side independently uniform over the multiples of 28 in
    [224, 1344].

Parameter enumeration order: patch-embed weight; then for each block
ln1_w, ln1_b, qkv_w, qkv_b, proj_w, proj_b, ln2_w, ln2_b, fc1_w, fc1_b,
fc2_w, fc2_b; then merger ln_w, ln_b, fc1_w, fc1_b, fc2_w, fc2_b.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Tuple

import numpy as np

BLOCK_KEYS = ("ln1_w", "ln1_b", "qkv_w", "qkv_b", "proj_w", "proj_b",
              "ln2_w", "ln2_b", "fc1_w", "fc1_b", "fc2_w", "fc2_b")
MERGER_KEYS = ("ln_w", "ln_b", "fc1_w", "fc1_b", "fc2_w", "fc2_b")


@dataclass(frozen=True)
class Workload:
    """One encoder workload: the images it packs and the tower it runs."""
    name: str
    images: Tuple[Tuple[int, int, int], ...]   # (height, width, frames) per image
    depth: int
    dim: int = 1280
    heads: int = 16
    mlp: int = 5120
    out_dim: int = 1536
    in_channels: int = 3
    patch: int = 14
    temporal: int = 2
    merge: int = 2
    dtype: str = "bf16"                        # "bf16" or "f32"
    ln_eps: float = 1e-6
    rope_theta: float = 1e4
    seed: int = 0
    tol: float = 2e-2                          # rel-L2 bar for this dtype
    window: int = 0                            # attention window side in patches (0: none)
    full_blocks: Tuple[int, ...] = ()          # blocks with full attention when windowed
    description: str = ""

    @property
    def patch_dim(self) -> int:
        return self.in_channels * self.temporal * self.patch * self.patch

    @property
    def merged_dim(self) -> int:
        return self.dim * self.merge * self.merge


def mixed_sides(seed: int = 0, count: int = 16) -> List[Tuple[int, int]]:
    """(H, W) pairs of the mixed native-resolution batch."""
    hw = 28 * np.random.default_rng((seed, 2)).integers(8, 49, size=(count, 2))
    return [(int(h), int(w)) for h, w in hw]


def _workloads() -> Dict[str, Workload]:
    toy = Workload(
        name="toy_112_fp32", images=((112, 112, 1),), depth=2, dtype="f32", tol=1e-4,
        description="one 112x112 image, 8x8 grid, 2 blocks, merger to 1536, fp32")
    w448 = Workload(
        name="qwen2vl_2b_448", images=((448, 448, 1),), depth=32,
        description="one 448x448 image, 32x32 grid, 32 blocks, merger to 1536, bf16")
    w672x4 = Workload(
        name="qwen2vl_2b_672x4_varlen", images=((672, 672, 1),) * 4, depth=32,
        description="four 672x672 images packed varlen, 32 blocks, merger to 1536, bf16")
    mixed = Workload(
        name="mixed16_varlen_7b_merger",
        images=tuple((h, w, 1) for h, w in mixed_sides(0, 16)), depth=32, out_dim=3584,
        description="16 images, sides uniform over multiples of 28 in [224,1344], "
                    "32 blocks, merger to 3584, bf16")
    maxres = Workload(
        name="maxres_3584", images=((3584, 3584, 1),), depth=32, out_dim=3584,
        description="one 3584x3584 image, 256x256 grid, 32 blocks, merger to 3584, bf16")
    maxres_win = Workload(
        name="qwen25vl_7b_3584_window", images=((3584, 3584, 1),), depth=32, out_dim=3584, window=8,
        full_blocks=(7, 15, 23, 31),
        description="one 3584x3584 image, 256x256 grid, 32 blocks attending in 8x8-patch windows "
                    "except blocks 7/15/23/31, merger to 3584, bf16")
    video = Workload(
        name="video_448_16f", images=((448, 448, 16),), depth=32,
        description="one 16-frame 448x448 clip (8 temporal patches of distinct frame pairs, one attention "
                    "segment), 32 blocks, merger to 1536, bf16")
    return {w.name: w for w in (toy, w448, w672x4, mixed, maxres, maxres_win, video)}


WORKLOADS: Dict[str, Workload] = _workloads()
TOY, W448, W672X4, MIXED16, MAXRES, MAXRES_WIN, VIDEO16 = (
    WORKLOADS[k] for k in ("toy_112_fp32", "qwen2vl_2b_448", "qwen2vl_2b_672x4_varlen", "mixed16_varlen_7b_merger",
                           "maxres_3584", "qwen25vl_7b_3584_window", "video_448_16f"))


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even), returned as float32.

    Used only to make drawn parameters exactly representable in bf16."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).reshape(x.shape)


def _draw(seed: int, idx: int, shape, gain: bool, bf16: bool) -> np.ndarray:
    g = np.random.default_rng((seed, 0, idx))
    a = g.standard_normal(int(np.prod(shape)), dtype=np.float32).reshape(shape) * np.float32(0.02)
    if gain:
        a += np.float32(1.0)
    return round_bf16(a) if bf16 else a


def param_shapes(wl: Workload, depth: int | None = None):
    """(name, shape, is_ln_gain) in enumeration order."""
    d, m, hid, o = wl.dim, wl.mlp, wl.merged_dim, wl.out_dim
    out = [("patch_w", (d, wl.in_channels, wl.temporal, wl.patch, wl.patch), False)]
    blk = {"ln1_w": ((d,), True), "ln1_b": ((d,), False),
           "qkv_w": ((3 * d, d), False), "qkv_b": ((3 * d,), False),
           "proj_w": ((d, d), False), "proj_b": ((d,), False),
           "ln2_w": ((d,), True), "ln2_b": ((d,), False),
           "fc1_w": ((m, d), False), "fc1_b": ((m,), False),
           "fc2_w": ((d, m), False), "fc2_b": ((d,), False)}
    for l in range(wl.depth if depth is None else depth):
        for k in BLOCK_KEYS:
            out.append((f"blocks.{l}.{k}", blk[k][0], blk[k][1]))
    mer = {"ln_w": ((d,), True), "ln_b": ((d,), False), "fc1_w": ((hid, hid), False),
           "fc1_b": ((hid,), False), "fc2_w": ((o, hid), False), "fc2_b": ((o,), False)}
    for k in MERGER_KEYS:
        out.append((f"merger.{k}", mer[k][0], mer[k][1]))
    return out


def params(wl: Workload, depth: int | None = None) -> Dict[str, np.ndarray]:
    """All parameters as float32 arrays (bf16-exact for bf16 workloads).

    ``depth`` < wl.depth draws only the first blocks; the merger keeps its
    enumeration index of the full tower so its values never change."""
    bf16 = wl.dtype == "bf16"
    shapes = param_shapes(wl)
    want = wl.depth if depth is None else depth
    out: Dict[str, np.ndarray] = {}
    for i, (name, shape, gain) in enumerate(shapes):
        if name.startswith("blocks."):
            if int(name.split(".")[1]) >= want:
                continue
        out[name] = _draw(wl.seed, i, shape, gain, bf16)
    return out


def pixels(wl: Workload) -> List[np.ndarray]:
    """Per image float32 array [frames][channels][H][W], U(-1, 1)."""
    out = []
    for k, (h, w, f) in enumerate(wl.images):
        g = np.random.default_rng((wl.seed, 1, k))
        out.append(g.uniform(-1.0, 1.0, (f, wl.in_channels, h, w)).astype(np.float32))
    return out


def small_workload(name: str, images, depth: int = 2, dtype: str = "bf16", out_dim: int = 1536,
                   seed: int = 0) -> Workload:
    """A reduced workload with the full tower widths, for tests at oracle-friendly sizes."""
    return Workload(name=name, images=tuple(tuple(x) for x in images), depth=depth, dtype=dtype,
                    out_dim=out_dim, seed=seed, tol=1e-4 if dtype == "f32" else 2e-2)
