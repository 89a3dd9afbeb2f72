"""Plain CPU oracle of the Qwen2-VL native-resolution vision encoder forward pass.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this module; the product path
never does.  It shares no code with the HIP library and imports nothing
from it.

What it computes, step by step (sources are the reference pages, cited by
title and section):

  grid        smart resize to multiples of patch*merge = 28 inside a pixel
              budget, grid_thw = (T, H/14, W/14)
              [Qwen2-VL ZeroModels docs: intro and Qwen2VLImageProcessor
              table; Qwen2.5-VL-7B-Instruct record: VISION TOKENS]
  seq_meta    2x2 merge-group order of the patches, (h, w) of each patch,
              cu_seqlens of the packed images
              [Qwen2-VL-2B LiteRT-LM card, Conversion notes: static
              rewrite / No GATHER_ND bullets]
  patchify    2x14x14x3 temporal patches, a still frame duplicated
              [LiteRT-LM card, Conversion notes: Conv3d -> Conv2d fold]
  normalize   optional per-channel CLIP normalisation of the pixels
              [ZeroModels docs, Qwen2VLImageProcessor table: image_mean,
              image_std]
  fold        still images: the duplicated frame folded into a Conv2d
              weight summed over the temporal taps, K = C*14*14
              [LiteRT-LM card, Conversion notes: Conv3d -> Conv2d fold]
  quantize    optional int8 weights of the block matrices: symmetric, one
              scale per output channel [LiteRT-LM card, table rows Vision /
              Adapter: int8 weights]
  patch_embed Conv3d with kernel = stride = (2,14,14) as a matrix product
  rope        2-D rotary positions over the (h, w) patch grid
              [Neurarch Qwen2-VL card, Structure table row "2D RoPE";
              LiteRT-LM card, Conversion notes]
  block       pre-norm ViT block: LN -> MHA (16 x 80) -> residual,
              LN -> MLP 5120 QuickGELU -> residual
              [Neurarch card, Structure table ViT Block rows; ZeroModels
              docs, Qwen2VLModel vision_* arguments]
  attention   full bidirectional attention inside each image of a packed
              batch (block-diagonal by cu_seqlens) [LiteRT-LM card,
              Conversion notes]
  windows     optional windowed attention (Qwen2.5-VL style): attention
              inside windows of `window` x `window` patches except in the
              listed full-attention blocks [Qwen2.5-VL-7B-Instruct record,
              TWO-PART MODEL]
  merge       LayerNorm -> 4 consecutive tokens concatenated (5120) ->
              Linear -> GELU -> Linear to the decoder width
              [Neurarch card, Exported PyTorch: PatchMerger; LiteRT-LM
              card, Adapter row]

Readings where the pages are silent are listed in the design notes of the
repository; each is restated at the function that takes it.

Arithmetic is float64 by default (``dtype`` argument), with numpy's BLAS
for matrix products.  Parity: every function here is pinned by a CPU test
against page values, closed forms, invariants, brute force or a library
routine (tests/test_oracle_pins.py).
"""
from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor
import os
from typing import Dict, List, Sequence, Tuple

import numpy as np

PATCH = 14
MERGE = 2
TEMPORAL = 2
MIN_PIXELS = 3136
MAX_PIXELS = 12845056
CLIP_MEAN = (0.48145466, 0.4578275, 0.40821073)
CLIP_STD = (0.26862954, 0.26130258, 0.27577711)


# ---------------------------------------------------------------- grid (integer)
def smart_resize(height: int, width: int, factor: int = PATCH * MERGE,
                 min_pixels: int = MIN_PIXELS, max_pixels: int = MAX_PIXELS) -> Tuple[int, int]:
    """Resized (H', W'): both multiples of ``factor`` and H'W' inside [min, max].

    The pages fix only the constraints (sides multiples of 28, pixel budget
    3136 .. 12,845,056, tokens = pixels / 784) [ZeroModels docs intro;
    Qwen2.5-VL-7B record, VISION TOKENS].  Reading taken: each side goes to
    the nearest multiple (ties to even, never below one factor); if the
    area then exceeds the budget both sides shrink by the common factor
    beta = sqrt(HW / max) and round down; if it falls short both grow by
    sqrt(min / HW) and round up.  A result still outside the budget
    (extreme aspect ratios) is an error.  Double-precision expressions are
    evaluated in this exact order.
    """
    if height <= 0 or width <= 0:
        raise ValueError("image sides must be positive")
    h = max(factor, int(round(height / factor)) * factor)
    w = max(factor, int(round(width / factor)) * factor)
    if h * w > max_pixels:
        beta = math.sqrt((height * width) / max_pixels)
        h = max(factor, int(math.floor(height / (beta * factor))) * factor)
        w = max(factor, int(math.floor(width / (beta * factor))) * factor)
    elif h * w < min_pixels:
        beta = math.sqrt(min_pixels / (height * width))
        h = int(math.ceil(height * beta / factor)) * factor
        w = int(math.ceil(width * beta / factor)) * factor
    if not (min_pixels <= h * w <= max_pixels):
        raise ValueError(f"no grid inside the pixel budget for {height}x{width}")
    return h, w


def grid_thw(height: int, width: int, frames: int = 1, patch: int = PATCH, merge: int = MERGE,
             temporal: int = TEMPORAL, min_pixels: int = MIN_PIXELS,
             max_pixels: int = MAX_PIXELS) -> Tuple[int, int, Tuple[int, int, int]]:
    """(H', W', (T, H'/patch, W'/patch)) with T = ceil(frames / temporal)
    [ZeroModels docs: image_grid_thw, temporal_patch_size]."""
    h, w = smart_resize(height, width, patch * merge, min_pixels, max_pixels)
    t = -(-frames // temporal)
    return h, w, (t, h // patch, w // patch)


# ---------------------------------------------------------- order and positions
def seq_meta(grids: Sequence[Tuple[int, int, int]], merge: int = MERGE):
    """cu_seqlens, (h, w) per sequence slot, and slot -> raster index.

    Each image's patches are listed so that every merge x merge group is
    contiguous: slot order enumerates (t, block row, block col, dy, dx)
    with dx fastest [LiteRT-LM card, Conversion notes: the 2x2-block order
    the merger expects].  The order of the four members, (0,0), (0,1),
    (1,0), (1,1), is the order of the four strided slices the same bullet
    lists.  Images are concatenated in input order; cu_seqlens holds the
    running patch counts.
    """
    cu = [0]
    pos: List[Tuple[int, int]] = []
    perm: List[int] = []
    for (t, gh, gw) in grids:
        if gh % merge or gw % merge:
            raise ValueError("grid sides must be multiples of the merge size")
        for tt in range(t):
            for bh in range(gh // merge):
                for bw in range(gw // merge):
                    for dy in range(merge):
                        for dx in range(merge):
                            h = merge * bh + dy
                            w = merge * bw + dx
                            pos.append((h, w))
                            perm.append(tt * gh * gw + h * gw + w)
        cu.append(cu[-1] + t * gh * gw)
    return (np.asarray(cu, dtype=np.int64), np.asarray(pos, dtype=np.int64).reshape(-1, 2),
            np.asarray(perm, dtype=np.int64))


# ------------------------------------------------------------------ patchify
def raster_patches(frames: np.ndarray, grid: Tuple[int, int, int], patch: int = PATCH,
                   temporal: int = TEMPORAL) -> np.ndarray:
    """Patch vectors of one image in raster order (t, h, w).

    ``frames`` is [F][C][H][W].  A patch vector lists (channel, temporal
    slot, row, col) with col fastest, i.e. the flattening of a Conv3d
    weight [out][C][temporal][patch][patch] [LiteRT-LM card, Conversion
    notes: the patch-embed is a Conv3d over 2 frames].  Temporal slot tau of
    temporal patch t reads frame min(temporal*t + tau, F-1), so a still
    image is duplicated into both slots [same bullet].
    """
    f, c, hh, ww = frames.shape
    t, gh, gw = grid
    if hh != gh * patch or ww != gw * patch:
        raise ValueError("image sides must equal grid * patch (no resampling)")
    idx = [min(temporal * tt + tau, f - 1) for tt in range(t) for tau in range(temporal)]
    x = frames[idx].reshape(t, temporal, c, gh, patch, gw, patch)
    # -> [t][gh][gw][c][temporal][patch row][patch col]
    x = x.transpose(0, 3, 5, 2, 1, 4, 6)
    return x.reshape(t * gh * gw, c * temporal * patch * patch)


def patchify(images: Sequence[np.ndarray], grids: Sequence[Tuple[int, int, int]],
             merge: int = MERGE) -> np.ndarray:
    """Packed patch matrix [N][C*2*14*14] in merge-group order (float32 values)."""
    _, _, perm = seq_meta(grids, merge)
    rows = []
    start = 0
    for img, g in zip(images, grids):
        r = raster_patches(img, g)
        n = r.shape[0]
        rows.append(r[perm[start:start + n]])
        start += n
    return np.concatenate(rows, axis=0)


def normalize(frames: np.ndarray, mean: Sequence[float] = CLIP_MEAN,
              std: Sequence[float] = CLIP_STD) -> np.ndarray:
    """Per-channel normalisation (x - mean_c) / std_c of [F][C][H][W] pixels,
    in float32 arithmetic (one subtraction, one division per value), with the
    processor's CLIP mean and std by default [ZeroModels docs,
    Qwen2VLImageProcessor table].  Reading: the pixels are already rescaled
    to [0, 1]; the rescale itself is the caller's."""
    x = np.asarray(frames, dtype=np.float32)
    c = x.shape[1]
    m = np.asarray(mean, dtype=np.float32)[:c].reshape(1, c, 1, 1)
    sd = np.asarray(std, dtype=np.float32)[:c].reshape(1, c, 1, 1)
    return (x - m) / sd


def patchify_folded(images: Sequence[np.ndarray], grids: Sequence[Tuple[int, int, int]],
                    merge: int = MERGE, patch: int = PATCH, width: int | None = None) -> np.ndarray:
    """Patch matrix of still images for the folded (Conv2d) patch-embed:
    row = the [C][14][14] pixels of the patch in the single frame, in the
    same merge-group order as ``patchify``; columns past C*14*14 up to
    ``width`` are zero.  A still image is duplicated into both temporal
    slots of the Conv3d, so the product with the temporally summed weight
    (``fold_patch_weight``) equals the Conv3d result [LiteRT-LM card,
    Conversion notes: Conv3d -> Conv2d fold].  Images with more than one
    frame are rejected: their temporal slots differ."""
    _, _, perm = seq_meta(grids, merge)
    rows = []
    start = 0
    for img, (t, gh, gw) in zip(images, grids):
        f, c, hh, ww = img.shape
        if f != 1 or t != 1:
            raise ValueError("the Conv2d fold applies to single-frame images only")
        if hh != gh * patch or ww != gw * patch:
            raise ValueError("image sides must equal grid * patch (no resampling)")
        x = img[0].reshape(c, gh, patch, gw, patch).transpose(1, 3, 0, 2, 4).reshape(gh * gw, c * patch * patch)
        rows.append(x[perm[start:start + gh * gw]])
        start += gh * gw
    out = np.concatenate(rows, axis=0)
    if width is not None and width > out.shape[1]:
        out = np.concatenate([out, np.zeros((out.shape[0], width - out.shape[1]), out.dtype)], axis=1)
    return out


def fold_patch_weight(w: np.ndarray, width: int | None = None) -> np.ndarray:
    """Conv3d weight [out][C][T][p][p] -> Conv2d weight [out][C*p*p], summed
    over the T temporal taps in tap order (in the weight's own precision),
    zero-padded to ``width`` columns [LiteRT-LM card, Conversion notes:
    Conv3d -> Conv2d fold]."""
    o, c, t, p, q = w.shape
    acc = w[:, :, 0]
    for tau in range(1, t):
        acc = acc + w[:, :, tau]
    out = acc.reshape(o, c * p * q)
    if width is not None and width > out.shape[1]:
        out = np.concatenate([out, np.zeros((o, width - out.shape[1]), out.dtype)], axis=1)
    return out


# -------------------------------------------------------------- elementwise ops
def bf16_round(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit pattern (uint16), round to nearest, ties to even.

    Plain bit arithmetic on the float32 pattern; NaN never occurs here."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16).reshape(np.shape(x))


def bf16_to_float(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def layer_norm(x: np.ndarray, gamma: np.ndarray, beta: np.ndarray, eps: float = 1e-6) -> np.ndarray:
    """LayerNorm over the last axis: (x - mean) / sqrt(var + eps) * gamma + beta,
    biased variance of the centred values.  eps 1e-6 is the workloads' value
    (the exported PyTorch's LayerNorm default would be 1e-5)."""
    mu = x.mean(axis=-1, keepdims=True)
    xc = x - mu
    var = (xc * xc).mean(axis=-1, keepdims=True)
    return xc / np.sqrt(var + eps) * gamma + beta


def quick_gelu(u: np.ndarray) -> np.ndarray:
    """u * sigmoid(1.702 u), the tower's MLP activation (workload definition)."""
    return u / (1.0 + np.exp(-1.702 * u))


def gelu_erf(u: np.ndarray) -> np.ndarray:
    """Exact GELU 0.5 u (1 + erf(u / sqrt 2)): the merger's nn.GELU() default
    [Neurarch card, Exported PyTorch: PatchMerger]."""
    from scipy.special import erf
    return 0.5 * u * (1.0 + erf(u / math.sqrt(2.0)))


# ---------------------------------------------------------------------- rope
def rope_angles(pos: np.ndarray, head_dim: int = 80, theta: float = 1e4) -> np.ndarray:
    """Rotation angle of each of the head_dim/2 rotation pairs for each slot.

    2-D rotary positions, each patch carrying its own (h, w) [Neurarch card,
    Structure "2D RoPE"; LiteRT-LM card, Conversion notes].  Reading: a
    quarter of the head (20 frequencies omega_k = theta^(-k/20)) rotates by
    h, the next quarter by w; pair j couples element j with element
    j + head_dim/2.  Angles in float64."""
    q = head_dim // 4
    omega = theta ** (-np.arange(q, dtype=np.float64) / q)
    h = pos[:, 0:1].astype(np.float64)
    w = pos[:, 1:2].astype(np.float64)
    return np.concatenate([h * omega, w * omega], axis=1)


def apply_rope(x: np.ndarray, angles: np.ndarray) -> np.ndarray:
    """Rotate each head vector: x'[j] = x[j] cos a_j - x[j+half] sin a_j,
    x'[j+half] = x[j+half] cos a_j + x[j] sin a_j.  x is [N][heads][hd],
    angles [N][hd/2]; cos/sin are evaluated in float64 and used in the
    working precision of x (float64 by default; float32 tables in the float32
    mode, as the rotary tables of the float32 path are)."""
    half = x.shape[-1] // 2
    c = np.cos(angles).astype(x.dtype, copy=False)[:, None, :]
    s = np.sin(angles).astype(x.dtype, copy=False)[:, None, :]
    x1 = x[..., :half]
    x2 = x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


# ----------------------------------------------------------------- attention
def _threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def attention_varlen(q: np.ndarray, k: np.ndarray, v: np.ndarray, cu_seqlens: np.ndarray,
                     q_rows: np.ndarray | None = None, chunk: int = 1024) -> np.ndarray:
    """Full bidirectional attention inside each packed image.

    q, k, v are [N][heads][hd].  For image i (rows cu[i]..cu[i+1]) and each
    head: S = q k^T / sqrt(hd), P = softmax over that image's keys (row max
    subtracted), O = P v [LiteRT-LM card, Conversion notes: packed patches
    with cu_seqlens; one image is one sequence].  ``q_rows`` restricts the
    output to the given query rows (keys are always the whole image).
    Work is spread over (image, head, query chunk) with a thread pool;
    each item is the plain formula."""
    n, heads, hd = q.shape
    scale = 1.0 / math.sqrt(hd)
    rows = np.arange(n) if q_rows is None else np.asarray(q_rows)
    out = np.zeros((len(rows), heads, hd), dtype=q.dtype)
    seg = np.searchsorted(cu_seqlens, rows, side="right") - 1
    jobs = []
    for i in range(len(cu_seqlens) - 1):
        sel = np.nonzero(seg == i)[0]
        if len(sel) == 0:
            continue
        for h in range(heads):
            for c0 in range(0, len(sel), chunk):
                jobs.append((i, h, sel[c0:c0 + chunk]))

    def run(job):
        i, h, sel = job
        a, b = int(cu_seqlens[i]), int(cu_seqlens[i + 1])
        s = (q[rows[sel], h, :] @ k[a:b, h, :].T) * scale
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p /= p.sum(axis=1, keepdims=True)
        out[sel, h, :] = p @ v[a:b, h, :]

    if len(jobs) > 1:
        with ThreadPoolExecutor(max_workers=_threads()) as ex:
            list(ex.map(run, jobs))
    else:
        for j in jobs:
            run(j)
    return out


# --------------------------------------------------------- windowed attention
def window_groups(grids: Sequence[Tuple[int, int, int]], window: int, merge: int = MERGE) -> List[np.ndarray]:
    """Token index lists (packed rows) of the attention windows of a batch.

    The Qwen2.5-VL record keeps the Qwen2-VL tower shapes but lets attention
    run inside windows of 112 px = 8 x 8 patches, with only four blocks
    attending over the whole image [Qwen2.5-VL-7B-Instruct record, TWO-PART
    MODEL].  Readings (the record says nothing more): windows tile each
    frame's patch grid from its top-left corner in steps of ``window``
    patches; a window at the right or bottom edge holds only the patches
    that exist (no padding token takes part); each frame of an image has its
    own windows; a window's tokens keep their packed order.  Windows are
    listed image by image, frame by frame, in raster order."""
    if window <= 0 or window % merge:
        raise ValueError("window must be a positive multiple of the merge size")
    cu, pos, _ = seq_meta(grids, merge)
    groups: List[np.ndarray] = []
    for i, (t, gh, gw) in enumerate(grids):
        nwx = (gw + window - 1) // window
        nwy = (gh + window - 1) // window
        for tt in range(t):
            rows = np.arange(cu[i] + tt * gh * gw, cu[i] + (tt + 1) * gh * gw)
            key = (pos[rows, 0] // window) * nwx + pos[rows, 1] // window
            for wk in range(nwy * nwx):
                groups.append(rows[key == wk])
    return groups


def attention_groups(q: np.ndarray, k: np.ndarray, v: np.ndarray, groups: Sequence[np.ndarray]) -> np.ndarray:
    """Attention inside each group of rows (any row subset, e.g. a window):
    for every group and head, softmax(q k^T / sqrt(hd)) v over the group's
    own keys, row max subtracted.  Rows outside every group stay zero."""
    n, heads, hd = q.shape
    scale = 1.0 / math.sqrt(hd)
    out = np.zeros_like(q)

    def run(g):
        for h in range(heads):
            s = (q[g, h, :] @ k[g, h, :].T) * scale
            s = s - s.max(axis=1, keepdims=True)
            p = np.exp(s)
            p /= p.sum(axis=1, keepdims=True)
            out[g, h, :] = p @ v[g, h, :]

    with ThreadPoolExecutor(max_workers=_threads()) as ex:
        list(ex.map(run, groups))
    return out


# ------------------------------------------------------------------- the tower
def patch_embed(x: np.ndarray, w: np.ndarray, b: np.ndarray | None = None) -> np.ndarray:
    """Conv3d with kernel = stride = (2, 14, 14) on non-overlapping patches is
    X W^T with W the weight flattened to [out][C*2*14*14] [LiteRT-LM card,
    Conversion notes; Neurarch card, Structure "Patchify 14x14"].  No bias in
    the workloads (reading: the pages show none for this tower)."""
    y = x @ w.reshape(w.shape[0], -1).T
    return y if b is None else y + b


def vision_block(z: np.ndarray, p: Dict[str, np.ndarray], cu_seqlens: np.ndarray,
                 angles: np.ndarray, heads: int = 16, eps: float = 1e-6,
                 groups: Sequence[np.ndarray] | None = None) -> np.ndarray:
    """One pre-norm rotary ViT block on the packed residual stream z [N][d].

      a = LN1(z); [q|k|v] = a Wqkv^T + b (q, k, v each head-major);
      q, k rotated by the 2-D rope; o = attention per image (or per
      window when ``groups`` lists the windows);
      z = z + o Wo^T + bo; a = LN2(z); z = z + QuickGELU(a W1^T + b1) W2^T + b2.
    Reading: pre-norm with biases on every Linear, QuickGELU, eps 1e-6, scale
    1/sqrt(hd) (the workloads' definition; the pages' generic exported
    encoder layer is a canvas stand-in, not this tower)."""
    n, d = z.shape
    hd = d // heads
    a = layer_norm(z, p["ln1_w"], p["ln1_b"], eps)
    qkv = a @ p["qkv_w"].T + p["qkv_b"]
    q = qkv[:, 0 * d:1 * d].reshape(n, heads, hd)
    k = qkv[:, 1 * d:2 * d].reshape(n, heads, hd)
    v = qkv[:, 2 * d:3 * d].reshape(n, heads, hd)
    q = apply_rope(q, angles)
    k = apply_rope(k, angles)
    if groups is None:
        o = attention_varlen(q, k, v, cu_seqlens).reshape(n, d)
    else:  # a windowed block: attention inside each window only
        o = attention_groups(q, k, v, groups).reshape(n, d)
    z = z + o @ p["proj_w"].T + p["proj_b"]
    a = layer_norm(z, p["ln2_w"], p["ln2_b"], eps)
    return z + quick_gelu(a @ p["fc1_w"].T + p["fc1_b"]) @ p["fc2_w"].T + p["fc2_b"]


def vision_block_rows(z: np.ndarray, p: Dict[str, np.ndarray], cu_seqlens: np.ndarray,
                      angles: np.ndarray, rows: np.ndarray, heads: int = 16,
                      eps: float = 1e-6, groups: Sequence[np.ndarray] | None = None) -> np.ndarray:
    """The same block evaluated only at output rows ``rows``.

    Keys and values are formed for every row of each image (or window, when
    ``groups`` lists the windows) that holds a requested row; queries,
    projection and MLP only for the requested rows.  Identical arithmetic to
    ``vision_block`` restricted to those outputs, for checks at sizes where
    the whole block is too slow."""
    n, d = z.shape
    hd = d // heads
    rows = np.asarray(rows)
    if groups is None:
        groups = [np.arange(cu_seqlens[i], cu_seqlens[i + 1]) for i in range(len(cu_seqlens) - 1)]
    owner = np.full(n, -1, dtype=np.int64)
    for gi, g in enumerate(groups):
        owner[g] = gi
    used = np.unique(owner[rows])
    if (used < 0).any():
        raise ValueError("a requested row belongs to no attention group")
    kv_rows = np.concatenate([groups[i] for i in used])
    sub_cu = np.concatenate([[0], np.cumsum([len(groups[i]) for i in used])])
    a = layer_norm(z[kv_rows], p["ln1_w"], p["ln1_b"], eps)
    kv = a @ p["qkv_w"][d:].T + p["qkv_b"][d:]
    k = apply_rope(kv[:, :d].reshape(-1, heads, hd), angles[kv_rows])
    v = kv[:, d:].reshape(-1, heads, hd)
    aq = layer_norm(z[rows], p["ln1_w"], p["ln1_b"], eps)
    q = apply_rope((aq @ p["qkv_w"][:d].T + p["qkv_b"][:d]).reshape(-1, heads, hd), angles[rows])
    # place the requested queries at their position inside the gathered images
    where = {int(r): j for j, r in enumerate(kv_rows)}
    qfull = np.zeros((len(kv_rows), heads, hd), dtype=q.dtype)
    local = np.array([where[int(r)] for r in rows])
    qfull[local] = q
    o = attention_varlen(qfull, k, v, sub_cu, q_rows=local).reshape(len(rows), d)
    zr = z[rows] + o @ p["proj_w"].T + p["proj_b"]
    a2 = layer_norm(zr, p["ln2_w"], p["ln2_b"], eps)
    return zr + quick_gelu(a2 @ p["fc1_w"].T + p["fc1_b"]) @ p["fc2_w"].T + p["fc2_b"]


# ------------------------------------------------------------ int8 weights
QUANT_KEYS = ("qkv_w", "proj_w", "fc1_w", "fc2_w")


def quantize_i8(w: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Symmetric int8 weights with one float32 scale per output channel (row)
    [LiteRT-LM card, table rows Vision / Adapter: int8 weights].  The card
    fixes neither the grouping nor the rounding; reading: per row,
    scale = max|w| / 127 (1 for an all-zero row), q = round half to even of
    w / scale, clamped to [-127, 127]; every step in float32 (so the codes are
    a plain function of the float32 weights, reproducible anywhere)."""
    w32 = np.asarray(w, dtype=np.float32)
    amax = np.max(np.abs(w32), axis=1)
    scale = np.where(amax > 0, amax / np.float32(127.0), np.float32(1.0)).astype(np.float32)
    q = np.clip(np.rint(w32 / scale[:, None]), -127, 127).astype(np.int8)
    return q, scale


def dequantized_params(params: Dict[str, np.ndarray], depth: int) -> Dict[str, np.ndarray]:
    """The parameters with every block matrix replaced by q * scale (float64):
    what an int8-weight tower computes with."""
    out = dict(params)
    for l in range(depth):
        for k in QUANT_KEYS:
            q, sc = quantize_i8(params[f"blocks.{l}.{k}"])
            out[f"blocks.{l}.{k}"] = q.astype(np.float64) * sc.astype(np.float64)[:, None]
    return out


def block_params(params: Dict[str, np.ndarray], l: int, dtype=np.float64) -> Dict[str, np.ndarray]:
    pre = f"blocks.{l}."
    return {k[len(pre):]: v.astype(dtype) for k, v in params.items() if k.startswith(pre)}


def vision_forward(x: np.ndarray, params: Dict[str, np.ndarray], grids, depth: int,
                   heads: int = 16, eps: float = 1e-6, theta: float = 1e4,
                   dtype=np.float64, return_all: bool = False, window: int = 0,
                   full_blocks: Sequence[int] = ()):
    """Patch-embed, then ``depth`` rotary blocks over the packed images
    [ZeroModels docs, Qwen2VLVisionModel: patch-embed -> rotary blocks ->
    merger].  Returns the residual stream [N][d] before the merger (the
    encoder output of the LiteRT-LM card's VISION_ENCODER); with
    ``return_all`` also every block's input.  ``window`` > 0 makes every
    block not listed in ``full_blocks`` attend inside windows of that many
    patches (``window_groups``)."""
    cu, pos, _ = seq_meta(grids)
    d = params["patch_w"].shape[0]
    angles = rope_angles(pos, d // heads, theta)
    groups = window_groups(grids, window) if window else None
    z = patch_embed(x.astype(dtype), params["patch_w"].astype(dtype))
    states = [z]
    for l in range(depth):
        g = groups if (groups is not None and l not in full_blocks) else None
        z = vision_block(z, block_params(params, l, dtype), cu, angles, heads, eps, groups=g)
        states.append(z)
    return (z, states) if return_all else z


def patch_merge(z: np.ndarray, params: Dict[str, np.ndarray], merge: int = MERGE,
                eps: float = 1e-6, dtype=np.float64) -> np.ndarray:
    """PatchMerger: LN(d) over each token, then each run of merge^2 consecutive
    tokens concatenated into one row of width merge^2 * d, then Linear ->
    exact GELU -> Linear to the decoder width [Neurarch card, Exported
    PyTorch: PatchMerger; LiteRT-LM card, Adapter row].  Tokens are already
    in merge-group order, so the grouping is a plain reshape.  A token count
    that is not a multiple of merge^2 cannot arise from even grids and is
    rejected."""
    g = merge * merge
    n, d = z.shape
    if n % g:
        raise ValueError("token count must be a multiple of merge^2")
    p = {k[len("merger."):]: v.astype(dtype) for k, v in params.items() if k.startswith("merger.")}
    y = layer_norm(z.astype(dtype), p["ln_w"], p["ln_b"], eps).reshape(n // g, g * d)
    hmid = gelu_erf(y @ p["fc1_w"].T + p["fc1_b"])
    return hmid @ p["fc2_w"].T + p["fc2_b"]


def encode(images: Sequence[np.ndarray], params: Dict[str, np.ndarray], depth: int,
           heads: int = 16, eps: float = 1e-6, theta: float = 1e4, dtype=np.float64,
           min_pixels: int = MIN_PIXELS, max_pixels: int = MAX_PIXELS, window: int = 0,
           full_blocks: Sequence[int] = (), normalize_pixels: bool = False):
    """Whole path for images whose sides already sit on the grid:
    grid -> (normalize) -> patchify -> tower -> merger.  Returns (grids,
    hidden, merged).  Always the Conv3d definition (no fold)."""
    if normalize_pixels:
        images = [normalize(im) for im in images]
    grids = []
    for img in images:
        f, _, h, w = img.shape
        hh, ww, g = grid_thw(h, w, f, min_pixels=min_pixels, max_pixels=max_pixels)
        if (hh, ww) != (h, w):
            raise ValueError("image sides must already be multiples of 28 inside the budget")
        grids.append(g)
    x = patchify(images, grids)
    z = vision_forward(x, params, grids, depth, heads, eps, theta, dtype, window=window, full_blocks=full_blocks)
    return grids, z, patch_merge(z, params, eps=eps, dtype=dtype)
