"""Parity of the HIP path (through the C ABI) with the CPU oracle on MI355X.

Integers and the patch matrix are compared bit for bit; floating-point
outputs by relative L2 error over the whole tensor, accumulated in float64:
<= 2e-2 for the bf16 path and <= 1e-4 for the float32 path.  Small cases,
the 448x448 image and the four packed 672x672 images run the oracle end to
end over whole tensors; the larger workloads check patchify exactly, then
nine blocks spread over the depth teacher-forced (the oracle block fed the
GPU's own input) on rows covering every 128-row query tile, and the merger
on the groups of those rows."""
import sys

import numpy as np
import pytest
import torch

import synth
from oracle import qv_oracle as O

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-2, "f32": 1e-4}


def _qv():
    import resolution_vit_vision_amd as qv
    return qv


def rel_l2(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.linalg.norm(got - ref) / np.linalg.norm(ref))


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    _qv().lib()


def _host(t):
    return t.float().cpu().numpy()


# --------------------------------------------------------------- patchify
PATCH_CASES = [
    ("one_4x4", [(56, 56, 1)]),
    ("ragged_3", [(84, 140, 1), (56, 56, 1), (224, 112, 1)]),
    ("video_frames", [(56, 84, 2), (56, 56, 3)]),
]


@pytest.mark.parametrize("name,images", PATCH_CASES, ids=[c[0] for c in PATCH_CASES])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_patchify_bit_exact(name, images, dtype):
    qv = _qv()
    wl = synth.small_workload(name, images)
    imgs = synth.pixels(wl)
    grids = [O.grid_thw(h, w, f)[2] for h, w, f in images]
    flat, descs = qv.pack_images(imgs)
    _say(f"patchify {name} {dtype} grids={grids}")
    px = torch.from_numpy(flat).cuda()
    got = qv.patchify(px, descs, grids, dtype)
    torch.cuda.synchronize()
    ref = O.patchify(imgs, grids)
    if dtype == "bf16":
        assert np.array_equal(got.view(torch.int16).cpu().numpy().view(np.uint16), O.bf16_round(ref))
    else:
        assert np.array_equal(got.cpu().numpy(), ref.astype(np.float32))


def test_patchify_padded_row_stride_leaves_pad_untouched():
    qv = _qv()
    imgs = synth.pixels(synth.small_workload("p", [(56, 84, 1)]))
    grids = [(1, 4, 6)]
    flat, descs = qv.pack_images(imgs)
    out = torch.full((24, 1184), 7.0, dtype=torch.bfloat16, device="cuda")
    qv.patchify(torch.from_numpy(flat).cuda(), descs, grids, "bf16", ld=1184, out=out)
    torch.cuda.synchronize()
    h = out.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(h[:, :1176], O.bf16_round(O.patchify(imgs, grids)))
    assert (out[:, 1176:].float().cpu().numpy() == 7.0).all()


# --------------------------------------------------------- small end to end
def _encode_case(images, depth, dtype, out_dim=1536, grids=None, seed=0):
    qv = _qv()
    wl = synth.small_workload("case", images, depth=depth, dtype=dtype, out_dim=out_dim, seed=seed)
    params = synth.params(wl)
    imgs = synth.pixels(wl)
    enc = qv.Encoder(params, imgs, depth=depth, out_dim=out_dim, dtype=dtype, grids=grids)
    enc.run()
    torch.cuda.synchronize()
    return wl, params, imgs, enc


def _oracle_encode(imgs, params, grids, depth):
    x = O.patchify(imgs, grids)
    z = O.vision_forward(x, params, grids, depth)
    return z, O.patch_merge(z, params)


SMALL = [
    # name, images (H, W, F), depth, dtype
    ("toy112_fp32", [(112, 112, 1)], 2, "f32"),
    ("ragged3_fp32", [(84, 140, 1), (56, 56, 1), (224, 252, 1)], 1, "f32"),
    ("ragged3_bf16", [(84, 140, 1), (56, 56, 1), (224, 252, 1)], 2, "bf16"),
    ("tiles_bf16", [(252, 364, 1), (112, 56, 1)], 2, "bf16"),
    # M = 1088: fc2 splits K in two runs (bf16 partial sums), ragged last row tile
    ("pair1088_bf16", [(448, 448, 1), (112, 112, 1)], 2, "bf16"),
    ("video_bf16", [(84, 112, 3)], 1, "bf16"),
]


@pytest.mark.parametrize("name,images,depth,dtype", SMALL, ids=[c[0] for c in SMALL])
def test_encoder_small_vs_oracle(name, images, depth, dtype):
    grids = [O.grid_thw(h, w, f)[2] for h, w, f in images]
    _say(f"encoder {name}: grids={grids} depth={depth} {dtype}")
    wl, params, imgs, enc = _encode_case(images, depth, dtype)
    assert enc.grids == [tuple(g) for g in grids]
    cu, _, _ = O.seq_meta(grids)
    assert np.array_equal(enc.cu.cpu().numpy(), cu)
    z, out = _oracle_encode(imgs, params, grids, depth)
    e_z = rel_l2(_host(enc.hidden), z)
    e_o = rel_l2(_host(enc.out), out)
    _say(f"  hidden rel-L2 {e_z:.3e}  merged rel-L2 {e_o:.3e}")
    assert e_z <= TOL[dtype] and e_o <= TOL[dtype]
    # each image's rows on their own (the block-diagonal mask has no leaks)
    for i in range(len(grids)):
        a, b = cu[i], cu[i + 1]
        assert rel_l2(_host(enc.hidden)[a:b], z[a:b]) <= TOL[dtype]


def test_patch_embed_only_depth0():
    for dtype in ("f32", "bf16"):
        images = [(84, 140, 1), (56, 56, 1)]
        grids = [O.grid_thw(h, w, f)[2] for h, w, f in images]
        wl, params, imgs, enc = _encode_case(images, 0, dtype)
        z = O.patch_embed(O.patchify(imgs, grids).astype(np.float64), params["patch_w"].astype(np.float64))
        assert rel_l2(_host(enc.hidden), z) <= TOL[dtype]


def test_packed_equals_separate_bitwise():
    """Packed varlen run == each image run alone, bit for bit (no cross-image
    leak; no dependence of a row's arithmetic on its neighbours)."""
    qv = _qv()
    images = [(84, 140, 1), (56, 56, 1), (252, 140, 1)]
    wl = synth.small_workload("pk", images, depth=2)
    params = synth.params(wl)
    imgs = synth.pixels(wl)
    packed = qv.Encoder(params, imgs, depth=2, out_dim=1536)
    packed.run()
    torch.cuda.synchronize()
    hp, op = packed.hidden.cpu(), packed.out.cpu()
    for i, im in enumerate(imgs):
        one = qv.Encoder(params, [im], depth=2, out_dim=1536)
        one.run()
        torch.cuda.synchronize()
        a, b = int(packed.cu_host[i]), int(packed.cu_host[i + 1])
        assert torch.equal(one.hidden.cpu(), hp[a:b])
        assert torch.equal(one.out.cpu(), op[a // 4:b // 4])


def test_deterministic_bitwise():
    qv = _qv()
    images = [(252, 364, 1), (84, 56, 1)]
    wl = synth.small_workload("det", images, depth=2)
    enc = qv.Encoder(synth.params(wl), synth.pixels(wl), depth=2, out_dim=1536)
    enc.run()
    torch.cuda.synchronize()
    h1, o1 = enc.hidden.clone(), enc.out.clone()
    enc.run()
    torch.cuda.synchronize()
    assert torch.equal(h1, enc.hidden) and torch.equal(o1, enc.out)


# ------------------------------------------------------- full-size workloads
@pytest.mark.parametrize("fold", [False, True], ids=["conv3d", "conv2d_fold"])
def test_full_448_end_to_end(fold):
    """One 448x448 image through all 32 blocks and the merger, oracle end to
    end (the oracle always takes the Conv3d definition)."""
    qv = _qv()
    wl = synth.W448
    _say(f"{wl.name} fold={fold}: drawing params")
    params = synth.params(wl)
    imgs = synth.pixels(wl)
    enc = qv.Encoder(params, imgs, depth=wl.depth, out_dim=wl.out_dim, dtype=wl.dtype, fold=fold)
    enc.run()
    torch.cuda.synchronize()
    grids = [O.grid_thw(h, w, f)[2] for h, w, f in wl.images]
    assert enc.grids == [(1, 32, 32)]
    _say(f"{wl.name}: oracle (float64, 32 blocks)")
    z, out = _oracle_encode(imgs, params, grids, wl.depth)
    e_z, e_o = rel_l2(_host(enc.hidden), z), rel_l2(_host(enc.out), out)
    _say(f"  hidden rel-L2 {e_z:.3e}  merged rel-L2 {e_o:.3e}")
    assert out.shape == (256, 1536) and enc.out.shape == (256, 1536)
    assert e_z <= wl.tol and e_o <= wl.tol


# the float64 oracle over 9216 patches and 32 blocks takes 1.5 to 3 minutes
# of host time, so this test gets a longer limit than the per-test default
@pytest.mark.timeout(480)
def test_full_672x4_end_to_end():
    """Four 672x672 images packed varlen (cu_seqlens 0, 2304, ..., 9216)
    through all 32 blocks and the merger in the benchmark's launch
    configuration (Conv2d fold), compared with the oracle's whole encoder
    (float64, Conv3d definition) over the whole hidden and merged tensors,
    and image by image."""
    qv = _qv()
    wl = synth.W672X4
    _say(f"{wl.name}: drawing params")
    params = synth.params(wl)
    imgs = synth.pixels(wl)
    enc = qv.Encoder(params, imgs, depth=wl.depth, out_dim=wl.out_dim, dtype=wl.dtype, fold=True)
    enc.run()
    torch.cuda.synchronize()
    grids = [O.grid_thw(h, w, f)[2] for h, w, f in wl.images]
    assert enc.grids == [(1, 48, 48)] * 4
    _say(f"{wl.name}: oracle (float64, 32 blocks, 9216 patches)")
    z, out = _oracle_encode(imgs, params, grids, wl.depth)
    hid, mo = _host(enc.hidden), _host(enc.out)
    e_z, e_o = rel_l2(hid, z), rel_l2(mo, out)
    _say(f"  hidden rel-L2 {e_z:.3e}  merged rel-L2 {e_o:.3e}")
    assert out.shape == (2304, 1536) and mo.shape == (2304, 1536)
    assert e_z <= wl.tol and e_o <= wl.tol
    for i in range(4):
        a, b = 2304 * i, 2304 * (i + 1)
        ei = rel_l2(hid[a:b], z[a:b])
        _say(f"  image {i}: hidden rel-L2 {ei:.3e}")
        assert ei <= wl.tol and rel_l2(mo[a // 4:b // 4], out[a // 4:b // 4]) <= wl.tol


def _band_rows(cu, rng, band=128, per_image=64):
    """Rows to check: in every image, one random row from each band of 128
    rows (the attention kernels' query tiles), the first and last rows, and
    further random rows up to `per_image`."""
    rows = []
    for i in range(len(cu) - 1):
        a, b = int(cu[i]), int(cu[i + 1])
        mine = {a, b - 1}
        for lo in range(a, b, band):
            mine.add(int(rng.integers(lo, min(lo + band, b))))
        extra = max(0, min(per_image, b - a) - len(mine))
        rest = np.setdiff1d(np.arange(a, b), np.fromiter(mine, dtype=np.int64))
        mine.update(int(x) for x in rng.choice(rest, size=extra, replace=False))
        rows += sorted(mine)
    return np.unique(np.asarray(rows))


# blocks teacher-forced at full size: spread over the depth, including the
# Qwen2.5-VL full-attention blocks 7/15/23/31 of the windowed workload
DEEP_BLOCKS = (0, 4, 7, 11, 15, 19, 23, 27, 31)
LIGHT_BLOCKS = (0, 7, 15, 23, 31)

FULL = [(n, "dtype", DEEP_BLOCKS) for n in ("qwen2vl_2b_672x4_varlen", "mixed16_varlen_7b_merger", "maxres_3584",
                                             "qwen25vl_7b_3584_window")]
FULL += [("video_448_16f", "dtype", LIGHT_BLOCKS)]
# int8 block matrices at full size (bench --weights int8): the blocks are
# checked against the oracle on the dequantized weights
FULL += [("qwen2vl_2b_672x4_varlen", "int8", LIGHT_BLOCKS), ("qwen25vl_7b_3584_window", "int8", LIGHT_BLOCKS)]


@pytest.mark.parametrize("name,weights,blocks", FULL, ids=[n if w == "dtype" else f"{n}-int8" for n, w, _ in FULL])
def test_full_size_sampled(name, weights, blocks):
    """Full-size workload in the benchmark's launch configuration (still
    images take the Conv2d fold there): exact patchify and metadata; blocks
    spread over the depth teacher-forced (the oracle block fed the GPU's own
    input) on rows that cover every 128-row query tile of every image (at
    least 64 rows per image; 512+ at 3584x3584); merger on the groups of
    those rows."""
    qv = _qv()
    wl = synth.WORKLOADS[name]
    _say(f"{name} weights={weights}: drawing inputs")
    params = synth.params(wl)
    imgs = synth.pixels(wl)
    grids = [O.grid_thw(h, w, f)[2] for h, w, f in wl.images]
    fold = all(f == 1 for _, _, f in wl.images)
    enc = qv.Encoder(params, imgs, depth=wl.depth, out_dim=wl.out_dim, dtype=wl.dtype, window=wl.window,
                     full_blocks=wl.full_blocks, fold=fold, weights=weights)
    block_ref = O.dequantized_params(params, wl.depth) if weights == "int8" else params
    assert enc.grids == [tuple(g) for g in grids]
    cu, pos, _ = O.seq_meta(grids)
    windows = O.window_groups(grids, wl.window) if wl.window else None
    assert np.array_equal(enc.cu_host, cu)
    rng = np.random.default_rng(7)
    enc.run()
    torch.cuda.synchronize()
    # patch matrix: bit-exact against the oracle's gather + RNE cast
    x_ref = O.patchify_folded(imgs, grids, width=592) if fold else O.patchify(imgs, grids)
    assert np.array_equal(enc.patches.view(torch.int16).cpu().numpy().view(np.uint16), O.bf16_round(x_ref))
    del x_ref
    out_full = _host(enc.out)
    hid_full = _host(enc.hidden)
    angles = O.rope_angles(pos)
    rows = _band_rows(cu, rng)
    for i in range(len(cu) - 1):
        assert ((rows >= cu[i]) & (rows < cu[i + 1])).sum() >= min(64, cu[i + 1] - cu[i])
    errs = {}
    for l in blocks:
        z_in = _host(qv.vision_forward(enc.vcfg.__class__(**{**enc.vcfg.__dict__, "depth": l}), enc.vw,
                                       enc.patches, enc.grids, enc.cu, ws=enc.ws)).astype(np.float64)
        z_out = _host(qv.vision_forward(enc.vcfg.__class__(**{**enc.vcfg.__dict__, "depth": l + 1}), enc.vw,
                                        enc.patches, enc.grids, enc.cu, ws=enc.ws))
        torch.cuda.synchronize()
        groups = windows if (windows is not None and l not in wl.full_blocks) else None
        ref = O.vision_block_rows(z_in, O.block_params(block_ref, l), cu, angles, rows, groups=groups)
        e = rel_l2(z_out[rows], ref)
        errs[l] = e
        _say(f"{name}: block {l} ({'windowed' if groups else 'full'}) teacher-forced on {len(rows)} rows: "
             f"rel-L2 {e:.3e}")
    assert max(errs.values()) <= wl.tol, errs
    groups = np.unique(rows // 4)
    zr = np.concatenate([hid_full[4 * g:4 * g + 4] for g in groups])
    ref = O.patch_merge(zr.astype(np.float64), params)
    e = rel_l2(out_full[groups], ref)
    _say(f"{name}: merger on {len(groups)} groups rel-L2 {e:.3e}")
    assert e <= wl.tol
    assert out_full.shape == (cu[-1] // 4, wl.out_dim)
    assert np.isfinite(out_full).all()
