"""Edge cases of the HIP path against the CPU oracle: the smallest grid
(one merge group), more images than one launch's metadata chunk, more
windows than one plan chunk, and a video whose frame count is odd."""
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


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def rel_l2(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.linalg.norm(got - ref) / np.linalg.norm(ref))


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    _qv().lib()


def _check(images, depth, dtype, window=0, full=(), seed=0, **grid_kw):
    qv = _qv()
    wl = synth.small_workload("edge", images, depth=depth, dtype=dtype, seed=seed)
    params, imgs = synth.params(wl), synth.pixels(wl)
    enc = qv.Encoder(params, imgs, depth=depth, out_dim=1536, dtype=dtype, window=window, full_blocks=full,
                     **grid_kw)
    enc.run()
    torch.cuda.synchronize()
    grids = [O.grid_thw(h, w, f, **grid_kw)[2] for h, w, f in images]
    assert enc.grids == [tuple(g) for g in grids]
    x = O.patchify(imgs, grids)
    z = O.vision_forward(x, params, grids, depth, window=window, full_blocks=full)
    out = O.patch_merge(z, params)
    e_z = rel_l2(enc.hidden.float().cpu().numpy(), z)
    e_o = rel_l2(enc.out.float().cpu().numpy(), out)
    _say(f"  {len(images)} image(s) grids[:3]={grids[:3]} {dtype} window={window}: "
         f"hidden rel-L2 {e_z:.3e} merged {e_o:.3e}")
    assert e_z <= TOL[dtype] and e_o <= TOL[dtype]
    return enc


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_smallest_grid_one_merge_group(dtype):
    """28x28 pixels with the pixel floor lowered to 784: grid (1, 2, 2), four
    patches, one merged token, alone and packed with a larger image."""
    enc = _check([(28, 28, 1)], 2, dtype, min_pixels=784)
    assert enc.out.shape == (1, 1536)
    _check([(28, 28, 1), (56, 84, 1), (28, 28, 1)], 1, dtype, min_pixels=784)


def test_more_images_than_one_metadata_chunk():
    """40 images (metadata and patch-gather launches take 16 or 32 images
    each): every chunk boundary inside the batch."""
    rng = np.random.default_rng(5)
    sides = [(28 * int(a), 28 * int(b)) for a, b in rng.integers(2, 6, size=(40, 2))]
    _check([(h, w, 1) for h, w in sides], 1, "bf16")


def test_more_windows_than_one_plan_chunk():
    """448x448 with 2x2-patch windows: 256 windows (plan uploads take 128)."""
    _check([(448, 448, 1)], 1, "bf16", window=2)


def test_odd_frame_count_video_repeats_last_frame():
    """5 frames: T = 3 temporal patches, the last one pairing frame 4 with
    itself."""
    _check([(56, 84, 5)], 2, "bf16")


def test_inconsistent_cu_seqlens_is_harmless_and_flagged():
    """The kernels take each image's rows from the host grid list: a device
    cu_seqlens that disagrees with it (every entry inside the buffer, only
    the boundaries wrong) leaves the output bit for bit unchanged, and the
    debug validation reports it as QV_ERR_SHAPE."""
    import os
    qv = _qv()
    from resolution_vit_vision_amd import _abi
    images = [(84, 140, 1), (56, 56, 1), (112, 84, 1)]
    wl = synth.small_workload("cu", images, depth=1)
    enc = qv.Encoder(synth.params(wl), synth.pixels(wl), depth=1, out_dim=1536)
    enc.run()
    torch.cuda.synchronize()
    h1 = enc.hidden.clone()
    good = enc.cu.clone()
    wrong = torch.tensor([0, 4, 8, int(good[-1])], dtype=good.dtype, device=good.device)
    enc.cu.copy_(wrong)
    enc.run()
    torch.cuda.synchronize()
    assert torch.equal(h1, enc.hidden)
    os.environ["QV_DEBUG_VALIDATE"] = "1"
    try:
        with pytest.raises(_abi.QvError) as ei:
            enc.run()
        assert ei.value.status == _abi.QV_ERR_SHAPE
    finally:
        del os.environ["QV_DEBUG_VALIDATE"]
        enc.cu.copy_(good)
        torch.cuda.synchronize()


def test_long_attention_overflow_redoes_with_running_max():
    """The long-sequence attention kernel first keeps the softmax reference
    at the first key tile's maximum; a score above it by more than the float
    exponent range turns its accumulators to inf, and the workgroup must
    redo its rows with the running maximum.  One patch of a 64x64 grid
    (4096 patches, past the first key tile) carries a spike that LayerNorm
    turns into a huge key component, and head 0's query bias makes its score
    up to about 370 (log2 units, times the cosine of the rotary offset
    between the two rows) while first-tile scores stay below about 30: the
    head-0 rows near that patch's row of the grid overflow and attend to it
    alone.  The block's update (output minus input) must match the
    oracle's."""
    qv = _qv()
    from resolution_vit_vision_amd.encoder import VisionConfig, VisionWeights
    rng = np.random.default_rng(41)
    d, m, n = 1280, 5120, 4096
    grids = [(1, 64, 64)]
    cu, pos, _ = O.seq_meta(grids)
    bf = lambda a: synth.round_bf16(np.asarray(a, dtype=np.float32)).astype(np.float64)
    x = bf(rng.standard_normal((n, 1176)))
    x[100, 0] = 2000.0                              # the spiked patch (row 100: past keys 0..31)
    pw = np.zeros((d, 3, 2, 14, 14))
    pw.reshape(d, 1176)[np.arange(1176), np.arange(1176)] = 1.0
    p = {"patch_w": pw}
    blk = {"ln1_w": np.ones(d), "ln1_b": np.zeros(d),
           "qkv_w": np.zeros((3 * d, d)), "qkv_b": np.zeros(3 * d),
           "proj_w": bf(0.02 * rng.standard_normal((d, d))), "proj_b": bf(0.02 * rng.standard_normal(d)),
           "ln2_w": np.ones(d), "ln2_b": np.zeros(d),
           "fc1_w": bf(0.02 * rng.standard_normal((m, d))), "fc1_b": bf(0.02 * rng.standard_normal(m)),
           "fc2_w": bf(0.02 * rng.standard_normal((d, m))), "fc2_b": bf(0.02 * rng.standard_normal(d))}
    blk["qkv_b"][0] = 64.0                          # head 0, q element 0
    blk["qkv_w"][d + 0, 0] = 1.0                    # head 0, k element 0 reads LN1(z)[0]
    blk["qkv_w"][2 * d:] = bf(0.02 * rng.standard_normal((d, d)))
    for k, v in blk.items():
        p["blocks.0." + k] = v
    cfg = VisionConfig(depth=1, patch_dim=1176, ld=1176)
    w = VisionWeights(p, 1, "bf16")
    patches = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).cuda()
    cu_d = torch.from_numpy(cu.astype(np.int32)).cuda()
    _say("long attention overflow: 64x64 grid, one spiked key, depth 1")
    hid = qv.vision_forward(cfg, w, patches, grids, cu_d)
    torch.cuda.synchronize()
    got = hid.cpu().double().numpy()
    assert np.isfinite(got).all()
    z = x @ pw.reshape(d, 1176).T                  # exact on the GPU too (identity weight, bf16 patches)
    ref = O.vision_block(z, O.block_params(p, 0), cu, O.rope_angles(pos))
    # the block's own contribution: the residual stream would hide it
    e = rel_l2(got - z, ref - z)
    _say(f"  block update rel-L2 {e:.3e}")
    assert e <= 2e-2


def test_long_attention_key_loop_tails():
    """The long-sequence attention kernel runs its key loop in whole-tile
    steady steps while the next tile is whole and three tiles ahead exist,
    then finishes with the general step (mask on the last tile).  Seven packed
    images of 2080-2200 patches (enough 128-row query tiles to take that
    kernel) give every remainder of the key-tile count modulo the unroll of
    4 and last tiles of 4, 16, 20 and 24 keys as well as whole ones; each image's
    loop ends on its own tail.  The block's update (output minus input) must
    match the oracle's."""
    qv = _qv()
    shapes = [(46, 46), (42, 50), (40, 52), (16, 134), (48, 44), (44, 50), (40, 54)]   # patches per side
    images = [(14 * a, 14 * b, 1) for a, b in shapes]
    ns = [a * b for a, b in shapes]
    tiles = [(n + 31) // 32 for n in ns]
    assert {t % 4 for t in tiles} == {0, 1, 2, 3}
    assert {n % 32 for n in ns} >= {0, 4, 16, 20, 24}
    wl = synth.small_workload("tails", images, depth=1)
    params, imgs = synth.params(wl), synth.pixels(wl)
    grids = [O.grid_thw(h, w, f)[2] for h, w, f in images]
    _say(f"long attention tails: n={ns} key tiles={tiles}")
    enc0 = qv.Encoder(params, imgs, depth=0, out_dim=1536)
    enc0.run()
    enc1 = qv.Encoder(params, imgs, depth=1, out_dim=1536)
    enc1.run()
    torch.cuda.synchronize()
    assert enc1.grids == [tuple(g) for g in grids]
    x = O.patchify(imgs, grids)
    z0 = O.vision_forward(x, params, grids, 0)
    z1 = O.vision_forward(x, params, grids, 1)
    g0 = enc0.hidden.float().cpu().numpy().astype(np.float64)
    g1 = enc1.hidden.float().cpu().numpy().astype(np.float64)
    cu = np.concatenate([[0], np.cumsum(ns)])
    for i in range(len(ns)):
        a, b = cu[i], cu[i + 1]
        e = rel_l2(g1[a:b] - g0[a:b], z1[a:b] - z0[a:b])
        _say(f"  image {i}: n={ns[i]} tiles={tiles[i]} block update rel-L2 {e:.3e}")
        assert e <= 2e-2
