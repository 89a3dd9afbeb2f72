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
