"""Conv3d -> Conv2d fold and CLIP normalisation in the patch gather, on
MI355X through the C ABI, against the CPU oracle.

The patch matrix and the folded weight are compared bit for bit (both sides
do the same float32 operations, then round to nearest even); the encoder
with the fold is compared with the oracle's unfolded Conv3d definition by
relative L2 (<= 2e-2 bf16, <= 1e-4 float32)."""
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


def _bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


IMAGES = [(84, 140, 1), (56, 56, 1), (224, 112, 1)]


@pytest.mark.parametrize("fold", [False, True])
@pytest.mark.parametrize("normalize", [False, True])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_patchify_ex_bit_exact(fold, normalize, dtype):
    qv = _qv()
    wl = synth.small_workload("px", IMAGES)
    imgs = [(0.5 * (im + 1.0)).astype(np.float32) for im in synth.pixels(wl)]  # pixels in [0, 1]
    grids = [O.grid_thw(h, w, f)[2] for h, w, f in IMAGES]
    _say(f"patchify_ex fold={fold} normalize={normalize} {dtype}")
    flat, descs = qv.pack_images(imgs)
    width = qv.patch_width(3, fold)
    out = torch.full((sum(t * a * b for t, a, b in grids), width + 8), 3.0, dtype=qv.encoder.TORCH_DTYPES[dtype],
                     device="cuda")
    qv.patchify(torch.from_numpy(flat).cuda(), descs, grids, dtype, ld=width + 8, out=out, fold=fold,
                normalize=normalize)
    torch.cuda.synchronize()
    src = [O.normalize(im) for im in imgs] if normalize else imgs
    ref = O.patchify_folded(src, grids, width=width) if fold else O.patchify(src, grids)
    assert ref.shape[1] == width
    if dtype == "bf16":
        assert np.array_equal(_bits(out)[:, :width], O.bf16_round(ref))
    else:
        assert np.array_equal(out[:, :width].cpu().numpy(), ref.astype(np.float32))
    assert (out[:, width:].float().cpu().numpy() == 3.0).all()  # columns past the row untouched


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_fold_patch_weight_bit_exact(dtype):
    qv = _qv()
    wl = synth.small_workload("fw", [(56, 56, 1)], depth=0, dtype=dtype)
    w3 = synth.params(wl)["patch_w"]                      # [1280][3][2][14][14], bf16-exact values in bf16
    wd = qv.encoder._dev(w3.reshape(1280, -1), dtype, "cuda", True)
    got = qv.fold_patch_weight(wd)
    torch.cuda.synchronize()
    ref = O.fold_patch_weight(w3.astype(np.float32), width=592)  # float32 sum of the two taps
    assert got.shape == (1280, 592)
    if dtype == "bf16":
        assert np.array_equal(_bits(got), O.bf16_round(ref))
    else:
        assert np.array_equal(got.cpu().numpy(), ref)


FOLD_CASES = [
    ("toy112_fold_norm_fp32", [(112, 112, 1)], 2, "f32", True),
    ("ragged3_fold_bf16", [(84, 140, 1), (56, 56, 1), (224, 252, 1)], 2, "bf16", False),
    ("ragged3_fold_norm_bf16", [(84, 140, 1), (56, 56, 1), (224, 252, 1)], 2, "bf16", True),
]


@pytest.mark.parametrize("name,images,depth,dtype,normalize", FOLD_CASES, ids=[c[0] for c in FOLD_CASES])
def test_folded_encoder_vs_conv3d_oracle(name, images, depth, dtype, normalize):
    """The device path with the folded Conv2d weight against the oracle's
    Conv3d definition over the duplicated frame."""
    qv = _qv()
    wl = synth.small_workload(name, images, depth=depth, dtype=dtype)
    params = synth.params(wl)
    imgs = synth.pixels(wl)
    if normalize:
        imgs = [(0.5 * (im + 1.0)).astype(np.float32) for im in imgs]
    grids = [O.grid_thw(h, w, f)[2] for h, w, f in images]
    _say(f"folded encoder {name}: grids={grids} {dtype} normalize={normalize}")
    enc = qv.Encoder(params, imgs, depth=depth, out_dim=1536, dtype=dtype, fold=True, normalize=normalize)
    assert enc.patches.shape[1] == 592 and enc.vw.tensors["patch_w"].shape == (1280, 592)
    enc.run()
    torch.cuda.synchronize()
    grids_o, z, out = O.encode(imgs, params, depth, normalize_pixels=normalize)
    e_z = rel_l2(enc.hidden.float().cpu().numpy(), z)
    e_o = rel_l2(enc.out.float().cpu().numpy(), out)
    _say(f"  hidden rel-L2 {e_z:.3e}  merged rel-L2 {e_o:.3e}")
    assert e_z <= TOL[dtype] and e_o <= TOL[dtype]
