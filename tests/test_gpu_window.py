"""Windowed attention (Qwen2.5-VL style) on MI355X, through the C ABI, against
the CPU oracle.

Blocks not listed as full-attention blocks attend only inside square
windows of `window` patches per frame, truncated at the right and bottom
edges.  Same bars as the full-attention parity tests: relative L2 over the
whole tensor, accumulated in float64, <= 2e-2 for bf16 and <= 1e-4 for
float32; plus exact structural checks (a change inside one window leaves
every other row of a windowed-only tower bit-identical; packed == separate)."""
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


def _run(params, imgs, depth, dtype, window, full_blocks, out_dim=1536, grids=None):
    qv = _qv()
    enc = qv.Encoder(params, imgs, depth=depth, out_dim=out_dim, dtype=dtype, window=window,
                     full_blocks=full_blocks, grids=grids)
    enc.run()
    torch.cuda.synchronize()
    return enc


WIN_SMALL = [
    # name, images (H, W, F), depth, dtype, window, full-attention blocks
    ("toy112_w4_fp32", [(112, 112, 1)], 2, "f32", 4, (1,)),
    ("ragged3_w4_fp32", [(84, 140, 1), (56, 56, 1), (224, 252, 1)], 2, "f32", 4, ()),
    ("pairs_w2_fp32", [(56, 84, 1), (112, 56, 1)], 1, "f32", 2, ()),
    ("ragged3_w8_bf16", [(84, 140, 1), (56, 56, 1), (224, 252, 1)], 3, "bf16", 8, (1,)),
    ("tiles_w10_bf16", [(252, 364, 1), (112, 56, 1)], 2, "bf16", 10, ()),
    ("tiles_w6_bf16", [(252, 364, 1), (168, 84, 1)], 2, "bf16", 6, (0,)),
    ("video_w4_bf16", [(84, 112, 3)], 2, "bf16", 4, (0,)),
]


@pytest.mark.parametrize("name,images,depth,dtype,window,full", WIN_SMALL, ids=[c[0] for c in WIN_SMALL])
def test_windowed_encoder_small_vs_oracle(name, images, depth, dtype, window, full):
    grids = [O.grid_thw(h, w, f)[2] for h, w, f in images]
    _say(f"windowed {name}: grids={grids} depth={depth} {dtype} window={window} full={full}")
    wl = synth.small_workload(name, images, depth=depth, dtype=dtype)
    params, imgs = synth.params(wl), synth.pixels(wl)
    enc = _run(params, imgs, depth, dtype, window, full)
    x = O.patchify(imgs, grids)
    z = O.vision_forward(x, params, grids, depth, window=window, full_blocks=full)
    out = O.patch_merge(z, params)
    e_z, e_o = rel_l2(_host(enc.hidden), z), rel_l2(_host(enc.out), out)
    # distance to the full-attention tower: the windows must matter at least
    # as much as the rounding does
    z_full = O.vision_forward(x, params, grids, depth)
    e_full = rel_l2(_host(enc.hidden), z_full)
    _say(f"  hidden rel-L2 {e_z:.3e}  merged rel-L2 {e_o:.3e}  (vs full attention {e_full:.3e})")
    assert e_z <= TOL[dtype] and e_o <= TOL[dtype]
    assert e_full > 2 * e_z


def test_windowed_isolation_bitwise():
    """Windowed-only tower (bf16): changing the pixels of one window changes
    that window's rows and leaves every other row bit-identical."""
    images = [(224, 252, 1), (84, 140, 1)]  # grids 16 x 18 and 6 x 10
    wl = synth.small_workload("iso", images, depth=2)
    params, imgs = synth.params(wl), synth.pixels(wl)
    a = _run(params, imgs, 2, "bf16", 8, ())
    imgs2 = [im.copy() for im in imgs]
    # patches (rows 8..15, cols 8..15) of image 0 = window (1, 1)
    imgs2[0][:, :, 8 * 14:16 * 14, 8 * 14:16 * 14] *= -1.0
    b = _run(params, imgs2, 2, "bf16", 8, ())
    ha, hb = a.hidden.cpu().numpy(), b.hidden.cpu().numpy()
    cu, pos, _ = O.seq_meta(a.grids)
    inwin = np.zeros(len(ha), bool)
    rows0 = np.arange(cu[0], cu[1])
    inwin[rows0] = (pos[rows0, 0] // 8 == 1) & (pos[rows0, 1] // 8 == 1)
    assert inwin.sum() == 64
    changed = (ha != hb).any(axis=1)
    assert changed[inwin].all()
    assert not changed[~inwin].any()


def test_windowed_packed_equals_separate_bitwise():
    qv = _qv()
    images = [(84, 140, 1), (56, 56, 1), (252, 140, 1)]
    wl = synth.small_workload("pkw", images, depth=2)
    params, imgs = synth.params(wl), synth.pixels(wl)
    packed = _run(params, imgs, 2, "bf16", 4, (1,))
    hp, op = packed.hidden.cpu(), packed.out.cpu()
    for i, im in enumerate(imgs):
        one = _run(params, [im], 2, "bf16", 4, (1,))
        a, b = int(packed.cu_host[i]), int(packed.cu_host[i + 1])
        assert torch.equal(one.hidden.cpu(), hp[a:b])
        assert torch.equal(one.out.cpu(), op[a // 4:b // 4])
    del qv


def test_window_covering_image_equals_full_attention_bitwise():
    """A window at least as large as every grid puts each frame in one window:
    the windowed tower is the full-attention tower, bit for bit (same
    kernels, same key order inside a window)."""
    images = [(56, 56, 1), (56, 84, 1), (84, 56, 1)]  # grids 4x4, 4x6, 6x4
    wl = synth.small_workload("cover", images, depth=2)
    params, imgs = synth.params(wl), synth.pixels(wl)
    w = _run(params, imgs, 2, "bf16", 10, ())
    f = _run(params, imgs, 2, "bf16", 0, ())
    assert torch.equal(w.hidden.cpu(), f.hidden.cpu()) and torch.equal(w.out.cpu(), f.out.cpu())


def test_windowed_448_end_to_end():
    """448x448 through all 32 blocks with 8x8-patch windows and full attention
    in blocks 7, 15, 23 and 31, then the merger; oracle end to end."""
    wl = synth.W448
    params, imgs = synth.params(wl), synth.pixels(wl)
    full = (7, 15, 23, 31)
    enc = _run(params, imgs, wl.depth, wl.dtype, 8, full, out_dim=wl.out_dim)
    grids = [O.grid_thw(h, w, f)[2] for h, w, f in wl.images]
    _say(f"{wl.name} windowed: oracle (float64, 32 blocks)")
    z = O.vision_forward(O.patchify(imgs, grids), params, grids, wl.depth, window=8, full_blocks=full)
    out = O.patch_merge(z, params)
    e_z, e_o = rel_l2(_host(enc.hidden), z), rel_l2(_host(enc.out), out)
    _say(f"  hidden rel-L2 {e_z:.3e}  merged rel-L2 {e_o:.3e}")
    assert e_z <= wl.tol and e_o <= wl.tol
