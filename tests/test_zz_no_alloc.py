"""qv_vision_forward_noalloc (static device workspace, no allocation) against
qv_vision_forward (caller's workspace) through the C ABI: two calls in a
row, the second on a smaller batch, each bit for bit equal to the existing
entry point on the same inputs; a batch whose workspace exceeds the static
array is refused before anything is launched."""
import ctypes
import sys

import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import resolution_vit_vision_amd as qv
    qv.lib()


def _pair(images, depth, window=0, full_blocks=(), weights="dtype"):
    """(existing entry point's hidden, no-alloc entry point's hidden) for one
    batch, same weights, patches and stream."""
    import resolution_vit_vision_amd as qv
    wl = synth.small_workload("na", images, depth=depth)
    enc = qv.Encoder(synth.params(wl), synth.pixels(wl), depth=depth, out_dim=1536, window=window,
                     full_blocks=full_blocks, fold=True, weights=weights)
    enc.run()
    torch.cuda.synchronize()
    ref = enc.hidden.clone()
    got = torch.full_like(enc.hidden, float("nan"))
    qv.vision_forward_noalloc(enc.vcfg, enc.vw, enc.patches, enc.grids, enc.cu, got)
    torch.cuda.synchronize()
    return enc, ref, got


def test_noalloc_matches_workspace_forward_twice():
    import resolution_vit_vision_amd as qv
    # first call: one 448x448 image, 4 blocks (32.5 MiB of workspace at full depth)
    _say("no-alloc call 1: 448x448, 4 blocks")
    enc, ref, got = _pair([(448, 448, 1)], depth=4)
    from resolution_vit_vision_amd import _abi
    assert qv.vision_workspace_size(enc.vcfg, enc.grids) <= _abi.QV_SCRATCH_BYTES
    assert torch.equal(ref, got), float((ref - got).abs().max())
    # second call, smaller: two ragged images whose padded attention rows need
    # the zero fill again (the array still holds the first call's data)
    _say("no-alloc call 2: 84x140 + 56x56, 2 blocks")
    enc2, ref2, got2 = _pair([(84, 140, 1), (56, 56, 1)], depth=2)
    assert torch.equal(ref2, got2), float((ref2 - got2).abs().max())
    # and the first shape again after the smaller one
    got3 = torch.full_like(enc.hidden, float("nan"))
    qv.vision_forward_noalloc(enc.vcfg, enc.vw, enc.patches, enc.grids, enc.cu, got3)
    torch.cuda.synchronize()
    assert torch.equal(ref, got3)


def test_noalloc_windowed_and_int8():
    _say("no-alloc: windowed 8x8-patch windows, int8 block matrices")
    _, ref, got = _pair([(224, 336, 1)], depth=2, window=8, full_blocks=(1,), weights="int8")
    assert torch.equal(ref, got)


def test_noalloc_refuses_batches_beyond_the_scratch():
    import resolution_vit_vision_amd as qv
    from resolution_vit_vision_amd import _abi
    from resolution_vit_vision_amd.encoder import VisionConfig
    grids = [(1, 48, 48)] * 4                  # four 672x672 images: ~203 MiB of workspace
    cfg = VisionConfig(depth=1, patch_dim=592, ld=592)
    assert qv.vision_workspace_size(cfg, grids) > _abi.QV_SCRATCH_BYTES
    g = np.asarray(grids, np.int32)
    c = cfg.c()
    blocks = (_abi.BlockW * 1)(_abi.BlockW(*([0x2000] * 12 + [0] * 4)))
    w = _abi.VisionW(0x3000, None, blocks)
    fake = ctypes.c_void_p(0x1000)             # never used: the call fails before any launch
    st = qv.lib().qv_vision_forward_noalloc(ctypes.byref(c), ctypes.byref(w), fake, g.ctypes.data, len(g), fake,
                                            fake, None)
    assert st == _abi.QV_ERR_WORKSPACE
    assert b"static scratch" in qv.lib().qv_last_error()
