"""The encoder forward under HIP graph capture.

qv_vision_forward and qv_patch_merge allocate nothing, synchronise nothing
and clear memory with a kernel (no hipMemsetAsync), so a caller can capture
a whole forward (patchify, tower, merger) into a graph.  Each replay, with
eager forwards and synchronisations in between, must reproduce the eager
result bit for bit."""
import sys

import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


def _qv():
    import resolution_vit_vision_amd as qv
    return qv


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    _qv().lib()


CASES = [
    # name, images (H, W, F), depth, window, full blocks, int8 weights
    ("ragged_bf16", [(84, 140, 1), (56, 56, 1), (224, 252, 1)], 2, 0, (), False),
    ("window_padded", [(224, 252, 1), (84, 140, 1)], 2, 8, (1,), False),
    ("int8_448", [(448, 448, 1)], 2, 0, (), True),
]


@pytest.mark.parametrize("name,images,depth,window,full,int8", CASES, ids=[c[0] for c in CASES])
def test_graph_replay_bitwise(name, images, depth, window, full, int8):
    qv = _qv()
    print(f"graph {name}", flush=True)
    sys.stdout.flush()
    wl = synth.small_workload(name, images, depth=depth, dtype="bf16")
    params, imgs = synth.params(wl), synth.pixels(wl)
    enc = qv.Encoder(params, imgs, depth=depth, out_dim=1536, dtype="bf16", window=window, full_blocks=full,
                     fold=True, weights="int8" if int8 else "dtype")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        enc.run()  # warm-up on the capture stream's side
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    ref_h, ref_o = enc.hidden.clone(), enc.out.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        enc.run()
    torch.cuda.synchronize()
    for i in range(3):
        enc.hidden.zero_()
        enc.out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(enc.hidden, ref_h) and torch.equal(enc.out, ref_o), f"replay {i}"
        enc.run()  # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(enc.hidden, ref_h) and torch.equal(enc.out, ref_o), f"eager after replay {i}"
