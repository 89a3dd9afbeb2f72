"""The PatchMerger alone on MI355X (qv_patch_merge through the C ABI) against
the CPU oracle, over token counts that take each of its paths: at small M
the two Linears split K into runs whose float32 partial sums one reduction
adds in a fixed order (fc1: 128x160 tiles; fc2: 128x128 tiles for N = 1536
and 3584), at larger M they run unsplit.  bf16 bar: relative L2 over the
whole tensor, accumulated in float64, <= 2e-2."""
import sys

import numpy as np
import pytest
import torch

import synth
from oracle import qv_oracle as O

pytestmark = pytest.mark.gpu

TOL = 2e-2


def _qv():
    import resolution_vit_vision_amd as qv
    return qv


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    _qv().lib()


CASES = [
    # merged rows M, decoder width: which products split (runs)
    (16, 1536),    # fc1 4, fc2 8
    (16, 3584),    # fc1 4, fc2 8
    (77, 1536),    # ragged single tile
    (256, 1536),   # 448x448: fc1 4, fc2 8
    (256, 3584),   # fc1 4, fc2 4
    (601, 3584),   # both unsplit, ragged last tile
    (1024, 1536),  # fc1 unsplit, fc2 2
]


@pytest.mark.parametrize("m,out_dim", CASES, ids=[f"M{m}_D{d}" for m, d in CASES])
def test_merger_vs_oracle(m, out_dim):
    qv = _qv()
    print(f"merger M={m} out_dim={out_dim}", flush=True)
    sys.stdout.flush()
    wl = synth.small_workload("merge", [(56, 56, 1)], depth=0, dtype="bf16", out_dim=out_dim)
    params = synth.params(wl)
    rng = np.random.default_rng(m * 7 + out_dim)
    z = rng.standard_normal((4 * m, 1280)).astype(np.float32)
    cfg = qv.MergerConfig(dim=1280, out_dim=out_dim, dtype="bf16")
    w = qv.MergerWeights(params, "bf16")
    hidden = torch.from_numpy(z).cuda()
    out = qv.patch_merge(cfg, w, hidden)
    torch.cuda.synchronize()
    ref = O.patch_merge(z.astype(np.float64), params)
    got = out.float().cpu().numpy().astype(np.float64)
    e = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
    print(f"  rel-L2 {e:.3e}", flush=True)
    assert got.shape == (m, out_dim)
    assert e <= TOL
    # the split partial sums are added in a fixed order: a second call agrees bit for bit
    out2 = qv.patch_merge(cfg, w, hidden)
    torch.cuda.synchronize()
    assert torch.equal(out, out2)
