"""int8 weight-only block matrices on MI355X, through the C ABI, against the
CPU oracle.

Quantization (qv_quantize_i8) is integer work decided in float32: codes and
scales must equal oracle.quantize_i8 bit for bit.  The int8 tower computes
scale[n] * sum_k a[m][k] code[n][k] (bf16 activations, exact codes, float32
sums); it is compared with the oracle
run on the dequantized weights (code * scale in float64) at the bf16 bar
(relative L2 over the whole tensor, accumulated in float64, <= 2e-2), and
must sit clearly closer to that than to the unquantized tower, so the test
sees the quantization."""
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


def _quant_cases():
    rng = np.random.default_rng(11)
    cases = []
    cases.append(("gauss_1280", rng.standard_normal((96, 1280)).astype(np.float32) * 0.02))
    cases.append(("ragged_cols", rng.standard_normal((37, 1000)).astype(np.float32)))
    m = rng.uniform(-1, 1, (20, 300)).astype(np.float32)
    m[3] = 0.0                                   # all-zero row: scale 1, codes 0
    m[4] = 0.0
    m[4, 17] = -5.0                              # one nonzero element: code -127
    m[5] = np.float32(1e-30) * rng.standard_normal(300).astype(np.float32)  # tiny values
    m[6] = np.round(m[6] * 254) / 254            # many values near half-way points
    m[7, :] = np.float32(127.0)                  # all equal: codes 127, scale 1
    m[8] = np.arange(300, dtype=np.float32) - 149.5  # a ramp through zero
    cases.append(("special_rows", m))
    # rows whose codes hit exact .5 ties: max 127 (scale 1), entries k + 0.5
    t = np.tile((np.arange(-126, 127, dtype=np.float32) + 0.5), (4, 1))
    t[:, 0] = 127.0
    cases.append(("ties", t))
    return cases


@pytest.mark.parametrize("name,w", _quant_cases(), ids=[c[0] for c in _quant_cases()])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_quantize_bit_exact(name, w, dtype):
    qv = _qv()
    _say(f"quantize {name} {w.shape} from {dtype}")
    ld = w.shape[1] + 24                         # a row stride wider than the row
    wp = np.zeros((w.shape[0], ld), np.float32)
    wp[:, :w.shape[1]] = w
    t = torch.from_numpy(wp).cuda()
    if dtype == "bf16":
        t = t.to(torch.bfloat16)
    view = t[:, :w.shape[1]]
    q, sc = qv.quantize_i8(view)
    torch.cuda.synchronize()
    src = view.float().cpu().numpy()             # exactly the values the kernel read
    q_ref, sc_ref = O.quantize_i8(src)
    assert np.array_equal(sc.cpu().numpy().view(np.uint32), sc_ref.view(np.uint32))
    assert np.array_equal(q.cpu().numpy(), q_ref)


def _run(params, images_np, depth, out_dim=1536, **kw):
    qv = _qv()
    enc = qv.Encoder(params, images_np, depth=depth, out_dim=out_dim, dtype="bf16", weights="int8", **kw)
    enc.run()
    torch.cuda.synchronize()
    return enc


INT8_SMALL = [
    # name, images (H, W, F), depth, window, full-attention blocks
    ("ragged3", [(84, 140, 1), (56, 56, 1), (224, 252, 1)], 2, 0, ()),     # M = 364: split out-proj / fc2
    ("one_1296", [(504, 504, 1)], 1, 0, ()),                               # M = 1296: unsplit GEMMs
    ("pair_1088", [(448, 448, 1), (112, 112, 1)], 2, 0, ()),               # M = 1088, ragged last tile
    ("window8", [(224, 252, 1), (84, 140, 1)], 2, 8, (1,)),                # windowed q/k/v layout
    ("video3", [(84, 112, 3)], 2, 0, ()),                                  # T = 2 frames
]


@pytest.mark.parametrize("name,images,depth,window,full", INT8_SMALL, ids=[c[0] for c in INT8_SMALL])
def test_int8_encoder_vs_oracle(name, images, depth, window, full):
    grids = [O.grid_thw(h, w, f)[2] for h, w, f in images]
    _say(f"int8 {name}: grids={grids} depth={depth} window={window} full={full}")
    wl = synth.small_workload(name, images, depth=depth, dtype="bf16")
    params, imgs = synth.params(wl), synth.pixels(wl)
    enc = _run(params, imgs, depth, window=window, full_blocks=full)
    x = O.patchify(imgs, grids)
    pq = O.dequantized_params(params, depth)
    z = O.vision_forward(x, pq, grids, depth, window=window, full_blocks=full)
    out = O.patch_merge(z, pq)
    e_z = rel_l2(enc.hidden.cpu().numpy(), z)
    e_o = rel_l2(enc.out.float().cpu().numpy(), out)
    z_f = O.vision_forward(x, params, grids, depth, window=window, full_blocks=full)
    e_f = rel_l2(enc.hidden.cpu().numpy(), z_f)
    _say(f"  hidden rel-L2 {e_z:.3e}  merged rel-L2 {e_o:.3e}  (vs unquantized weights {e_f:.3e})")
    assert e_z <= TOL and e_o <= TOL
    assert e_f > 2 * e_z


INT8_WIDE = [
    # M = 4096: fc1 and q/k/v have enough 256 x 256 tiles for the
    # widened-codes path, the out-projection and fc2 stay on the int8 kernel;
    # M = 13392: all four widened, ragged last tile
    ("mixed_4096", [(448, 448, 1)] * 4),
    ("wide_13392", [(448, 448, 1)] * 13 + [(112, 140, 1)]),
]


@pytest.mark.parametrize("name,images", INT8_WIDE, ids=[c[0] for c in INT8_WIDE])
def test_int8_large_m_vs_oracle(name, images):
    grids = [O.grid_thw(h, w, f)[2] for h, w, f in images]
    _say(f"int8 {name}: {len(images)} images, M = {sum(t * h * w for t, h, w in grids)}, depth 1")
    wl = synth.small_workload(name, images, depth=1, dtype="bf16")
    params, imgs = synth.params(wl), synth.pixels(wl)
    enc = _run(params, imgs, 1)
    pq = O.dequantized_params(params, 1)
    z = O.vision_forward(O.patchify(imgs, grids), pq, grids, 1)
    out = O.patch_merge(z, pq)
    e_z = rel_l2(enc.hidden.cpu().numpy(), z)
    e_o = rel_l2(enc.out.float().cpu().numpy(), out)
    _say(f"  hidden rel-L2 {e_z:.3e}  merged rel-L2 {e_o:.3e}")
    assert e_z <= TOL and e_o <= TOL


def test_int8_codes_on_device_match_oracle():
    """The encoder's device-side codes and scales for every block matrix are
    the oracle's, bit for bit."""
    wl = synth.small_workload("codes", [(56, 56, 1)], depth=2, dtype="bf16")
    params = synth.params(wl)
    enc = _run(params, synth.pixels(wl), 2)
    for l in range(2):
        for k in O.QUANT_KEYS:
            q_ref, sc_ref = O.quantize_i8(params[f"blocks.{l}.{k}"])
            q = enc.vw.tensors[f"blocks.{l}.{k}"].cpu().numpy()
            sc = enc.vw.tensors[f"blocks.{l}.{k[:-2]}_s"].cpu().numpy()
            assert np.array_equal(q, q_ref) and np.array_equal(sc.view(np.uint32), sc_ref.view(np.uint32))


def test_int8_448_end_to_end():
    """448x448 through all 32 blocks with int8 block matrices, then the merger;
    oracle end to end on the dequantized weights."""
    wl = synth.W448
    params, imgs = synth.params(wl), synth.pixels(wl)
    enc = _run(params, imgs, wl.depth, out_dim=wl.out_dim)
    grids = [O.grid_thw(h, w, f)[2] for h, w, f in wl.images]
    _say(f"{wl.name} int8: oracle (float64, 32 blocks)")
    pq = O.dequantized_params(params, wl.depth)
    z = O.vision_forward(O.patchify(imgs, grids), pq, grids, wl.depth)
    out = O.patch_merge(z, pq)
    e_z = rel_l2(enc.hidden.cpu().numpy(), z)
    e_o = rel_l2(enc.out.float().cpu().numpy(), out)
    _say(f"  hidden rel-L2 {e_z:.3e}  merged rel-L2 {e_o:.3e}")
    assert e_z <= wl.tol and e_o <= wl.tol


def test_int8_repeatable_bitwise():
    """Split-K partial sums are reduced in a fixed order: two runs agree bit
    for bit."""
    wl = synth.small_workload("rep", [(224, 252, 1), (56, 84, 1)], depth=2, dtype="bf16")
    params, imgs = synth.params(wl), synth.pixels(wl)
    a = _run(params, imgs, 2)
    h1, o1 = a.hidden.clone(), a.out.clone()
    a.run()
    torch.cuda.synchronize()
    assert torch.equal(h1, a.hidden) and torch.equal(o1, a.out)
