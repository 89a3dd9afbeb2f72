"""Pins of the CPU oracle to things other than itself: page-printed values,
closed forms, invariants, brute force on tiny inputs and library routines.

Each test names the oracle function it pins and what a plausible mistake
(dropped term, wrong sign or index, transposed operand) would do to it."""
import math
import os

import numpy as np
import synth
import pytest
import torch
import torch.nn.functional as F

from oracle import qv_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_rows(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as fh:
        for line in fh:
            line = line.split("#", 1)[0].strip()
            if line:
                rows.append(line)
    return rows


# ------------------------------------------------------------------ grid
def test_grid_page_values():
    """smart_resize / grid_thw against the grid and token counts the pages print."""
    for row in _golden_rows("page_grids.txt"):
        lhs, rhs = row.split("->")
        h, w, f = map(int, lhs.split())
        t, gh, gw, n, m = map(int, rhs.split())
        hh, ww, g = O.grid_thw(h, w, f)
        assert (hh, ww) == (h, w)
        assert g == (t, gh, gw)
        assert t * gh * gw == n
        assert hh * ww // 784 == m == n // 4


def _nearest_multiple_even_tie(x, f):
    """Brute force: the multiple of f nearest to x (ties to the even multiple), >= f."""
    best = None
    for k in range(1, x // f + 3):
        d = abs(k * f - x)
        key = (d, k % 2)  # equal distance: prefer even k
        if best is None or key < best[0]:
            best = (key, k * f)
    return best[1]


def test_grid_bruteforce_properties():
    """Every result: sides multiples of 28, tokens in [4, 16384]; in-budget sides
    equal the brute-force nearest multiple; over/under budget sides are the
    largest/smallest multiples of the common rescale."""
    f = 28
    rng = np.random.default_rng(123)
    cases = [(h, w) for h in range(1, 2001, 13) for w in range(1, 2001, 17)]
    cases += [tuple(x) for x in rng.integers(1, 6000, size=(3000, 2))]
    for h, w in cases:
        try:
            hh, ww = O.smart_resize(int(h), int(w))
        except ValueError:
            # only extreme aspect ratios may fail
            assert max(h, w) / min(h, w) > 100
            continue
        assert hh % f == 0 and ww % f == 0
        assert 4 <= hh * ww // 784 <= 16384
        nh, nw = _nearest_multiple_even_tie(int(h), f), _nearest_multiple_even_tie(int(w), f)
        if O.MIN_PIXELS <= nh * nw <= O.MAX_PIXELS:
            assert (hh, ww) == (nh, nw)
        elif nh * nw > O.MAX_PIXELS:
            s = math.sqrt(O.MAX_PIXELS / (h * w))
            assert hh <= max(f, h * s + 1e-9) and (hh == f or hh + f > h * s - 1e-9)
        else:
            s = math.sqrt(O.MIN_PIXELS / (h * w))
            assert hh >= h * s - 1e-9 and hh - f < h * s + 1e-9


def test_grid_idempotent_and_token_formula():
    """Valid sides map to themselves and tokens = pixels / 784 (Qwen2.5-VL record)."""
    for h in range(56, 3585, 28 * 7):
        for w in range(56, 3585, 28 * 5):
            if not (O.MIN_PIXELS <= h * w <= O.MAX_PIXELS):
                continue
            hh, ww, g = O.grid_thw(h, w)
            assert (hh, ww) == (h, w)
            assert g[1] * g[2] // 4 == h * w // 784
    # the round-half-even tie: 70 = 2.5 * 28 goes to 56, 98 = 3.5 * 28 to 112
    assert O.smart_resize(70, 112)[0] == 56
    assert O.smart_resize(98, 112)[0] == 112


def test_grid_frames():
    assert O.grid_thw(56, 56, 1)[2][0] == 1
    assert O.grid_thw(56, 56, 2)[2][0] == 1
    assert O.grid_thw(56, 56, 3)[2][0] == 2


# ------------------------------------------------------- order / positions
def test_merge_order_golden_4x4():
    cu, pos, perm = O.seq_meta([(1, 4, 4)])
    want = np.array([list(map(int, r.split())) for r in _golden_rows("merge_order_4x4.txt")])
    assert (perm == want[:, 1]).all()
    assert (pos == want[:, 2:4]).all()
    assert list(cu) == [0, 16]


def test_seq_meta_bijection_and_cu():
    grids = [(1, 4, 6), (2, 2, 2), (1, 48, 48), (1, 6, 10)]
    cu, pos, perm = O.seq_meta(grids)
    assert list(cu) == [0, 24, 32, 32 + 2304, 32 + 2304 + 60]
    for i, (t, gh, gw) in enumerate(grids):
        p = perm[cu[i]:cu[i + 1]]
        assert sorted(p.tolist()) == list(range(t * gh * gw))
        # (h, w) agrees with the raster index
        assert (pos[cu[i]:cu[i + 1], 0] == (p % (gh * gw)) // gw).all()
        assert (pos[cu[i]:cu[i + 1], 1] == p % gw).all()
    # four 672x672 images: cu_seqlens 0, 2304, ..., 9216 (packed-batch workload)
    cu4, _, _ = O.seq_meta([(1, 48, 48)] * 4)
    assert list(cu4) == [0, 2304, 4608, 6912, 9216]
    with pytest.raises(ValueError):
        O.seq_meta([(1, 3, 4)])


def test_strided_slice_identity():
    """LiteRT-LM card: raster order + four strided slices concatenated equals the
    merge-group order reshaped to [N/4][4C]."""
    rng = np.random.default_rng(0)
    for gh, gw in [(4, 4), (6, 10), (8, 2)]:
        c = 5
        f = rng.standard_normal((gh, gw, c))
        slices = [f[0::2, 0::2], f[0::2, 1::2], f[1::2, 0::2], f[1::2, 1::2]]
        ref = np.concatenate(slices, axis=-1).reshape(-1, 4 * c)
        _, _, perm = O.seq_meta([(1, gh, gw)])
        got = f.reshape(gh * gw, c)[perm].reshape(-1, 4 * c)
        assert np.array_equal(ref, got)


# --------------------------------------------------- patchify / patch-embed
def _conv3d_reference(frames, weight):
    """torch conv3d (CPU, float64) on frames padded to a multiple of 2."""
    fr = frames
    if fr.shape[0] % 2:
        fr = np.concatenate([fr, fr[-1:]], axis=0)
    x = torch.from_numpy(fr.astype(np.float64)).permute(1, 0, 2, 3)[None]  # [1][C][F][H][W]
    y = F.conv3d(x, torch.from_numpy(weight.astype(np.float64)), stride=(2, 14, 14))
    return y[0].permute(1, 2, 3, 0).reshape(-1, weight.shape[0]).numpy()  # raster [T*gh*gw][out]


def test_patch_embed_equals_conv3d():
    rng = np.random.default_rng(1)
    out = 16
    w = rng.standard_normal((out, 3, 2, 14, 14))
    for (h, wd, f) in [(56, 84, 1), (28, 112, 2), (84, 56, 3)]:
        img = rng.uniform(-1, 1, (f, 3, h, wd)).astype(np.float32)
        g = O.grid_thw(h, wd, f)[2]
        x = O.patchify([img], [g])
        got = O.patch_embed(x.astype(np.float64), w)
        _, _, perm = O.seq_meta([g])
        ref = _conv3d_reference(img, w)[perm]
        np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_conv2d_fold_for_still_image():
    """LiteRT-LM card: Conv3d over the duplicated still frame equals Conv2d with
    the summed temporal kernel w[:,:,0] + w[:,:,1]."""
    rng = np.random.default_rng(2)
    w = rng.standard_normal((8, 3, 2, 14, 14))
    img = rng.uniform(-1, 1, (1, 3, 56, 84)).astype(np.float32)
    g = O.grid_thw(56, 84, 1)[2]
    got = O.patch_embed(O.patchify([img], [g]).astype(np.float64), w)
    x2 = torch.from_numpy(img[0].astype(np.float64))[None]
    y = F.conv2d(x2, torch.from_numpy(w[:, :, 0] + w[:, :, 1]), stride=14)[0]
    ref = y.permute(1, 2, 0).reshape(-1, 8).numpy()
    _, _, perm = O.seq_meta([g])
    np.testing.assert_allclose(got, ref[perm], rtol=1e-12, atol=1e-12)


def test_patchify_rejects_off_grid():
    img = np.zeros((1, 3, 56, 57), np.float32)
    with pytest.raises(ValueError):
        O.raster_patches(img, (1, 4, 4))


# ----------------------------------------------------------------- bf16 cast
def test_bf16_round_matches_torch():
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.standard_normal(20000).astype(np.float32) * 10.0 ** rng.integers(-8, 8, 20000),
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 3.0e38, -1e-40], np.float32)])
    x = x.astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(O.bf16_round(x), ref)
    assert np.array_equal(O.bf16_to_float(O.bf16_round(x)), torch.from_numpy(x).to(torch.bfloat16).float().numpy())


# ---------------------------------------------------------------------- rope
def _rand_heads(rng, n, heads=2, hd=80):
    return rng.standard_normal((n, heads, hd))


def test_rope_closed_form_angles():
    """omega_k = 1e4^(-k/20): omega_5 = 0.1, omega_10 = 0.01, omega_15 = 0.001; pairs
    0..19 turn with h, 20..39 with w; pair j couples elements j and j+40."""
    pos = np.array([[3, 0], [0, 7], [1, 0]])
    a = O.rope_angles(pos)
    assert a[0, 5] == pytest.approx(0.3, rel=1e-14)
    assert a[0, 10] == pytest.approx(0.03, rel=1e-14)
    assert a[1, 20 + 15] == pytest.approx(0.007, rel=1e-13)
    assert (a[0, 20:] == 0).all() and (a[1, :20] == 0).all()
    x = np.zeros((3, 1, 80))
    x[:, 0, 5] = 1.0
    y = O.apply_rope(x, a)
    assert y[0, 0, 5] == pytest.approx(math.cos(0.3)) and y[0, 0, 45] == pytest.approx(math.sin(0.3))
    assert y[1, 0, 5] == 1.0 and y[1, 0, 45] == 0.0    # w rotation leaves pair 5 alone
    x2 = np.zeros((3, 1, 80))
    x2[:, 0, 40] = 1.0                                   # second element of pair 0
    y2 = O.apply_rope(x2, a)
    assert y2[2, 0, 0] == pytest.approx(-math.sin(1.0)) and y2[2, 0, 40] == pytest.approx(math.cos(1.0))


def test_rope_norm_and_identity():
    rng = np.random.default_rng(4)
    x = _rand_heads(rng, 50)
    pos = rng.integers(0, 256, size=(50, 2))
    y = O.apply_rope(x, O.rope_angles(pos))
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-12)
    z = O.apply_rope(x, O.rope_angles(np.zeros((50, 2), np.int64)))
    np.testing.assert_array_equal(z, x)


def test_rope_relative_offset():
    """(R_p q) . (R_r k) depends only on p - r."""
    rng = np.random.default_rng(5)
    q = _rand_heads(rng, 1, 1)
    k = _rand_heads(rng, 1, 1)
    for _ in range(20):
        p, r, s = rng.integers(0, 200, size=(3, 2))
        lhs = (O.apply_rope(q, O.rope_angles(p[None])) * O.apply_rope(k, O.rope_angles(r[None]))).sum()
        rhs = (O.apply_rope(q, O.rope_angles((p + s)[None])) * O.apply_rope(k, O.rope_angles((r + s)[None]))).sum()
        assert lhs == pytest.approx(rhs, rel=1e-9, abs=1e-9)
        d = (O.apply_rope(q, O.rope_angles((p - r)[None])) * k).sum()
        assert lhs == pytest.approx(d, rel=1e-9, abs=1e-9)


# ------------------------------------------------------------- layer norm
def test_layer_norm_vs_torch_and_moments():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((33, 1280)) * 3 + 1.5
    g = 1 + 0.02 * rng.standard_normal(1280)
    b = 0.02 * rng.standard_normal(1280)
    ref = F.layer_norm(torch.from_numpy(x), (1280,), torch.from_numpy(g), torch.from_numpy(b), eps=1e-6).numpy()
    np.testing.assert_allclose(O.layer_norm(x, g, b, 1e-6), ref, rtol=1e-12, atol=1e-12)
    y = O.layer_norm(x, np.ones(1280), np.zeros(1280), 1e-6)
    np.testing.assert_allclose(y.mean(axis=1), 0, atol=1e-12)
    np.testing.assert_allclose(y.var(axis=1), 1, rtol=1e-5)


# ----------------------------------------------------------- activations
def test_gelu_and_quick_gelu():
    u = np.linspace(-9, 9, 1001)
    np.testing.assert_allclose(O.gelu_erf(u), F.gelu(torch.from_numpy(u), approximate="none").numpy(),
                               rtol=1e-12, atol=1e-14)
    # g(u) - g(-u) = u for both (sigmoid(x) + sigmoid(-x) = 1, erf odd)
    np.testing.assert_allclose(O.quick_gelu(u) - O.quick_gelu(-u), u, atol=1e-12)
    np.testing.assert_allclose(O.gelu_erf(u) - O.gelu_erf(-u), u, atol=1e-12)
    assert O.quick_gelu(np.array([0.0]))[0] == 0.0
    # slope 1/2 at the origin, and the 1.702 factor: d/du at 0 of u*sig(a u) = 1/2; second
    # derivative at 0 is a/2
    e = 1e-4
    second = (O.quick_gelu(np.array([e]))[0] + O.quick_gelu(np.array([-e]))[0]) / e ** 2
    assert second == pytest.approx(1.702 / 2, rel=1e-4)


# --------------------------------------------------------------- attention
def _brute_attention(q, k, v, cu):
    n, heads, hd = q.shape
    out = np.zeros_like(q)
    for i in range(len(cu) - 1):
        for h in range(heads):
            for a in range(cu[i], cu[i + 1]):
                s = [sum(q[a, h, d] * k[b, h, d] for d in range(hd)) / math.sqrt(hd)
                     for b in range(cu[i], cu[i + 1])]
                m = max(s)
                e = [math.exp(x - m) for x in s]
                z = sum(e)
                for d in range(hd):
                    out[a, h, d] = sum(e[j] * v[cu[i] + j, h, d] for j in range(len(e))) / z
    return out


def test_attention_bruteforce_tiny():
    rng = np.random.default_rng(7)
    cu = np.array([0, 4, 12, 16])
    q, k, v = (rng.standard_normal((16, 2, 6)) for _ in range(3))
    np.testing.assert_allclose(O.attention_varlen(q, k, v, cu), _brute_attention(q, k, v, cu), rtol=1e-12,
                               atol=1e-12)


def test_attention_vs_sdpa_block_diagonal_and_packed():
    rng = np.random.default_rng(8)
    cu = np.array([0, 24, 40, 100])
    n = 100
    q, k, v = (rng.standard_normal((n, 3, 80)) for _ in range(3))
    seg = np.searchsorted(cu, np.arange(n), side="right") - 1
    mask = torch.from_numpy(seg[:, None] == seg[None, :])
    t = lambda a: torch.from_numpy(a).permute(1, 0, 2)
    ref = F.scaled_dot_product_attention(t(q), t(k), t(v), attn_mask=mask).permute(1, 0, 2).numpy()
    got = O.attention_varlen(q, k, v, cu)
    np.testing.assert_allclose(got, ref, rtol=1e-10, atol=1e-12)
    # packed == per image
    for i in range(3):
        a, b = cu[i], cu[i + 1]
        one = O.attention_varlen(q[a:b], k[a:b], v[a:b], np.array([0, b - a]))
        np.testing.assert_allclose(got[a:b], one, rtol=1e-12, atol=1e-12)
    # restricted query rows give the same rows
    rows = np.array([3, 30, 99, 41])
    np.testing.assert_allclose(O.attention_varlen(q, k, v, cu, q_rows=rows), got[rows], rtol=1e-12)


def test_attention_equal_keys_is_mean_of_values():
    rng = np.random.default_rng(9)
    q = rng.standard_normal((8, 1, 80))
    k = np.repeat(rng.standard_normal((1, 1, 80)), 8, axis=0)
    v = rng.standard_normal((8, 1, 80))
    got = O.attention_varlen(q, k, v, np.array([0, 8]))
    np.testing.assert_allclose(got, np.repeat(v.mean(axis=0, keepdims=True), 8, axis=0), rtol=1e-12)


def test_attention_position_shift_invariance():
    """Adding one constant (dh, dw) to every position leaves rotary attention unchanged."""
    rng = np.random.default_rng(10)
    cu, pos, _ = O.seq_meta([(1, 4, 6)])
    q, k, v = (rng.standard_normal((24, 2, 80)) for _ in range(3))
    out = []
    for shift in ([0, 0], [5, 11]):
        a = O.rope_angles(pos + np.array(shift))
        out.append(O.attention_varlen(O.apply_rope(q, a), O.apply_rope(k, a), v, cu))
    np.testing.assert_allclose(out[0], out[1], rtol=1e-9, atol=1e-12)


# --------------------------------------------------------------- the block
def _block_params(rng, d=1280, m=5120, scale=0.02):
    p = {"ln1_w": 1 + scale * rng.standard_normal(d), "ln1_b": scale * rng.standard_normal(d),
         "qkv_w": scale * rng.standard_normal((3 * d, d)), "qkv_b": scale * rng.standard_normal(3 * d),
         "proj_w": scale * rng.standard_normal((d, d)), "proj_b": scale * rng.standard_normal(d),
         "ln2_w": 1 + scale * rng.standard_normal(d), "ln2_b": scale * rng.standard_normal(d),
         "fc1_w": scale * rng.standard_normal((m, d)), "fc1_b": scale * rng.standard_normal(m),
         "fc2_w": scale * rng.standard_normal((d, m)), "fc2_b": scale * rng.standard_normal(d)}
    return p


def test_block_uniform_attention_special_case():
    """With the q and k thirds of W_qkv and b_qkv zero, every score is 0, so each
    token attends uniformly to its own image: o = image mean of the value rows.
    With W_fc2 = 0 the MLP adds b2.  Pins the [q|k|v] split, value rows not
    rotated, per-image segments, and both residual adds of a pre-norm block."""
    rng = np.random.default_rng(11)
    d = 1280
    p = _block_params(rng)
    p["qkv_w"][:2 * d] = 0
    p["qkv_b"][:2 * d] = 0
    p["fc2_w"][:] = 0
    grids = [(1, 2, 4), (1, 4, 4)]
    cu, pos, _ = O.seq_meta(grids)
    z = rng.standard_normal((cu[-1], d))
    got = O.vision_block(z, p, cu, O.rope_angles(pos))
    a = (z - z.mean(1, keepdims=True)) / np.sqrt(z.var(1, keepdims=True) + 1e-6) * p["ln1_w"] + p["ln1_b"]
    vrows = a @ p["qkv_w"][2 * d:].T + p["qkv_b"][2 * d:]
    want = np.empty_like(z)
    for i in range(len(grids)):
        s = slice(cu[i], cu[i + 1])
        want[s] = z[s] + vrows[s].mean(axis=0) @ p["proj_w"].T + p["proj_b"] + p["fc2_b"]
    np.testing.assert_allclose(got, want, rtol=1e-10, atol=1e-10)


def test_block_is_pre_norm_scale_invariant():
    """Pre-norm: each half adds f(LN(input)) to its input.  With the MLP's output
    weight zero (so it adds only b2), block(c z) - c z equals block(z) - z for
    c > 0 (up to eps); likewise with the attention projection zeroed.  A
    post-norm block (LN after the residual add) fails both."""
    rng = np.random.default_rng(12)
    cu, pos, _ = O.seq_meta([(1, 4, 4)])
    z = rng.standard_normal((16, 1280))
    a = O.rope_angles(pos)
    for zero in (("fc2_w",), ("proj_w", "proj_b")):
        p = _block_params(rng)
        for key in zero:
            p[key][:] = 0
        d1 = O.vision_block(z, p, cu, a) - z
        d2 = O.vision_block(7.0 * z, p, cu, a) - 7.0 * z
        np.testing.assert_allclose(d1, d2, rtol=1e-5, atol=1e-5)


def test_block_rows_equals_block():
    rng = np.random.default_rng(13)
    p = _block_params(rng)
    grids = [(1, 4, 4), (1, 6, 2), (1, 2, 2)]
    cu, pos, _ = O.seq_meta(grids)
    z = rng.standard_normal((cu[-1], 1280))
    a = O.rope_angles(pos)
    full = O.vision_block(z, p, cu, a)
    rows = np.array([0, 5, 17, 20, 27, 31])
    np.testing.assert_allclose(O.vision_block_rows(z, p, cu, a, rows), full[rows], rtol=1e-10, atol=1e-12)


def test_block_rows_equals_block_windowed():
    """Sampled rows of a windowed block (ragged edge windows) equal the whole
    windowed block at those rows."""
    rng = np.random.default_rng(14)
    p = _block_params(rng)
    grids = [(1, 6, 10), (2, 4, 2)]
    cu, pos, _ = O.seq_meta(grids)
    z = rng.standard_normal((cu[-1], 1280))
    a = O.rope_angles(pos)
    g = O.window_groups(grids, 4)
    full = O.vision_block(z, p, cu, a, groups=g)
    rows = np.array([0, 7, 22, 45, 59, 60, 71, 75])
    np.testing.assert_allclose(O.vision_block_rows(z, p, cu, a, rows, groups=g), full[rows],
                               rtol=1e-10, atol=1e-12)
    # and they differ from the full-attention rows (the windows matter here)
    assert not np.allclose(O.vision_block_rows(z, p, cu, a, rows), full[rows])


def _both_block_forms(z, p, cu, angles, **kw):
    """The block through vision_block (whole) and vision_block_rows (every row,
    and a scattered subset), so a wiring pin holds for both forms."""
    full = O.vision_block(z, p, cu, angles, **kw)
    n = z.shape[0]
    sub = np.arange(0, n, 3)
    return [(np.arange(n), full),
            (np.arange(n), O.vision_block_rows(z, p, cu, angles, np.arange(n), **kw)),
            (sub, O.vision_block_rows(z, p, cu, angles, sub, **kw))]


# QuickGELU u * sigmoid(1.702 u) at u = -2, -1, -0.5, 0, 0.5, 1, 2, 3: the
# activation the tower's configuration names for its MLP.  Tabulated from the
# definition to 16 digits; exact GELU(1) would be 0.8413447460685429 and the
# identity 1.0, so a swapped activation misses these by >= 4e-3.
QUICK_GELU_TABLE = ((-2.0, -0.06434137685579186), (-1.0, -0.1542042340671787),
                    (-0.5, -0.1496115633936199), (0.0, 0.0), (0.5, 0.35038843660638014),
                    (1.0, 0.8457957659328212), (2.0, 1.9356586231442083), (3.0, 2.981928690292214))


def test_block_mlp_activation_and_fc1_bias_closed_form():
    """Neurarch card, Structure table, ViT Block rows (MLP 5120) with the MLP
    activation the configuration names (QuickGELU).  With W_qkv, b_qkv, W_o and
    b_o zero the attention half adds nothing; with W_1 = 0 the MLP input is
    u = b_1 exactly, whatever LN2 gives.  W_2 routes unit j to output column
    j for j < 8 and b_2 is a known vector, so block(z) - z = QuickGELU(b_1[j])
    + b_2 on those columns and b_2 elsewhere.  A different activation (exact
    GELU, none) or a dropped fc1 bias misses the tabulated values; torch's
    sigmoid gives the same table independently."""
    rng = np.random.default_rng(21)
    d, m = 1280, 5120
    p = _block_params(rng)
    for key in ("qkv_w", "qkv_b", "proj_w", "proj_b", "fc1_w"):
        p[key][:] = 0
    u = np.array([x for x, _ in QUICK_GELU_TABLE])
    want_act = np.array([y for _, y in QUICK_GELU_TABLE])
    p["fc1_b"] = rng.standard_normal(m)
    p["fc1_b"][:8] = u
    p["fc2_w"] = np.zeros((d, m))
    p["fc2_w"][np.arange(8), np.arange(8)] = 1.0
    p["fc2_b"] = 0.1 * rng.standard_normal(d)
    ut = torch.tensor(u, dtype=torch.float64)
    np.testing.assert_allclose((ut * torch.sigmoid(1.702 * ut)).numpy(), want_act, rtol=1e-14, atol=1e-16)
    grids = [(1, 2, 4), (1, 2, 2)]
    cu, pos, _ = O.seq_meta(grids)
    z = rng.standard_normal((cu[-1], d))
    want = np.tile(p["fc2_b"], (cu[-1], 1))
    want[:, :8] += want_act
    for rows, got in _both_block_forms(z, p, cu, O.rope_angles(pos)):
        np.testing.assert_allclose(got - z[rows], want[rows], rtol=1e-12, atol=1e-13)


def test_block_ln2_uses_its_own_affine_and_eps():
    """Pre-norm MLP half: a = LN2(z) with LN2's own gain and bias and eps 1e-6
    (Neurarch card, Structure table, ViT Block rows; LayerNorm eps of the
    configuration).  Attention adds nothing (W_qkv, b_qkv, W_o, b_o zero).
    Row i of z is c_i + a_i * s with s = (+1, -1, +1, ...), so its mean is c_i
    and its biased variance a_i^2: LN2 gives s_j * r_i * g2[j] + b2ln[j] with
    r_i = a_i / sqrt(a_i^2 + 1e-6) in closed form.  W_1 = I on the first 8
    columns (b_1 = 0) and W_2 routes them out, so block(z) - z =
    QuickGELU(LN2(z)[:, :8]) (activation as pinned above).  a_i down to 1e-3
    makes eps visible (r = 0.7071 at a = 1e-3); LN1's affine is set far from
    LN2's so borrowing it fails."""
    rng = np.random.default_rng(22)
    d, m = 1280, 5120
    p = _block_params(rng)
    for key in ("qkv_w", "qkv_b", "proj_w", "proj_b", "fc1_w", "fc1_b", "fc2_b"):
        p[key][:] = 0
    p["ln1_w"][:] = 3.0
    p["ln1_b"][:] = -1.0
    p["ln2_w"] = 1 + 0.5 * rng.standard_normal(d)
    p["ln2_b"] = 0.5 * rng.standard_normal(d)
    p["fc1_w"][np.arange(8), np.arange(8)] = 1.0
    p["fc2_w"] = np.zeros((d, m))
    p["fc2_w"][np.arange(8), np.arange(8)] = 1.0
    grids = [(1, 2, 4)]
    cu, pos, _ = O.seq_meta(grids)
    s = np.where(np.arange(d) % 2 == 0, 1.0, -1.0)
    c = np.array([0.0, 5.0, -3.0, 1e3, 0.25, -0.5, 2.0, 7.0])
    a = np.array([1.0, 2.0, 1e-3, 0.5, 3e-3, 10.0, 1.0, 0.1])
    z = c[:, None] + a[:, None] * s[None, :]
    r = a / np.sqrt(a * a + 1e-6)
    u = s[None, :8] * r[:, None] * p["ln2_w"][None, :8] + p["ln2_b"][None, :8]
    ut = torch.from_numpy(u)
    want = np.zeros_like(z)
    want[:, :8] = (ut * torch.sigmoid(1.702 * ut)).numpy()
    for rows, got in _both_block_forms(z, p, cu, O.rope_angles(pos)):
        np.testing.assert_allclose(got - z[rows], want[rows], rtol=1e-9, atol=1e-9)


def test_block_rope_on_q_and_k_closed_form_scores():
    """Inside the block both q and k carry their patch's 2-D rotation and v
    does not (Neurarch card, Structure table row "2D RoPE"; LiteRT-LM card,
    Conversion notes: each patch carries its own 2-D rope).

    q = alpha (e_0 + e_20) and k = alpha (e_0 + e_40 + e_20 + e_60) for every
    token (from the biases, W_q = W_k = 0) touch only rotation pair 0 (angle
    h, elements 0 and 40) and pair 20 (angle w, elements 20 and 60); rotating
    the pair (x, y) by a gives (x cos a - y sin a, y cos a + x sin a), so
    q_i . k_r = alpha^2 (cos D + sin D) summed over D = h_i - h_r and
    w_i - w_r: a closed form with no rope routine in it, and not symmetric in
    q and k (swapping them flips the sine terms).  Token l of an image is
    z = e_{2l} - e_{2l+1}, which LN1 (gain 1, bias 0) maps to
    kappa (e_{2l} - e_{2l+1}), kappa = 1 / sqrt(2/1280 + 1e-6); W_v row r =
    e_{2r} then makes v_l = kappa e_l inside head 0.  W_o = I, MLP output 0,
    so block(z) - z in head 0 column r is kappa P[i, r], the softmax over the
    image's keys of the closed-form scores / sqrt(80).  No rotation on k (or
    on q) makes P uniform, a rotated v leaks into columns 40..47, a wrong
    scale or segment changes P."""
    rng = np.random.default_rng(23)
    d, hd, alpha = 1280, 80, 3.0
    p = _block_params(rng)
    for key in ("qkv_w", "qkv_b", "proj_b", "fc2_w", "fc2_b"):
        p[key][:] = 0
    p["ln1_w"][:] = 1.0
    p["ln1_b"][:] = 0.0
    p["proj_w"] = np.eye(d)
    # q = alpha (e_0 + e_20); k = alpha (e_0 + e_40 + e_20 + e_60): head 0, pairs 0 and 20
    p["qkv_b"][[0, 20]] = alpha
    p["qkv_b"][d + np.array([0, 40, 20, 60])] = alpha
    p["qkv_w"][2 * d + np.arange(8), 2 * np.arange(8)] = 1.0
    # merge-group slot order of a 2 x 4 grid and of a 2 x 2 grid, listed by hand
    hw = {(1, 2, 4): [(0, 0), (0, 1), (1, 0), (1, 1), (0, 2), (0, 3), (1, 2), (1, 3)],
          (1, 2, 2): [(0, 0), (0, 1), (1, 0), (1, 1)]}
    grids = [(1, 2, 4), (1, 2, 2)]
    pos = np.array(hw[grids[0]] + hw[grids[1]], dtype=np.float64)
    cu = np.array([0, 8, 12])
    angles = rng.uniform(-3, 3, (12, hd // 2))   # pairs other than 0 and 20 play no part
    angles[:, 0] = pos[:, 0]
    angles[:, 20] = pos[:, 1]
    n = 12
    z = np.zeros((n, d))
    local = np.concatenate([np.arange(8), np.arange(4)])
    z[np.arange(n), 2 * local] = 1.0
    z[np.arange(n), 2 * local + 1] = -1.0
    kappa = 1.0 / math.sqrt(2.0 / d + 1e-6)
    want = np.zeros((n, d))
    for i in range(len(cu) - 1):
        seg = np.arange(cu[i], cu[i + 1])
        for qi in seg:
            dh, dw = pos[qi, 0] - pos[seg, 0], pos[qi, 1] - pos[seg, 1]
            s = alpha ** 2 * (np.cos(dh) + np.sin(dh) + np.cos(dw) + np.sin(dw)) / math.sqrt(hd)
            e = np.exp(s - s.max())
            want[qi, :len(seg)] = kappa * e / e.sum()
    assert want[:8, :8].std() > 0.01            # the scores really vary across keys
    for rows, got in _both_block_forms(z, p, cu, angles):
        np.testing.assert_allclose(got - z[rows], want[rows], rtol=1e-10, atol=1e-12)


# ---------------------------------------------------------------- merger
def test_merger_identity_special_case_and_shapes():
    """fc1 = I, b1 = 0, fc2 = I[:out], b2 = 0 leaves GELU(LN(z) grouped) — pins
    LN before grouping, the 4-token concat, GELU-erf between the Linears."""
    rng = np.random.default_rng(14)
    d, n = 8, 12
    z = rng.standard_normal((n, d))
    p = {"merger.ln_w": 1 + 0.1 * rng.standard_normal(d), "merger.ln_b": 0.1 * rng.standard_normal(d),
         "merger.fc1_w": np.eye(4 * d), "merger.fc1_b": np.zeros(4 * d),
         "merger.fc2_w": np.eye(4 * d)[:5], "merger.fc2_b": np.zeros(5)}
    got = O.patch_merge(z, p)
    ln = F.layer_norm(torch.from_numpy(z), (d,), torch.from_numpy(p["merger.ln_w"]),
                      torch.from_numpy(p["merger.ln_b"]), eps=1e-6)
    ref = F.gelu(ln.reshape(n // 4, 4 * d))[:, :5].numpy()
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)
    with pytest.raises(ValueError):
        O.patch_merge(z[:10], p)


def test_page_shapes_through_merger():
    """Encoder/adapter shapes of the pages: rows N and N/4, widths 1280 and out_dim."""
    for row in _golden_rows("page_shapes.txt"):
        lhs, rhs = row.split("->")
        h, w, out_dim = map(int, lhs.split())
        n, dw, m, mw = map(int, rhs.split())
        g = O.grid_thw(h, w)[2]
        cu, _, _ = O.seq_meta([g])
        assert cu[-1] == n and dw == 1280
        z = np.zeros((n, 16))
        p = {"merger.ln_w": np.ones(16), "merger.ln_b": np.zeros(16), "merger.fc1_w": np.zeros((64, 64)),
             "merger.fc1_b": np.zeros(64), "merger.fc2_w": np.zeros((out_dim, 64)),
             "merger.fc2_b": np.zeros(out_dim)}
        assert O.patch_merge(z, p).shape == (m, mw)


# -------------------------------------------------------------- the tower
def test_tower_raster_order_equals_block_order():
    """LiteRT-LM card: running the blocks in raster order, each patch carrying its
    own 2-D rope, then merging by four strided slices equals the block-order
    encoder followed by the contiguous merge."""
    rng = np.random.default_rng(15)
    d = 1280
    grids = [(1, 4, 6), (1, 4, 4)]
    imgs = [rng.uniform(-1, 1, (1, 3, 14 * g[1], 14 * g[2])).astype(np.float32) for g in grids]
    params = {"patch_w": 0.02 * rng.standard_normal((d, 3, 2, 14, 14))}
    for k, v in _block_params(rng).items():
        params["blocks.0." + k] = v
    for k, v in {"ln_w": 1 + 0.02 * rng.standard_normal(d), "ln_b": 0.02 * rng.standard_normal(d),
                 "fc1_w": 0.02 * rng.standard_normal((4 * d, 4 * d)), "fc1_b": 0.02 * rng.standard_normal(4 * d),
                 "fc2_w": 0.02 * rng.standard_normal((24, 4 * d)), "fc2_b": 0.02 * rng.standard_normal(24)}.items():
        params["merger." + k] = v
    _, z_blk, out_blk = O.encode(imgs, params, depth=1)
    # raster-order tower
    xs, poss, cu = [], [], [0]
    for img, (t, gh, gw) in zip(imgs, grids):
        xs.append(O.raster_patches(img, (t, gh, gw)))
        hh, ww = np.meshgrid(np.arange(gh), np.arange(gw), indexing="ij")
        poss.append(np.stack([hh.ravel(), ww.ravel()], 1))
        cu.append(cu[-1] + gh * gw)
    z = O.patch_embed(np.concatenate(xs).astype(np.float64), params["patch_w"])
    z = O.vision_block(z, O.block_params(params, 0), np.array(cu), O.rope_angles(np.concatenate(poss)))
    outs = []
    for i, (t, gh, gw) in enumerate(grids):
        f = O.layer_norm(z[cu[i]:cu[i + 1]], params["merger.ln_w"], params["merger.ln_b"]).reshape(gh, gw, d)
        g = np.concatenate([f[0::2, 0::2], f[0::2, 1::2], f[1::2, 0::2], f[1::2, 1::2]], -1).reshape(-1, 4 * d)
        outs.append(O.gelu_erf(g @ params["merger.fc1_w"].T + params["merger.fc1_b"]) @ params["merger.fc2_w"].T
                    + params["merger.fc2_b"])
    np.testing.assert_allclose(out_blk, np.concatenate(outs), rtol=1e-9, atol=1e-12)


def test_tower_depth_zero_is_patch_embed():
    rng = np.random.default_rng(16)
    img = rng.uniform(-1, 1, (1, 3, 56, 56)).astype(np.float32)
    w = rng.standard_normal((12, 3, 2, 14, 14))
    g = (1, 4, 4)
    z = O.vision_forward(O.patchify([img], [g]), {"patch_w": w}, [g], depth=0, heads=3)
    _, _, perm = O.seq_meta([g])
    np.testing.assert_allclose(z, _conv3d_reference(img, w)[perm], rtol=1e-12)


# ------------------------------------------------------------ windowed attention
def test_window_groups_hand_listed():
    """window_groups on a 4 x 6 grid with 4-patch windows, listed by hand from
    the merge-group order (groups (0,0) (0,1) (0,2) / (1,0) (1,1) (1,2), four
    slots each): the left window holds groups (0,0) (0,1) (1,0) (1,1), the
    truncated right window groups (0,2) (1,2).  A swapped h/w or a window
    key without the row term fails here."""
    got = [list(map(int, g)) for g in O.window_groups([(1, 4, 6)], 4)]
    assert got == [list(range(0, 8)) + list(range(12, 20)), list(range(8, 12)) + list(range(20, 24))]


@pytest.mark.parametrize("grids,window", [([(1, 10, 10)], 4), ([(1, 8, 8), (1, 6, 14)], 4),
                                          ([(2, 6, 4)], 2), ([(1, 16, 12)], 8)])
def test_window_groups_partition(grids, window):
    """Windows partition each frame; sizes follow min(W, edge remainder) on
    both axes; all members of a window share (image, frame, h // W, w // W)."""
    cu, pos, _ = O.seq_meta(grids)
    groups = O.window_groups(grids, window)
    allrows = np.sort(np.concatenate(groups))
    np.testing.assert_array_equal(allrows, np.arange(cu[-1]))
    gi = 0
    for i, (t, gh, gw) in enumerate(grids):
        for tt in range(t):
            for wy in range(-(-gh // window)):
                for wx in range(-(-gw // window)):
                    g = groups[gi]
                    gi += 1
                    assert len(g) == min(window, gh - wy * window) * min(window, gw - wx * window)
                    assert np.all((g >= cu[i] + tt * gh * gw) & (g < cu[i] + (tt + 1) * gh * gw))
                    assert np.all(pos[g, 0] // window == wy) and np.all(pos[g, 1] // window == wx)
    assert gi == len(groups)


def _brute_masked_attention(q, k, v, same):
    n, heads, hd = q.shape
    out = np.zeros_like(q)
    for h in range(heads):
        for a in range(n):
            js = [b for b in range(n) if same(a, b)]
            s = [sum(q[a, h, d] * k[b, h, d] for d in range(hd)) / math.sqrt(hd) for b in js]
            m = max(s)
            e = [math.exp(x - m) for x in s]
            z = sum(e)
            for d in range(hd):
                out[a, h, d] = sum(e[j] * v[b, h, d] for j, b in enumerate(js)) / z
    return out


def test_window_attention_bruteforce():
    """attention_groups over the windows of a 6 x 6 grid (W = 4: windows of
    16, 8, 8 and 4 patches) equals a masked triple loop where a attends b
    iff both sit in the same window (h // 4, w // 4)."""
    grids = [(1, 6, 6)]
    _, pos, _ = O.seq_meta(grids)
    rng = np.random.default_rng(11)
    q, k, v = (rng.standard_normal((36, 2, 4)) for _ in range(3))
    got = O.attention_groups(q, k, v, O.window_groups(grids, 4))
    same = lambda a, b: (pos[a, 0] // 4, pos[a, 1] // 4) == (pos[b, 0] // 4, pos[b, 1] // 4)
    np.testing.assert_allclose(got, _brute_masked_attention(q, k, v, same), rtol=1e-12, atol=1e-12)


def _tiny_tower_params(d=64, heads=4, mlp=128, depth=2, seed=3):
    rng = np.random.default_rng(seed)
    p = {"patch_w": rng.standard_normal((d, 3 * 2 * 14 * 14)) * 0.02}
    for l in range(depth):
        pre = f"blocks.{l}."
        p[pre + "ln1_w"] = 1 + rng.standard_normal(d) * 0.02
        p[pre + "ln1_b"] = rng.standard_normal(d) * 0.02
        p[pre + "qkv_w"] = rng.standard_normal((3 * d, d)) * 0.2
        p[pre + "qkv_b"] = rng.standard_normal(3 * d) * 0.02
        p[pre + "proj_w"] = rng.standard_normal((d, d)) * 0.2
        p[pre + "proj_b"] = rng.standard_normal(d) * 0.02
        p[pre + "ln2_w"] = 1 + rng.standard_normal(d) * 0.02
        p[pre + "ln2_b"] = rng.standard_normal(d) * 0.02
        p[pre + "fc1_w"] = rng.standard_normal((mlp, d)) * 0.2
        p[pre + "fc1_b"] = rng.standard_normal(mlp) * 0.02
        p[pre + "fc2_w"] = rng.standard_normal((d, mlp)) * 0.2
        p[pre + "fc2_b"] = rng.standard_normal(d) * 0.02
    return p


def test_windowed_tower_special_cases():
    """A window covering the whole grid, or every block listed as full, gives
    the unwindowed tower; a real window changes the result."""
    grids = [(1, 6, 8), (1, 4, 4)]
    p = _tiny_tower_params()
    rng = np.random.default_rng(5)
    x = rng.standard_normal((48 + 16, 3 * 2 * 14 * 14))
    full = O.vision_forward(x, p, grids, 2, heads=4)
    np.testing.assert_allclose(O.vision_forward(x, p, grids, 2, heads=4, window=8), full, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(O.vision_forward(x, p, grids, 2, heads=4, window=2, full_blocks=(0, 1)), full,
                               rtol=1e-12, atol=1e-12)
    assert not np.allclose(O.vision_forward(x, p, grids, 2, heads=4, window=2), full, rtol=1e-6)


def test_windowed_block_isolates_windows():
    """In a windowed block, changing the input rows of one window changes the
    output rows of that window only (LayerNorm and the MLP are per row)."""
    grids = [(1, 8, 8)]
    cu, pos, _ = O.seq_meta(grids)
    p = O.block_params(_tiny_tower_params(depth=1), 0)
    angles = O.rope_angles(pos, 16)
    groups = O.window_groups(grids, 4)
    rng = np.random.default_rng(9)
    z = rng.standard_normal((64, 64))
    base = O.vision_block(z, p, cu, angles, heads=4, groups=groups)
    z2 = z.copy()
    z2[groups[1]] += rng.standard_normal((len(groups[1]), 64))
    out = O.vision_block(z2, p, cu, angles, heads=4, groups=groups)
    changed = np.nonzero(np.any(np.abs(out - base) > 0, axis=1))[0]
    np.testing.assert_array_equal(np.sort(changed), np.sort(groups[1]))


# ------------------------------------------------ Conv2d fold, CLIP normalisation
def test_fold_identity_equals_conv3d():
    """Still images: folded patches x temporally summed weight == the Conv3d
    product over the duplicated frame (the LiteRT-LM fold), in float64."""
    rng = np.random.default_rng(21)
    sides = [(56, 84), (28 * 3, 28 * 2)]
    imgs = [rng.uniform(-1, 1, (1, 3, h, w)) for h, w in sides]
    grids = [O.grid_thw(h, w, 1)[2] for h, w in sides]
    w3 = rng.standard_normal((64, 3, 2, 14, 14))
    ref = O.patch_embed(O.patchify(imgs, grids), w3)
    xf = O.patchify_folded(imgs, grids, width=592)
    wf = O.fold_patch_weight(w3, width=592)
    assert xf.shape == (ref.shape[0], 592) and wf.shape == (64, 592)
    np.testing.assert_allclose(xf @ wf.T, ref, rtol=1e-12, atol=1e-12)
    # a weight whose two taps differ shows the sum is over the temporal axis
    # (not over channels or rows): tap 1 = 0 leaves half the Conv3d product
    w_half = w3.copy()
    w_half[:, :, 1] = 0
    np.testing.assert_allclose(O.patchify_folded(imgs, grids) @ O.fold_patch_weight(w_half).T,
                               O.patch_embed(O.patchify(imgs, grids), w_half), rtol=1e-12, atol=1e-12)


def test_folded_rows_are_the_first_temporal_slice_and_pads_zero():
    rng = np.random.default_rng(22)
    imgs = [rng.uniform(0, 1, (1, 3, 56, 112)).astype(np.float32)]
    grids = [(1, 4, 8)]
    full = O.patchify(imgs, grids).reshape(32, 3, 2, 14, 14)
    xf = O.patchify_folded(imgs, grids, width=600)
    assert np.array_equal(xf[:, :588].reshape(32, 3, 14, 14), full[:, :, 0])
    assert np.array_equal(full[:, :, 0], full[:, :, 1])  # the still frame is duplicated
    assert (xf[:, 588:] == 0).all()
    # hand-listed element: merge-group slot 5 is (block row 0, block col 1,
    # dy 0, dx 1) -> patch (h 0, w 3); element (c 2, r 3, q 4)
    assert xf[5, 2 * 196 + 3 * 14 + 4] == imgs[0][0, 2, 3, 3 * 14 + 4]


def test_fold_rejects_multi_frame_images():
    img = np.zeros((2, 3, 28, 28), np.float32)
    with pytest.raises(ValueError):
        O.patchify_folded([img], [(1, 2, 2)])


def test_normalize_closed_forms():
    m = np.array(O.CLIP_MEAN, np.float32)
    s = np.array(O.CLIP_STD, np.float32)
    x = np.stack([np.full((2, 2), m[c]) for c in range(3)])[None].astype(np.float32)
    assert (O.normalize(x) == 0).all()                      # the mean maps to 0
    y = O.normalize(x + s.reshape(1, 3, 1, 1))              # one std above -> ~1
    np.testing.assert_allclose(y, 1.0, rtol=0, atol=2e-7)
    # channel order: a grey pixel of 0.5 lands at (0.5 - mean_c) / std_c per channel
    g = O.normalize(np.full((1, 3, 1, 1), 0.5, np.float32))[0, :, 0, 0]
    np.testing.assert_allclose(g, [(0.5 - 0.48145466) / 0.26862954, (0.5 - 0.4578275) / 0.26130258,
                                   (0.5 - 0.40821073) / 0.27577711], rtol=1e-6)
    # the CLIP constants of the processor table
    assert O.CLIP_MEAN == (0.48145466, 0.4578275, 0.40821073)
    assert O.CLIP_STD == (0.26862954, 0.26130258, 0.27577711)


# ------------------------------------------------------------ int8 weights
def test_quantize_i8_hand_example():
    w = np.array([[0.5, -1.0, 0.25, 0.0],       # amax 1.0 -> scale 1/127
                  [3.0, 1.5, -0.75, 2.25],       # amax 3.0 -> scale 3/127
                  [0.0, 0.0, 0.0, 0.0],          # all zero -> scale 1, codes 0
                  [127.0, 62.5, -0.5, 1.5]],     # scale exactly 1: ties 62.5 -> 62, -0.5 -> 0, 1.5 -> 2
                 dtype=np.float32)
    q, s = O.quantize_i8(w)
    assert s.dtype == np.float32 and q.dtype == np.int8
    assert s[0] == np.float32(1.0) / np.float32(127) and s[1] == np.float32(3.0) / np.float32(127) and s[2] == 1
    # 0.5 * 127 = 63.5 -> 64 (half to even), 0.25 * 127 = 31.75 -> 32; the
    # largest magnitude of a row maps to +-127
    assert q[0].tolist() == [64, -127, 32, 0]
    assert q[1].tolist() == [127, 64, -32, 95]   # 1.5/3*127 = 63.5 -> 64; 2.25/3*127 = 95.25 -> 95
    assert (q[2] == 0).all()
    assert s[3] == 1 and q[3].tolist() == [127, 62, 0, 2]


def test_quantize_i8_error_bound_and_extremes():
    rng = np.random.default_rng(31)
    w = (rng.standard_normal((64, 300)) * 0.02).astype(np.float32)
    q, s = O.quantize_i8(w)
    err = np.abs(q.astype(np.float64) * s[:, None] - w)
    # rounding to the nearest code: at most half a step (plus float32 slack)
    assert (err <= s[:, None].astype(np.float64) * (0.5 + 1e-5)).all()
    assert (np.abs(q).max(axis=1) == 127).all()      # each row's extreme is used
    assert q.min() >= -127                           # -128 never appears
    # the scale is per row: scaling one row leaves the others' codes alone
    w2 = w.copy()
    w2[3] *= 10
    q2, s2 = O.quantize_i8(w2)
    assert np.array_equal(np.delete(q2, 3, 0), np.delete(q, 3, 0)) and np.array_equal(q2[3], q[3])


def test_dequantized_params_touch_only_block_matrices():
    wl = synth.small_workload("q", [(56, 56, 1)], depth=2)
    p = synth.params(wl)
    d = O.dequantized_params(p, 2)
    for k, v in p.items():
        name = k.split(".")[-1]
        if k.startswith("blocks.") and name in O.QUANT_KEYS:
            q, s = O.quantize_i8(v)
            assert np.array_equal(d[k], q.astype(np.float64) * s.astype(np.float64)[:, None])
            assert not np.array_equal(d[k], v)
        else:
            assert d[k] is v
