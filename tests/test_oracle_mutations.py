"""Mutation check of the oracle's pins (CPU only).

Each case plants one plausible mistake in a copy of the oracle's source (a
wrong sign, index, constant, operand or wiring), loads the copy as a fresh
module, and runs the pins named for it with that module in place of the
oracle.  At least one of them must fail; if none does, the pins cannot tell
that mistake from the method and the case fails.  The oracle itself is
never modified: the copy lives only in memory."""
import os
import types

import pytest

import tests.test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "qv_oracle.py")

# (name, [(old, new, expected count), ...], pins expected to catch it)
MUTATIONS = [
    ("block MLP activation QuickGELU -> exact GELU (both block forms)",
     [('quick_gelu(a @ p["fc1_w"].T', 'gelu_erf(a @ p["fc1_w"].T', 1),
      ('quick_gelu(a2 @ p["fc1_w"].T', 'gelu_erf(a2 @ p["fc1_w"].T', 1)],
     ["test_block_mlp_activation_and_fc1_bias_closed_form"]),
    ("fc1 bias dropped (both block forms)",
     [('quick_gelu(a @ p["fc1_w"].T + p["fc1_b"])', 'quick_gelu(a @ p["fc1_w"].T)', 1),
      ('quick_gelu(a2 @ p["fc1_w"].T + p["fc1_b"])', 'quick_gelu(a2 @ p["fc1_w"].T)', 1)],
     ["test_block_mlp_activation_and_fc1_bias_closed_form"]),
    ("LN2 borrows LN1's gain and bias (both block forms)",
     [('p["ln2_w"], p["ln2_b"]', 'p["ln1_w"], p["ln1_b"]', 2)],
     ["test_block_ln2_uses_its_own_affine_and_eps"]),
    ("no rope on k (both block forms)",
     [("k = apply_rope(k, angles)", "k = k", 1),
      ("k = apply_rope(kv[:, :d].reshape(-1, heads, hd), angles[kv_rows])", "k = kv[:, :d].reshape(-1, heads, hd)", 1)],
     ["test_block_rope_on_q_and_k_closed_form_scores"]),
    ("no rope on q (both block forms)",
     [("q = apply_rope(q, angles)", "q = q", 1),
      ("q = apply_rope((aq @ p[\"qkv_w\"][:d].T + p[\"qkv_b\"][:d]).reshape(-1, heads, hd), angles[rows])",
       "q = (aq @ p[\"qkv_w\"][:d].T + p[\"qkv_b\"][:d]).reshape(-1, heads, hd)", 1)],
     ["test_block_rope_on_q_and_k_closed_form_scores"]),
    ("rope also on v (whole-block form)",
     [("v = qkv[:, 2 * d:3 * d].reshape(n, heads, hd)",
       "v = apply_rope(qkv[:, 2 * d:3 * d].reshape(n, heads, hd), angles)", 1)],
     ["test_block_rope_on_q_and_k_closed_form_scores", "test_block_uniform_attention_special_case"]),
    ("QuickGELU constant 1.702 -> 1", [("np.exp(-1.702 * u)", "np.exp(-1.0 * u)", 1)],
     ["test_gelu_and_quick_gelu", "test_block_mlp_activation_and_fc1_bias_closed_form"]),
    ("rotation sign", [("x1 * c - x2 * s", "x1 * c + x2 * s", 1)],
     ["test_rope_closed_form_angles", "test_rope_relative_offset"]),
    ("frequency exponent -k/(hd/2) instead of -k/(hd/4)",
     [("-np.arange(q, dtype=np.float64) / q", "-np.arange(q, dtype=np.float64) / (2 * q)", 1)],
     ["test_rope_closed_form_angles"]),
    ("h and w axes swapped",
     [("np.concatenate([h * omega, w * omega], axis=1)", "np.concatenate([w * omega, h * omega], axis=1)", 1)],
     ["test_rope_closed_form_angles", "test_block_rope_on_q_and_k_closed_form_scores"]),
    ("attention scale 1/hd", [("scale = 1.0 / math.sqrt(hd)\n    rows", "scale = 1.0 / hd\n    rows", 1)],
     ["test_attention_bruteforce_tiny", "test_attention_vs_sdpa_block_diagonal_and_packed"]),
    ("segment leak: keys from the whole batch",
     [("s = (q[rows[sel], h, :] @ k[a:b, h, :].T) * scale", "s = (q[rows[sel], h, :] @ k[:, h, :].T) * scale", 1),
      ("out[sel, h, :] = p @ v[a:b, h, :]", "out[sel, h, :] = p @ v[:, h, :]", 1)],
     ["test_attention_vs_sdpa_block_diagonal_and_packed"]),
    ("dy, dx order swapped in the merge group",
     [("h = merge * bh + dy\n                            w = merge * bw + dx",
       "h = merge * bh + dx\n                            w = merge * bw + dy", 1)],
     ["test_merge_order_golden_4x4", "test_strided_slice_identity"]),
    ("patch vector order: temporal slot before channel",
     [("x = x.transpose(0, 3, 5, 2, 1, 4, 6)", "x = x.transpose(0, 3, 5, 1, 2, 4, 6)", 1)],
     ["test_patch_embed_equals_conv3d"]),
    ("still frame not duplicated (second slot zero)",
     [("idx = [min(temporal * tt + tau, f - 1)", "idx = [min(temporal * tt + tau, f)", 1)],
     ["test_patch_embed_equals_conv3d"]),
    ("LayerNorm eps 1e-5 in every block", [("eps: float = 1e-6,\n                 groups", "eps: float = 1e-5,\n                 groups", 1),
                                          ("eps: float = 1e-6, groups", "eps: float = 1e-5, groups", 1)],
     ["test_block_ln2_uses_its_own_affine_and_eps"]),
    ("LayerNorm unbiased variance", [("var = (xc * xc).mean(axis=-1, keepdims=True)",
                                      "var = (xc * xc).sum(axis=-1, keepdims=True) / (x.shape[-1] - 1)", 1)],
     ["test_layer_norm_vs_torch_and_moments"]),
    ("q and k thirds swapped",
     [("q = qkv[:, 0 * d:1 * d]", "q = qkv[:, 1 * d:2 * d]", 1), ("k = qkv[:, 1 * d:2 * d]", "k = qkv[:, 0 * d:1 * d]", 1)],
     ["test_block_uniform_attention_special_case", "test_block_rope_on_q_and_k_closed_form_scores"]),
    ("k and v thirds swapped",
     [("k = qkv[:, 1 * d:2 * d]", "k = qkv[:, 2 * d:3 * d]", 1), ("v = qkv[:, 2 * d:3 * d]", "v = qkv[:, 1 * d:2 * d]", 1)],
     ["test_block_uniform_attention_special_case"]),
    ("post-norm attention half",
     [("z = z + o @ p[\"proj_w\"].T + p[\"proj_b\"]\n    a = layer_norm(z, p[\"ln2_w\"]",
       "z = layer_norm(z + o @ p[\"proj_w\"].T + p[\"proj_b\"], p[\"ln1_w\"], p[\"ln1_b\"], eps)\n    a = layer_norm(z, p[\"ln2_w\"]", 1)],
     ["test_block_is_pre_norm_scale_invariant"]),
    ("out-projection bias dropped (whole-block form)",
     [("z = z + o @ p[\"proj_w\"].T + p[\"proj_b\"]", "z = z + o @ p[\"proj_w\"].T", 1)],
     ["test_block_uniform_attention_special_case"]),
    ("merger activation QuickGELU instead of exact GELU",
     [("hmid = gelu_erf(y @ p[\"fc1_w\"].T", "hmid = quick_gelu(y @ p[\"fc1_w\"].T", 1)],
     ["test_merger_identity_special_case_and_shapes"]),
    ("merger without its LayerNorm",
     [("y = layer_norm(z.astype(dtype), p[\"ln_w\"], p[\"ln_b\"], eps).reshape(n // g, g * d)",
       "y = z.astype(dtype).reshape(n // g, g * d)", 1)],
     ["test_merger_identity_special_case_and_shapes"]),
    ("smart resize rounds half up instead of to even",
     [("h = max(factor, int(round(height / factor)) * factor)",
       "h = max(factor, int(math.floor(height / factor + 0.5)) * factor)", 1)],
     ["test_grid_bruteforce_properties"]),
    ("bf16 rounding ties away from zero",
     [("(u + 0x7FFF + ((u >> 16) & 1)) >> 16", "(u + 0x8000) >> 16", 1)],
     ["test_bf16_round_matches_torch"]),
    ("T = floor(F / 2)", [("t = -(-frames // temporal)", "t = max(1, frames // temporal)", 1)],
     ["test_grid_frames"]),
    ("fold uses only the first temporal tap",
     [("acc = acc + w[:, :, tau]", "acc = acc", 1)],
     ["test_fold_identity_equals_conv3d"]),
    ("int8 rounding half away from zero",
     [("q = np.clip(np.rint(w32 / scale[:, None])", "q = np.clip(np.trunc(w32 / scale[:, None] + np.copysign(0.5, w32))", 1)],
     ["test_quantize_i8_hand_example"]),
]


def _mutant(edits):
    with open(SRC) as fh:
        src = fh.read()
    for old, new, count in edits:
        assert src.count(old) == count, f"mutation anchor {old!r} found {src.count(old)} times, expected {count}"
        src = src.replace(old, new)
    mod = types.ModuleType("qv_oracle_mutant")
    mod.__file__ = SRC
    exec(compile(src, SRC + " (mutant)", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name,edits,catchers", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_mutation_is_caught(name, edits, catchers, monkeypatch):
    mod = _mutant(edits)
    monkeypatch.setattr(pins, "O", mod)
    caught = []
    for fn in catchers:
        try:
            getattr(pins, fn)()
        except Exception:  # an assertion or the mutant's own error: either way the pin rejects it
            caught.append(fn)
    assert caught, f"mutation '{name}' passed every pin named for it: {catchers}"


def test_unmutated_oracle_passes_the_catchers():
    """The catchers pass on the real oracle, so a failure above is the mutation's."""
    names = sorted({fn for _, _, cs in MUTATIONS for fn in cs})
    for fn in names:
        getattr(pins, fn)()
