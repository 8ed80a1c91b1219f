"""The CPU oracle against its pins, and the pins against planted mistakes."""
import ast
import importlib.util
import os
import types

import pytest

import oracle.tsp_oracle as O
from oracle_pins import ALL_PINS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_pin(pin):
    pin(O)


# Each mutation plants one plausible mistake in a copy of the oracle's source
# text; at least one pin must then fail.
MUTATIONS = {
    "zigzag_wrong_partner": ("return (r, 2 * D - 1 - r)", "return (r, 2 * D - 2 - r)"),
    "zigzag_swapped_order": ("return (r, 2 * D - 1 - r)", "return (2 * D - 1 - r, r)"),
    "rms_eps_outside": ("np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)",
                        "(np.sqrt(np.mean(x * x, axis=-1, keepdims=True)) + eps)"),
    "rms_no_gain": ("+ eps) * np.asarray(g, F64)", "+ eps)"),
    "silu_sign": ("return z / (1.0 + np.exp(-z))", "return z / (1.0 + np.exp(z))"),
    "attn_no_scale": ("scale = 1.0 / math.sqrt(d)", "scale = 1.0"),
    "attn_mask_excludes_diagonal": ("np.arange(kmax)[None, :] > pb[:, None]",
                                    "np.arange(kmax)[None, :] >= pb[:, None]"),
    "attn_no_mask": ("sc[np.arange(kmax)[None, :] > pb[:, None]] = -np.inf", "pass"),
    "attn_no_normalise": ("/ e.sum(axis=1, keepdims=True)", ""),
    "wo_transposed": ("return xs[rows] + a @ np.asarray(w.wo, F64)",
                      "return xs[rows] + a @ np.asarray(w.wo, F64).T"),
    "no_attention_residual": ("return xs[rows] + a @ np.asarray(w.wo, F64)",
                              "return a @ np.asarray(w.wo, F64)"),
    "gate_on_wrong_branch": ("(silu(n @ np.asarray(w1, F64)) * (n @ np.asarray(w3, F64)))",
                             "(silu(n @ np.asarray(w3, F64)) * (n @ np.asarray(w1, F64)))"),
    "no_mlp_residual": ("return x1 + swiglu_mlp(rmsnorm(x1, w.g2, eps), w.w1, w.w3, w.w2)",
                        "return swiglu_mlp(rmsnorm(x1, w.g2, eps), w.w1, w.w3, w.w2)"),
    "norm2_on_input": ("    return mlp_block(x1, w, eps)\n",
                       "    return x1 + swiglu_mlp(rmsnorm(np.asarray(x_full, F64)[rows], w.g2, eps),"
                       " w.w1, w.w3, w.w2)\n"),
    "head_slice_off_by_one": ("k_t = rope(n1 @ np.asarray(w.wk[:, kc], F64)",
                              "k_t = rope(n1 @ np.asarray(np.roll(w.wk, 1, axis=1)[:, kc], F64)"),
    "rope_turns_clockwise": ("out[:, 0::2] = u * c - v * s\n    out[:, 1::2] = u * s + v * c",
                             "out[:, 0::2] = u * c + v * s\n    out[:, 1::2] = -u * s + v * c"),
    "rope_frequency_exponent": ("** (-2.0 * np.arange(d // 2) / d)", "** (-1.0 * np.arange(d // 2) / d)"),
    "rope_query_local_positions": ("rope(q[:, c], rows, rope_theta)",
                                   "rope(q[:, c], np.arange(rows.size), rope_theta)"),
    "rope_keys_not_rotated": ("k_t = rope(n1 @ np.asarray(w.wk[:, kc], F64), np.arange(P), rope_theta)",
                              "k_t = n1 @ np.asarray(w.wk[:, kc], F64)"),
    "gqa_heads_interleaved": ("kc = slice((t // grp) * d, (t // grp + 1) * d)",
                              "kc = slice((t % (n_heads // grp)) * d, (t % (n_heads // grp) + 1) * d)"),
    "fold_rope_local_positions": ("return np.concatenate([rope(m[:, t * d:(t + 1) * d], p, rope_theta)",
                                  "return np.concatenate([rope(m[:, t * d:(t + 1) * d], np.arange(p.size), rope_theta)"),
    "pairs_count_strict": ("np.sum(zigzag_positions(S, D, r) + 1)", "np.sum(zigzag_positions(S, D, r))"),
    "flops_missing_o_proj": ("return 8 * T * h * h + 6", "return 6 * T * h * h + 6"),
    "fold_missing_partial": ("y[r] += o @ wo_j", "y[r] = o @ wo_j"),
    "ring_skips_last": ("for t in range(D):                  # ring step t",
                        "for t in range(D - 1):              # ring step t"),
}


def _load_mutant(old, new):
    path = os.path.join(ROOT, "oracle", "tsp_oracle.py")
    src = open(path).read()
    assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
    src = src.replace(old, new)
    ast.parse(src)
    mod = types.ModuleType("tsp_oracle_mutant")
    exec(compile(src, "<mutant>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_mutation(name):
    mutant = _load_mutant(*MUTATIONS[name])
    failed = []
    for pin in ALL_PINS:
        try:
            pin(mutant)
        except (AssertionError, ValueError, IndexError) as e:
            failed.append(pin.__name__)
    assert failed, f"no pin caught mutation {name}"


def test_oracle_is_independent_of_product():
    """The oracle imports nothing of the HIP-side package, and the package
    imports nothing of the oracle."""
    def imports(path):
        tree = ast.parse(open(path).read())
        names = set()
        for n in ast.walk(tree):
            if isinstance(n, ast.Import):
                names |= {a.name.split(".")[0] for a in n.names}
            elif isinstance(n, ast.ImportFrom) and n.module:
                names.add(n.module.split(".")[0])
        return names

    for f in os.listdir(os.path.join(ROOT, "oracle")):
        if f.endswith(".py"):
            assert "folded_tensor_sequence_rank_amd" not in imports(os.path.join(ROOT, "oracle", f))
    pkg = os.path.join(ROOT, "folded_tensor_sequence_rank_amd")
    for dp, _, fs in os.walk(pkg):
        for f in fs:
            if f.endswith(".py"):
                assert "oracle" not in imports(os.path.join(dp, f)), f
