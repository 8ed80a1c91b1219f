"""Host-side checks of the benchmark: its FLOP model, and that only its CPU
baseline leg touches the oracle."""
import ast
import os
import sys

import oracle.tsp_oracle as O
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_flop_model_matches_oracle_closed_form():
    for name in ("tiny_fp32", "7b_s16k", "7b_s64k", "7b_s128k", "7b_s16k_b4"):
        cfg = synth.get_config(name)
        for r in sorted({0, cfg.ranks[0], cfg.fold - 1}):
            got = sum(bench.flops_per_step(cfg, r).values())
            assert got == cfg.batch * O.flops_rank(cfg.hidden, cfg.ffn, cfg.seq, cfg.fold, r)


def test_flop_model_grouped_kv():
    """K and V projections shrink with the K/V heads; nothing else changes."""
    mha = synth.get_config("7b_s64k")
    gqa = synth.get_config("7b_gqa8_rope_s64k")
    a, b = bench.flops_per_step(mha, 3), bench.flops_per_step(gqa, 3)
    T, h = mha.local_tokens, mha.hidden
    assert a["qkv"] - b["qkv"] == 2 * T * h * 2 * (h - 8 * 128)
    assert {k: v for k, v in a.items() if k != "qkv"} == {k: v for k, v in b.items() if k != "qkv"}


def test_only_cpu_baseline_imports_the_oracle():
    tree = ast.parse(open(os.path.join(ROOT, "bench.py")).read())
    users = set()
    for fn in ast.walk(tree):
        if isinstance(fn, ast.FunctionDef):
            for node in ast.walk(fn):
                mods = ([a.name for a in node.names] if isinstance(node, ast.Import) else
                        [node.module or ""] if isinstance(node, ast.ImportFrom) else [])
                if any(m.split(".")[0] == "oracle" for m in mods):
                    users.add(fn.name)
    top = [n for n in tree.body if isinstance(n, (ast.Import, ast.ImportFrom))]
    assert not any("oracle" in ast.dump(n) for n in top)
    assert users == {"cpu_baseline"}, users


def test_bench_refuses_more_than_one_gpu():
    """One GPU's share is the measurement; --gpus N > 1 exits with a message
    before touching any device."""
    import subprocess
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "single MI355X" in r.stderr and r.stdout == ""
