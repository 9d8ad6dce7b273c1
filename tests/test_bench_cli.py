"""bench.py without a GPU: the one-GPU refusal, the measurement modes it
offers, and the algorithmic byte and FLOP counts behind its roofline figures,
counted here element by element from the shapes."""

import json
import os
import subprocess
import sys

import numpy as np

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BF16 = 2  # bytes


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["requested_gpus"] == 2 and "one GPU" in line["error"]


def test_measurement_modes_are_offered():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--help"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 0
    for flag in ("--steps", "--warmup", "--no-cpu-baseline", "--copy-probe", "--gemm-probe", "--serving-gemm-probe",
                 "--head-gemm-probe"):
        assert flag in r.stdout


def test_attention_bytes_count_every_tensor_once():
    # Per cached token: K and V of 8 KV heads x 128 dims.  Per sequence: the
    # queries (32 heads x 8 positions x 128), the output (same shape), and the
    # block's own K and V (8 heads x 8 positions x 128 each).
    lens = np.array([1, 16, 8200])
    per_token = 2 * 8 * 128 * BF16
    per_seq = 2 * 32 * 8 * 128 * BF16 + 2 * 8 * 8 * 128 * BF16
    assert bench.attn_bytes(lens) == int(lens.sum()) * per_token + len(lens) * per_seq
    # The serving workload: 64 sequences of 8192 cached tokens plus 302 new rows.
    assert bench.attn_bytes(np.full(64, 8192) + np.bincount(np.arange(302) % 64, minlength=64)) == 2159206400


def test_verify_bytes_follow_the_rows_each_decision_reads():
    V = 262144
    temp = np.array([0.0, 0.7, -1.0, 1.0])
    greedy_rows, sampled_rows = 8, 7 + 7
    assert bench.verify_bytes(temp) == (2 * greedy_rows + 2 * sampled_rows) * V * BF16


def test_fusion_flops_and_bytes():
    M = 302
    w_c = 2560 * (5 * 2560)
    w_kv = (5 * 2 * 8 * 128) * 2560
    flops, nbytes = bench.fuse_flops_bytes(M)
    assert flops == 2 * M * (w_c + w_kv)
    # Weights once, the five captured rows in, K and V of every layer out.
    assert nbytes == (w_c + w_kv) * BF16 + M * (5 * 2560 + 5 * 2 * 8 * 128) * BF16


def test_every_name_a_function_reads_is_defined():
    # bench.py's measurement functions only run on a GPU; this catches a name
    # read in one of them that nothing defines (a local lost in an edit) on
    # the CPU: locals, parameters, comprehension targets, module globals and
    # builtins are the names a function may read.
    import ast
    import builtins
    tree = ast.parse(open(os.path.join(ROOT, "bench.py")).read())
    known = set(dir(builtins))
    for node in tree.body:
        if isinstance(node, (ast.FunctionDef, ast.ClassDef)):
            known.add(node.name)
        elif isinstance(node, (ast.Import, ast.ImportFrom)):
            known.update((a.asname or a.name).split(".")[0] for a in node.names)
        elif isinstance(node, (ast.Assign, ast.AnnAssign)):
            for t in node.targets if isinstance(node, ast.Assign) else [node.target]:
                known.update(n.id for n in ast.walk(t) if isinstance(n, ast.Name))
    missing = []
    for fn in (n for n in tree.body if isinstance(n, ast.FunctionDef)):
        local = set()
        for n in ast.walk(fn):
            if isinstance(n, (ast.FunctionDef, ast.Lambda)):
                args = n.args
                local.update(a.arg for a in args.args + args.kwonlyargs)
                local.update(a.arg for a in (args.vararg, args.kwarg) if a)
                if isinstance(n, ast.FunctionDef):
                    local.add(n.name)
            elif isinstance(n, ast.Name) and isinstance(n.ctx, (ast.Store, ast.Del)):
                local.add(n.id)
            elif isinstance(n, (ast.Import, ast.ImportFrom)):
                local.update((a.asname or a.name).split(".")[0] for a in n.names)
            elif isinstance(n, ast.ExceptHandler) and n.name:
                local.add(n.name)
        missing += [(fn.name, n.lineno, n.id) for n in ast.walk(fn)
                    if isinstance(n, ast.Name) and isinstance(n.ctx, ast.Load) and n.id not in local | known]
    assert not missing, missing
