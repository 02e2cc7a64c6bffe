"""Host logic of bench.py (no GPU): the per-role naming of a pass's launches
in a rocprofv3 kernel trace, for the skinny (up to 32 rows) and the wide
(batched) paths, the gpus guard, and the algorithmic W12 byte count."""

import csv
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

SKINNY_LAYER = ["void tvp::w12_skinny_kernel<32, 1, 2, 4>(tvp::GemmArgs)",
                "void tvp::tree_attn_kernel<128, 2>(tvp::AttnArgs)",
                "void tvp::w12_skinny_kernel<32, 1, 2, 16>(tvp::GemmArgs)",
                "tvp::resid_norm_kernel(float const*)",
                "void tvp::w12_skinny_kernel<32, 2, 2, 3>(tvp::GemmArgs)",
                "void tvp::w12_skinny_kernel<32, 1, 2, 16>(tvp::GemmArgs)",
                "tvp::resid_norm_kernel(float const*)"]
WIDE_LAYER = ["void tvp::w12_wide_kernel<6, 1, 3>(tvp::GemmArgs)", "tvp::w12_wide_fixup_kernel(tvp::GemmArgs)",
              "void tvp::tree_attn_kernel<128, 2>(tvp::AttnArgs)",
              "void tvp::w12_wide_kernel<6, 1, 3>(tvp::GemmArgs)", "tvp::resid_norm_kernel(float const*)",
              "void tvp::w12_wide_kernel<6, 1, 3>(tvp::GemmArgs)", "tvp::w12_wide_fixup_kernel(tvp::GemmArgs)",
              "void tvp::w12_wide_kernel<6, 1, 3>(tvp::GemmArgs)", "tvp::resid_norm_kernel(float const*)"]
HEAD = ["tvp::tree_prep_kernel(int const*)", "tvp::rope_table_kernel(int const*)", "tvp::embed_kernel(int const*)",
        "tvp::resid_norm_kernel(float const*)"]


def _trace(tmp_path, names):
    p = tmp_path / "x_kernel_trace.csv"
    with open(p, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        for i, n in enumerate(names):
            w.writerow([n, i * 10_000, i * 10_000 + 1000 * (i % 7 + 1)])
    return str(p)


def test_skinny_pass_roles(tmp_path):
    tail = ["void tvp::w12_skinny_kernel<32, 2, 2, 5>(tvp::GemmArgs)", "tvp::argmax_finalize_kernel(x)",
            "tvp::accept_kernel(x)", "tvp::kv_commit_kernel(x)",
            # the benchmark's own gate/up timing launches follow the pass and are not pass roles
            "void tvp::w12_skinny_kernel<32, 2, 2, 3>(tvp::GemmArgs)",
            "void tvp::w12_skinny_kernel<32, 2, 2, 3>(tvp::GemmArgs)"]
    roles = bench.pass_roles(_trace(tmp_path, HEAD + SKINNY_LAYER * 3 + tail))
    assert {r: len(v) for r, v in roles.items()} == {
        "QKV GEMM + RoPE + KV write": 3, "tree attention": 3, "O GEMM (K slices)": 3,
        "residual + norm after O": 3, "gate/up GEMM": 3, "down GEMM (K slices)": 3,
        "residual + norm after down": 3, "norm (first or final)": 1, "LM head + argmax": 1,
        "LM-head argmax finalize": 1, "tree preparation": 1, "RoPE table": 1, "embedding": 1,
        "acceptance walk": 1, "KV commit": 1}
    # durations are end - start in microseconds, in launch order
    n_head = len(HEAD)
    assert roles["QKV GEMM + RoPE + KV write"][0] == ((n_head % 7) + 1)


def test_wide_pass_roles(tmp_path):
    tail = ["void tvp::w12_wide_kernel<6, 1, 3>(tvp::GemmArgs)", "tvp::w12_wide_fixup_kernel(tvp::GemmArgs)",
            "tvp::argmax_finalize_kernel(x)", "tvp::accept_kernel(x)"]
    roles = bench.pass_roles(_trace(tmp_path, HEAD + WIDE_LAYER * 2 + tail))
    assert {r: len(v) for r, v in roles.items()} == {
        "wide QKV GEMM": 2, "wide QKV fix-up (RoPE, KV write)": 2, "tree attention": 2,
        "wide O GEMM (split sums)": 2, "residual + norm after O": 2, "wide gate/up GEMM": 2,
        "wide gate/up fix-up (SwiGLU)": 2, "wide down GEMM (split sums)": 2, "residual + norm after down": 2,
        "norm (first or final)": 1, "wide LM head": 1, "wide LM-head fix-up (argmax keys)": 1,
        "LM-head argmax finalize": 1, "tree preparation": 1, "RoPE table": 1, "embedding": 1,
        "acceptance walk": 1}


def test_algorithmic_w12_bytes():
    # planes (k + ceil(k/2) bytes per channel), base byte, CSR pointers (n + 1), 4 bytes per escape
    assert bench.w12_algorithmic_bytes(2, 3, 5) == 2 * 3 + 2 * 2 + 2 + 4 * 3 + 4 * 5


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, cwd=ROOT, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stdout
