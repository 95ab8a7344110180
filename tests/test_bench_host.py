"""Host logic of bench.py (no GPU): the kernel-source hash that ties the committed counter figures to the code
they were taken with."""

import json
import sys

import bench

WORKLOADS = ("decode_bf16", "prefill_bf16", "skew_prefill_bf16", "prefill32k_bf16", "decode_fp8", "ep_share_fp8",
             "tiny_fp32")


def test_code_tokens_ignore_comments_and_layout():
    a = "int f(int x) {\n  return x + 1;  // one more\n}\n"
    b = "/* adds one */ int f(int x) { return x + 1; }"
    assert bench.code_tokens(a) == bench.code_tokens(b)


def test_code_tokens_keep_code_and_literals():
    assert bench.code_tokens("int y = 2;") != bench.code_tokens("int y = 3;")
    s = "const char* p = \"a // b /* c */\"; char q = '\"'; char r = '\\'';"
    assert bench.code_tokens(s) == s


def test_committed_traffic_matches_the_current_kernels():
    """Every committed gate/up counter summary was taken with the GEMM code as it stands, so the bench
    reports non-null roofline traffic for every workload; a change to that code needs the counters again."""
    missing = [w for w in WORKLOADS if bench.committed_traffic(w) is None]
    assert not missing, f"counter summaries stale or missing for {missing} (hash {bench.kernel_source_hash()})"


def test_more_than_one_gpu_is_refused_with_a_message(monkeypatch, capsys):
    """One GPU only: --gpus N > 1, or a launch with several ranks, exits with status 2 and a JSON message
    before anything touches a GPU."""
    monkeypatch.setattr(sys, "argv", ["bench.py", "--gpus", "2"])
    assert bench.main() == 2
    msg = json.loads(capsys.readouterr().out.strip())
    assert "one GPU" in msg["error"]
    monkeypatch.setattr(sys, "argv", ["bench.py"])
    monkeypatch.setenv("WORLD_SIZE", "8")
    assert bench.main() == 2
    assert "one GPU" in json.loads(capsys.readouterr().out.strip())["error"]
