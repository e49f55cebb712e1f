"""bench.py's command line on the CPU: the one-GPU contract and the help text
(no GPU work; both paths return before torch is imported)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=120, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    for n in ("2", "8"):
        r = _run("--gpus", n)
        assert r.returncode == 2
        assert "one GPU only" in r.stderr and f"--gpus {n}" in r.stderr
        assert r.stdout == ""  # no JSON line


def test_help_lists_the_workloads():
    r = _run("--help")
    assert r.returncode == 0
    for w in ("prefill-8k-bf16-hbm", "prefill-16k-fp8-hbm", "prefill-8k-bf16-host", "decode-256",
              "spec-decode-256x4", "select-rows-8k"):
        assert w in r.stdout


def _bench_module():
    import importlib.util
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_lookup_byte_counts():
    """Algorithmic bytes of one lookup, worked by hand: per (token, head) the table row read plus the
    1 KiB bf16 row written, plus the tokens and query_start_loc (8k prefill: 8192 x 8 rows of 512, 13
    requests; 16k fp8: 16384 x 16 rows of 512 code bytes and a 4-byte scale, 30 requests)."""
    b = _bench_module()
    assert b.lookup_bytes_of("bf16", 8192, 8, 512, 13) == 8192 * 8 * (1024 + 1024) + 8192 * 4 + 14 * 4
    assert b.lookup_bytes_of("fp8", 16384, 16, 512, 30) == 16384 * 16 * (516 + 1024) + 16384 * 4 + 31 * 4
    assert b.lookup_bytes_of("nvfp4", 8192, 8, 512, 13) == 8192 * 8 * (256 + 32 + 1024) + 8192 * 4 + 14 * 4
    assert b.row_in_bytes("fp8-global", 512) == 512


def test_traffic_record_matches_the_kv_proj_source():
    """The bench line's kv_proj traffic comes from a committed counter record keyed by the kernel
    source's hash; the record must be the current source's, so the line carries a figure."""
    b = _bench_module()
    assert b.recorded_traffic("prefill-8k-bf16-hbm") is not None
    assert b.recorded_traffic("decode-256") is None  # recorded for the 8k prefill only
