"""bench.py's command-line contract that needs no GPU: the measured path runs on one GPU,
so --gpus above 1 ends at once with a one-line JSON error and exit status 2."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert p.returncode == 2
    line = json.loads(p.stdout.strip().splitlines()[-1])
    assert "error" in line and "--gpus must be 1" in line["error"]


def _bench():
    sys.path.insert(0, ROOT)
    import bench
    return bench


def test_kernel_fingerprint_ignores_comments_only(tmp_path):
    """The counter summary is keyed to the kernel sources' code text: an edited comment or
    blank line keeps the fingerprint, an edited statement changes it."""
    bench = _bench()
    base = "// header\nint f(int x) {  // trailing\n  /* block\n     comment */ return x + 1;\n}\n"
    variants = {
        "same_comment_edit": "// another header\nint f(int x) {\n\n  /* other */ return x + 1;   \n}\n",
        "code_edit": "// header\nint f(int x) {  // trailing\n  /* block\n     comment */ return x + 2;\n}\n",
    }
    p = tmp_path / "k.hip"
    p.write_text(base)
    ref = bench.code_text(str(p))
    assert "header" not in ref and "comment" not in ref and "return x + 1;" in ref
    p.write_text(variants["same_comment_edit"])
    assert bench.code_text(str(p)) == ref
    p.write_text(variants["code_edit"])
    assert bench.code_text(str(p)) != ref


def test_committed_counter_summary_matches_the_sources():
    """profiles/k_gateup_four_slots_mtp_zipf_counters.md was taken from the current kernel code,
    so the bench line reports its traffic (a code change without new counters would void it)."""
    bench = _bench()
    assert bench.counter_traffic("k_gateup", "four_slots_mtp_zipf") is not None
