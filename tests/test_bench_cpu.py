"""bench.py's contract checks that need no GPU: more than one GPU is refused
with a message and a nonzero status, before anything touches a device."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2", "--steps", "1"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_bench_help_lists_the_workloads():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--help"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 0
    for w in ("llama8b", "layerset28", "muonbp", "grasp", "fp32_256x512"):
        assert w in r.stdout


def test_timer_and_call_steps_split_the_timed_steps():
    """The per-kernel timer runs on the even-numbered timed steps, whole-call
    figures come from the odd ones; together they are every step once, and a
    20-step MuonBP region (P = 5) keeps its 4 : 1 block/full mix in both."""
    sys.path.insert(0, ROOT)
    import bench
    for n in range(1, 41):
        t, c = bench.timer_steps(n), bench.call_steps(n)
        assert t and c
        if n >= 2:
            assert sorted(t + c) == list(range(n)) and not set(t) & set(c)
        else:
            assert t == c == [0]
    full = [(k + 1) % 5 == 0 for k in range(20)]
    for idx in (bench.timer_steps(20), bench.call_steps(20)):
        assert sum(full[k] for k in idx) == 2 and len(idx) == 10
