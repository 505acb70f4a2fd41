"""bench.py's command-line contract that needs no GPU: more than one GPU is
refused with a message and a non-zero status, before anything is imported
that would touch a device."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args, env=None):
    e = dict(os.environ)
    e.update(env or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True,
                          text=True, env=e, timeout=120)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_launcher_world_size_is_refused():
    r = _run(env={"WORLD_SIZE": "4"})
    assert r.returncode == 2
    assert "WORLD_SIZE 4" in r.stderr


def test_tolerance_ratio_fails_on_nan():
    """The benchmark's pre-timing check: a NaN or an infinity where the
    oracle is finite fails it (a plain max() would skip a NaN)."""
    import numpy as np
    sys.path.insert(0, ROOT)
    import bench
    ref = np.array([1.0, 2.0, 3.0])
    assert bench.tol_ratio(ref + 0.001, ref) <= 1
    assert bench.tol_ratio(np.array([1.0, np.nan, 3.0]), ref) == float("inf")
    assert bench.tol_ratio(np.array([1.0, np.inf, 3.0]), ref) == float("inf")
    assert bench.tol_ratio(np.array([1.0, 2.5, 3.0]), ref) > 1


def test_profile_dispatches_are_assigned_to_calls():
    """rocprofv3 rows of a --profile run are attributed to the calls of a
    step by dispatch order: build, shrink (one or two kernels), then one
    expand per output."""
    sys.path.insert(0, ROOT)
    import bench
    names = ["build_segments_kernel", "shrink_kernel", "shrink_reduce_kernel", "expand_kernel<1>",
             "expand_kernel<2>", "at::neg_kernel", "build_segments_kernel", "bgmv_shrink_kernel",
             "expand_kernel<1>", "expand_kernel<2>"]
    rows = [{"Dispatch_Id": str(i + 1), "Kernel_Name": n} for i, n in enumerate(names)]
    units = [u for u, _ in bench.assign_units(list(reversed(rows)), 2)]
    assert units == ["build", "shrink", "shrink", "expand[0]", "expand[1]", None,
                     "build", "shrink", "expand[0]", "expand[1]"]
    assert [u for u, _ in bench.assign_units(rows[:4], 1)] == ["build", "shrink", "shrink", "expand"]
    # the argument pool's one-time build forms no step; a split expand's
    # per-token launch belongs to the call whose tile launch precedes it
    names = ["build_segments_kernel", "build_segments_kernel", "shrink_kernel", "expand_kernel<1>",
             "bgmv_expand_fast_kernel<1>", "expand_kernel<2>"]
    rows = [{"Dispatch_Id": str(i + 1), "Kernel_Name": n} for i, n in enumerate(names)]
    got = bench.assign_units(rows, 2, with_step=True)
    assert [u for u, _, _ in got] == ["build", "build", "shrink", "expand[0]", "expand[0]", "expand[1]"]
    assert bench.steps_of(got) == {"build": 2, "shrink": 1, "expand[0]": 1, "expand[1]": 1}
