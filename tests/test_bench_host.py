"""bench.py's host-side contract, without a GPU: it measures one GPU only, so
any other --gpus exits at once (status 2) with a message saying so, before
importing torch or touching a device; and two-word numerics are refused for
the workloads that do not have them (the shared-expert block, and the
mixture's separate one-word calls)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=120)


def test_more_than_one_gpu_is_refused():
    for n in ("2", "8"):
        p = run("--gpus", n)
        assert p.returncode == 2
        assert "one GPU" in p.stderr and p.stdout == ""


def test_two_words_refused_where_not_built():
    import bench
    for name, sep in (("moe_shared_d2048_dff1408_e60_k4_s5632", False), ("moe_d2048_dff768_e128_k8", True)):
        try:
            bench.make_workload(name, "x2", 1, separate=sep)
        except SystemExit as e:
            assert "two-word" in str(e)
        else:
            raise AssertionError("x2 accepted for %s" % name)


def test_suite_names_every_config_in_its_numerics():
    # one default run measures every configured workload (the GEMV, the norm
    # + GEMV, both mixture shapes, the chunk, the shared-expert variant) in
    # each numerics it is built for
    import bench
    import synthetic
    names = {n for n, _ in bench.SUITE} | {bench.DEFAULT_WORKLOAD}
    assert names == set(synthetic.CONFIGS)
    for name, act in bench.SUITE:
        assert act in bench.ACT_CODE
        assert (name, act) != (bench.DEFAULT_WORKLOAD, "int8")  # the headline itself
    for name in ("norm_gemv_2048x4096", "moe_d4096_dff14336_e8_k2"):
        assert {a for n, a in bench.SUITE if n == name} == {"int8", "f32", "x2"}


def test_percentiles():
    import bench
    assert bench._pct([5.0, 1.0, 3.0, 2.0, 4.0], 0.5) == 3.0
    assert bench._pct(list(range(100)), 0.1) == 10 and bench._pct(list(range(100)), 0.9) == 90
