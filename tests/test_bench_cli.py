"""bench.py's command-line contract that needs no GPU: one GPU only."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr or "single MI355X" in r.stderr
    assert r.stdout == ""


def _bench():
    sys.path.insert(0, ROOT)
    import bench
    return bench


def test_spread_takes_p10_median_p90():
    b = _bench()
    assert b.spread([float(v) for v in range(10, 0, -1)]) == [2.0, 6.0, 10.0]
    assert b.spread([3.5]) == [3.5, 3.5, 3.5]


def test_load_profile_recovers_a_zipf_slope():
    """Loads proportional to rank^-a give slope -a over ranks 1-64; the
    top five and the minimum are reported over the mean."""
    b = _bench()
    import numpy as np
    a = 1.2
    loads = 10000.0 * np.arange(1, 257, dtype=np.float64) ** -a
    prof = b.load_profile(np.random.default_rng(0).permutation(loads), loads.mean())
    assert abs(prof["loglog_slope_ranks_1_64"] + a) < 1e-9
    assert prof["top5_over_mean"][0] == round(loads[0] / loads.mean(), 3)
    assert prof["min_over_mean"] == round(loads[-1] / loads.mean(), 3)
    flat = b.load_profile(np.full(256, 7.0), 7.0)
    assert flat["loglog_slope_ranks_1_64"] == 0.0 and flat["top5_over_mean"] == [1.0] * 5


def test_decode_bytes_counts_touched_experts_once():
    """Bytes of one decode step: every touched routed expert's three weight
    matrices once (17/32 byte per value in MXFP4), the shared experts, the
    fp32 router and the activations in and out."""
    b = _bench()
    import numpy as np
    from sparse_mixture_experts_04_amd import configs
    c = configs.get("C")
    counts = np.zeros(c.E, dtype=np.int64)
    counts[:200] = 1
    nbytes, n = b.decode_bytes(c, counts)
    per = 3 * c.d * c.F * 2
    assert n == 200
    assert nbytes == 200 * per + c.S * per + (c.E + c.S) * c.d * 4 + 2 * c.T * c.d * 2
    f = configs.get("Cfp4")
    nb4, n4 = b.decode_bytes(f, counts)
    assert n4 == 200
    assert nb4 == int(200 * 3 * f.d * f.F * (0.5 + 1 / 32) + f.S * per
                      + (f.E + f.S) * f.d * 4 + 2 * f.T * f.d * 2)
