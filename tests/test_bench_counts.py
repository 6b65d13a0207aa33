"""The bench's operation counts against brute force, its one-GPU guard and the
checks of its option combinations (host logic, no GPU)."""

import json
import os
import subprocess
import sys
from types import SimpleNamespace

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _pairs_brute(keys_per_block, N, causal):
    total = 0
    for i, keys in enumerate(keys_per_block):
        for r in range(128 * i, 128 * i + 128):
            total += sum(1 for k in keys if (k <= r or not causal))
    return total


def test_dense_ops():
    for causal in (True, False):
        p = SimpleNamespace(N=384, d=64, Hq=3, B=2, causal=causal)
        pairs = _pairs_brute([range(384)] * 3, 384, causal)
        assert bench.dense_algorithmic_ops(p) == 4.0 * 64 * pairs * 3 * 2


def test_sparse_pairs():
    rng = np.random.default_rng(0)
    N, nqb, mk = 512, 4, 5
    for causal in (True, False):
        idx = np.full((1, 2, nqb, mk), -1, np.int32)
        cnt = np.zeros((1, 2, nqb), np.int32)
        want = 0
        for h in range(2):
            blocks_i = []
            for i in range(nqb):
                nvis = 2 * i + 2 if causal else N // 64
                bl = sorted(rng.choice(nvis, min(nvis, 3), replace=False))
                idx[0, h, i, :len(bl)] = bl
                cnt[0, h, i] = len(bl)
                blocks_i.append([k for b in bl for k in range(64 * b, 64 * b + 64)])
            want += _pairs_brute(blocks_i, N, causal)
        assert bench.sparse_pairs(idx, cnt, causal) == want


def test_stripe_pairs():
    rng = np.random.default_rng(1)
    N, nqb, mk = 512, 4, 300
    for causal in (True, False):
        idx = np.full((2, 1, nqb, mk), -1, np.int32)
        cnt = np.zeros((2, 1, nqb), np.int32)
        want = 0
        for b in range(2):
            keys_i = []
            for i in range(nqb):
                nvis = 128 * i + 128 if causal else N
                keys = sorted(rng.choice(nvis, min(nvis, 150), replace=False))
                idx[b, 0, i, :len(keys)] = keys
                cnt[b, 0, i] = len(keys)
                keys_i.append(keys)
            want += _pairs_brute(keys_i, N, causal)
        assert bench.stripe_pairs(idx, cnt, causal) == want


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in json.loads(r.stdout.strip().splitlines()[-1])["error"]


def test_roofline_fractions():
    # 549.8 GOP (the 8K causal workload) in 0.5 ms: 1099.6 TOP/s
    ops = 4.0 * 128 * 8192 * 8193 / 2 * 32
    f = bench.roofline_fracs(ops, 0.5, 160e6)
    tops = ops / 0.5e-3 / 1e12
    assert abs(f["frac_int8"] - tops / 5000.0) < 1e-12
    # half the operations (P V) at the 16-bit peak
    assert abs(f["frac_fp16_pv_half"] - (tops / 2) / 2500.0) < 1e-12
    # blended bound 1 / (0.5/5000 + 0.5/2500) = 3333.3 TOP/s
    assert abs(bench.BLENDED_PEAK_TOPS - 10000.0 / 3.0) < 1e-9
    assert abs(f["frac_blended"] - tops / (10000.0 / 3.0)) < 1e-12
    assert abs(f["hbm_frac"] - 160e6 / 0.5e-3 / 8e12) < 1e-12
    assert bench.roofline_fracs(ops, 0.5, None)["hbm_frac"] is None


def test_option_combinations():
    # host-side checks of the step's options, before any GPU work
    from synthetic import make_config
    p2, _ = make_config(1)     # dense workload (no keep ratio of its own)

    def keep(*argv, p=p2):
        return bench.workload_keep(bench.parse(list(argv)), p)

    assert keep() is None
    assert keep("--promote") == (1, 10)
    assert keep("--promote", "--low4") == (1, 10)
    assert keep("--promote", "--patterns", "4", "4") == (1, 10)
    for bad in (["--low4"], ["--patterns", "4", "4"], ["--promote", "--adaptive", "0.02"],
                ["--promote", "--patterns", "65", "0"], ["--stripes", "1.0", "--patterns", "1", "1"]):
        with pytest.raises(SystemExit):
            keep(*bad)
