"""Host-side checks that need no GPU: the benchmark's one-GPU contract and the
dependency order of the decode chain."""
import os
import subprocess
import sys

import synth
from ternary_quantized_gemv_amd.staging import chain_groups

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr and r.stdout == ""


def test_chain_groups_cover_the_token_in_dependency_order():
    shapes = synth.decode_sweep_shapes()
    groups = chain_groups(36)
    assert len(groups) == 4 * 36 + 1 == 145
    seen, produced = [], set()
    for prods, src in groups:
        cols = {shapes[p][2] for p in prods}
        assert len(cols) == 1                      # a group shares one input length
        if src >= 0:
            assert src in produced                 # its input is an earlier group's output
            assert shapes[src][1] == cols.pop()    # of the right length
        else:
            assert not seen                        # only the first group reads the token's input
        seen += prods
        produced.update(prods)
    assert sorted(seen) == list(range(len(shapes)))  # every product exactly once
    names = [[shapes[p][0].split(".")[-1] for p in prods] for prods, _ in groups]
    assert names[:4] == [["q", "k", "v"], ["o"], ["gate", "up"], ["down"]]
    assert names[4:8] == names[:4] and len(names[-1]) == 1 and shapes[groups[-1][0][0]][1] == 151936


def test_parity_check_fails_closed():
    """The GPU tests' bar refuses any difference in the bits: one ulp up or
    down, a sign of zero, a NaN, a shape change -- and passes only identity."""
    import numpy as np
    import pytest
    from gpu_util import assert_parity

    g = np.random.default_rng(5)
    ref = g.standard_normal(4096).astype(np.float32)
    ref[7] = 0.0
    assert_parity(ref.copy(), ref, "identical")
    for i in (0, 1000, 4095):
        for direction in (np.inf, -np.inf):
            bad = ref.copy()
            bad[i] = np.nextafter(bad[i], np.float32(direction))
            with pytest.raises(AssertionError):
                assert_parity(bad, ref, f"one ulp at {i}")
    for bad_value in (np.float32(-0.0), np.float32(np.nan)):
        bad = ref.copy()
        bad[7] = bad_value
        with pytest.raises(AssertionError):
            assert_parity(bad, ref, "zero sign or NaN")
    with pytest.raises(AssertionError):
        assert_parity(ref[:-1], ref, "shape")
