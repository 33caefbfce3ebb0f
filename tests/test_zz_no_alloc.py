"""The sweep that allocates nothing (bq_token_sweep_noalloc: its plan goes to
the library's fixed device scratch) against the planned sweep
(bq_sweep_create + bq_token_sweep) on the same inputs, bit for bit: two calls
in a row, the second with a smaller list, so the scratch is reused with
different contents."""
import numpy as np
import pytest

import synth
from gpu_util import log, torch
from pins import same_bits

pytestmark = pytest.mark.gpu

Q1, Q2 = 1, 2


def _outputs(sw, entries, which, call):
    """Run `call` on the entries `which` (their y replaced by fresh NaN-filled
    tensors); returns those outputs as numpy arrays."""
    t = torch()
    ys = [t.full((entries[i][0].rows,), float("nan"), dtype=t.float32, device="cuda") for i in which]
    call([(entries[i][0], entries[i][1], y) for i, y in zip(which, ys)])
    t.cuda.synchronize()
    return [y.cpu().numpy() for y in ys]


def _check(fmt, shapes, seed, qa, second):
    import ternary_quantized_gemv_amd as bq
    from ternary_quantized_gemv_amd.staging import StagedSweep
    t = torch()
    canon = [synth.blocks(fmt, r, c, seed, i) for i, (_, r, c) in enumerate(shapes)]
    x = [synth.activation(c, seed, 1000 + i) for i, (_, _, c) in enumerate(shapes)]
    sw = StagedSweep(fmt, canon, shapes, x, qa, keep_host=False)
    try:
        sw.run()  # quantizer + planned sweep
        t.cuda.synchronize()
        y_ref = sw.y.cpu().numpy()
        ref = [y_ref[int(sw.yoff[i]):int(sw.yoff[i + 1])] for i in range(len(shapes))]
        first = list(range(len(shapes)))
        log(f"no-alloc sweep fmt={fmt}: first call, {len(first)} products")
        got = _outputs(sw, sw.entries, first, bq.bq_token_sweep_noalloc)
        for i, g in zip(first, got):
            assert same_bits(g, ref[i]), f"first call, product {i} ({shapes[i][0]})"
        log(f"no-alloc sweep fmt={fmt}: second call, {len(second)} products")
        got = _outputs(sw, sw.entries, second, bq.bq_token_sweep_noalloc)
        for i, g in zip(second, got):
            assert same_bits(g, ref[i]), f"second call, product {i} ({shapes[i][0]})"
        # and the planned sweep of the smaller list agrees too
        def planned(ents):
            plan = bq.bq_sweep_create(ents)
            bq.bq_token_sweep(plan)
            t.cuda.synchronize()
            plan.destroy()
        got2 = _outputs(sw, sw.entries, second, planned)
        assert all(same_bits(a, b) for a, b in zip(got, got2))
    finally:
        sw.close()


def test_noalloc_decode_token_then_smaller():
    """The full Q1_0 decode token (253 products), then 9 of them."""
    shapes = synth.decode_sweep_shapes()
    _check(Q1, shapes, 101, 128, [0, 1, 2, 3, 4, 5, 6, 100, 252])


def test_noalloc_q2_decode_token_then_smaller():
    """The full Q2_0 decode token, whose products of several table chunks make
    work items of two tiles per wavefront, then 5 of them."""
    shapes = synth.decode_sweep_shapes()
    _check(Q2, shapes, 103, 128, [0, 3, 6, 100, 252])


def test_noalloc_mix_then_smaller():
    """A ragged Q2_0 mix (one block, partial and several table chunks, ragged
    rows) at qa 64, then two of its products."""
    shapes = [("a", 100, 33 * 64), ("b", 64, 64), ("c", 700, 4096), ("d", 130, 96 * 64), ("e", 65, 40 * 64),
              ("f", 3, 128), ("g", 2000, 2048)]
    _check(Q2, shapes, 102, 64, [3, 5])


def test_noalloc_refuses_before_launch():
    import ternary_quantized_gemv_amd as bq
    t = torch()
    w = bq.Weights.upload(Q1, synth.blocks(Q1, 64, 256, 3), 64, 256)
    a = bq.Act(t.zeros(256, dtype=t.int8, device="cuda"), t.ones(2, device="cuda"), 256, 128)
    y = t.full((64,), 5.0, device="cuda")
    with pytest.raises(bq.BQError) as e:
        bq.bq_token_sweep_noalloc([(w, a, y)] * 1025)
    assert "1024" in str(e.value)
    t.cuda.synchronize()
    assert bool((y == 5.0).all())
