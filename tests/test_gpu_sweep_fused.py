"""The token sweep that quantizes its f32 activations inside the launch
(bq_sweep_create_x, StagedSweep.sweep_fused): every output must equal the
oracle's quantize-then-product on small mixes (ragged rows, partial and
several table chunks, an all-zero activation block and exact ties, every qa,
both formats), and on the full decode token the two-launch path
(quantizer + bq_token_sweep) bit for bit -- and, on the full decode token
of both formats, the oracle on every output and the two-launch path."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import log, paired_walk_shapes, torch
from pins import same_bits

pytestmark = pytest.mark.gpu

Q1, Q2 = 1, 2
THREADS = 16

# ragged rows, one block, 33 blocks (a partial second chunk), 96 blocks (three
# chunks), 40 blocks (32 + 8), two blocks
MIX = [("a", 100, 33 * 128), ("b", 64, 128), ("c", 700, 4096), ("d", 130, 96 * 128), ("e", 65, 40 * 128),
       ("f", 3, 256)]


def _staged(fmt, shapes, seed, qa, special):
    from ternary_quantized_gemv_amd.staging import StagedSweep
    canon = [synth.blocks(fmt, r, c, seed, i) for i, (_, r, c) in enumerate(shapes)]
    x = [synth.activation(c, seed, 1000 + i) for i, (_, _, c) in enumerate(shapes)]
    if special:
        for v in (v for v in x if v.size >= 2 * qa):
            v[:qa] = 0.0                                     # an all-zero block: d = 0, q = 0
            v[qa:qa + 5] = [127.0, 2.5, -2.5, 0.5, -1.5]     # d = 1 exactly: ties away from zero
            v[qa + 5:2 * qa] = np.clip(v[qa + 5:2 * qa], -1.0, 1.0)
    return StagedSweep(fmt, canon, shapes, x, qa), canon


def _check_fused(fmt, shapes, seed, qa, special):
    t = torch()
    log(f"fused sweep fmt={fmt} qa={qa} special={special}: {len(shapes)} products")
    sw, canon = _staged(fmt, shapes, seed, qa, special)
    try:
        sw.sweep_fused()
        t.cuda.synchronize()
        y = sw.y.cpu().numpy()
        q_ref, d_ref, _ = oracle.quantize_q8(sw.x, qa)
        for i, (name, rows, cols) in enumerate(sw.shapes):
            k0, k1 = int(sw.koff[i]), int(sw.koff[i + 1])
            ref = oracle.matvec(fmt, canon[i], rows, cols, q_ref[k0:k1], d_ref[k0 // qa:k1 // qa], qa,
                                threads=THREADS)[0]
            got = y[int(sw.yoff[i]):int(sw.yoff[i + 1])]
            assert same_bits(got, ref), f"{name}: {np.count_nonzero(got.view(np.uint32) != ref.view(np.uint32))} differ"
        # the two-launch path gives the same bits, and so does a second fused launch
        sw.y.fill_(float("nan"))
        sw.run()
        t.cuda.synchronize()
        assert same_bits(sw.y.cpu().numpy(), y)
        sw.y.fill_(float("nan"))
        sw.sweep_fused()
        t.cuda.synchronize()
        assert same_bits(sw.y.cpu().numpy(), y)
    finally:
        sw.close()


@pytest.mark.parametrize("fmt", [Q1, Q2])
@pytest.mark.parametrize("qa,special", [(128, True), (64, False), (32, True)])
def test_fused_sweep_against_oracle(fmt, qa, special):
    _check_fused(fmt, MIX, 70 + fmt + qa, qa, special)


@pytest.mark.parametrize("fmt,qa", [(Q1, 128), (Q1, 32), (Q2, 128), (Q2, 64)])
def test_fused_sweep_paired_walk(fmt, qa):
    """Work items of two tiles per wavefront over several chunks
    (gpu_util.paired_walk_shapes), quantizing in the launch."""
    _check_fused(fmt, paired_walk_shapes(fmt), 90 + fmt + qa, qa, True)


@pytest.mark.parametrize("fmt", [Q1, Q2])
def test_fused_sweep_decode_token(fmt):
    """All 253 products of the decode token in one fused launch: every output
    equals the oracle's quantize-then-product, and the two-launch path
    (quantizer + bq_token_sweep) gives the same bits."""
    from ternary_quantized_gemv_amd.staging import StagedSweep
    t = torch()
    shapes = synth.decode_sweep_shapes()
    log(f"fused sweep decode token fmt={fmt}: staging")
    canon = [synth.blocks(fmt, r, c, 80 + fmt, i) for i, (_, r, c) in enumerate(shapes)]
    x = [synth.activation(c, 80 + fmt, 1000 + i) for i, (_, _, c) in enumerate(shapes)]
    sw = StagedSweep(fmt, canon, shapes, x, 128)
    try:
        sw.sweep_fused()
        t.cuda.synchronize()
        y_one = sw.y.cpu().numpy()
        log(f"fused sweep decode token fmt={fmt}: oracle over {sw.rows_total} outputs")
        q_ref, d_ref, _ = oracle.quantize_q8(sw.x, 128)
        bad = 0
        for i, (name, rows, cols) in enumerate(sw.shapes):
            k0, k1 = int(sw.koff[i]), int(sw.koff[i + 1])
            ref = oracle.matvec(fmt, canon[i], rows, cols, q_ref[k0:k1], d_ref[k0 // 128:k1 // 128], 128,
                                threads=THREADS)[0]
            got = y_one[int(sw.yoff[i]):int(sw.yoff[i + 1])]
            nbad = int(np.count_nonzero(got.view(np.uint32) != ref.view(np.uint32)))
            if nbad:
                log(f"  {name}: {nbad} of {rows} outputs differ from the oracle")
            bad += nbad
        assert bad == 0, f"{bad} outputs of the one-launch token differ from the oracle"
        sw.y.fill_(float("nan"))
        sw.run()
        t.cuda.synchronize()
        assert same_bits(sw.y.cpu().numpy(), y_one)
    finally:
        sw.close()


def test_fused_sweep_refuses_f16_scales():
    from ternary_quantized_gemv_amd.staging import StagedSweep
    shapes = [("a", 64, 256)]
    sw = StagedSweep(Q1, [synth.blocks(Q1, 64, 256, 1, 0)], shapes, [synth.activation(256, 1, 0)], 32,
                     f16_scale=True)
    try:
        with pytest.raises(ValueError):
            sw.sweep_fused()
    finally:
        sw.close()
