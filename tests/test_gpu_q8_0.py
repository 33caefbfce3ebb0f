"""The q8_0 activation flavour end to end: f16-valued activation scales
(bq_quantize_act_q8_f16) with qa 32 -- one scale per 32 values, as in the
pages' activation binding -- and qa 128.  The quantizer must equal the
oracle's f16-scale quantizer bit for bit (ties, zero blocks, scales in the f16
subnormal range where the clamp binds, scales that narrow to zero), and the
products fed with those activations must equal the oracle's, through the
single-product kernels and through a whole decode-token sweep."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import bqmod, dev, log, stage_act, torch
from pins import same_bits
from test_gpu_parity import _check_sweep

pytestmark = pytest.mark.gpu

Q1, Q2 = 1, 2
THREADS = 16


def quantize_f16_gpu(x, qa):
    t, bq = torch(), bqmod()
    q = t.empty(x.size, dtype=t.int8, device="cuda")
    d = t.empty(x.size // qa, dtype=t.float32, device="cuda")
    bq.bq_quantize_act_q8_f16(dev(x.astype(np.float32)), qa, q, d)
    t.cuda.synchronize()
    return q.cpu().numpy(), d.cpu().numpy()


def special_input(n, qa, seed):
    x = synth.activation(n, seed, qa)
    x[:qa] = 0.0                                          # an all-zero block
    x[qa:2 * qa] = 0.0
    x[qa:qa + 6] = [127.0, 2.5, -2.5, 0.5, -0.5, 1.5]     # d = 1: exact ties
    # amax / 127 = 1.4 * 2^-24 narrows to the f16 subnormal 2^-24, so
    # x / d reaches 178 and the clamp binds
    x[2 * qa:3 * qa] = np.linspace(-1.0, 1.0, qa, dtype=np.float32) * np.float32(127 * 1.4 * 2.0 ** -24)
    x[3 * qa:4 * qa] = np.float32(1e-9)                   # amax / 127 narrows to 0
    x[4 * qa:5 * qa] *= np.float32(3000.0)                # large, still finite scales
    x[5 * qa:6 * qa] *= np.float32(1e-30)                 # far below the f16 range
    return x


@pytest.mark.parametrize("qa", [32, 64, 128])
@pytest.mark.parametrize("regime", ["normal", "layer", "special"])
def test_quantizer_f16_parity(qa, regime):
    log("quantizer f16", qa, regime)
    n = 12288 + 384
    if regime == "normal":
        x = synth.activation(n, 31, qa)
    elif regime == "layer":
        x = synth.layer_shaped(Q1, 1, n, 32, qa)[1]
    else:
        x = special_input(n, qa, 33)
    q_ref, d_ref, clamped = oracle.quantize_q8(x, qa, f16_scale=True)
    log(f"  {clamped} values clamped, {int(np.count_nonzero(d_ref == 0))} zero scales")
    if regime == "special":
        assert clamped > 0
    q, d = quantize_f16_gpu(x, qa)
    assert np.array_equal(q, q_ref)
    assert same_bits(d, d_ref)


@pytest.mark.parametrize("fmt", [Q1, Q2])
@pytest.mark.parametrize("rows,nb,qa", [(100, 33, 32), (4096, 32, 32), (700, 96, 128), (20000, 4, 32)])
def test_q8_0_products(fmt, rows, nb, qa):
    """GPU quantizer (f16 scales) -> GPU product, against the oracle's."""
    t, bq = torch(), bqmod()
    cols = nb * bq.BLOCK_LEN[fmt]
    log(f"q8_0 product fmt={fmt} {rows}x{cols} qa={qa}")
    w = synth.blocks(fmt, rows, cols, 41, rows)
    x = special_input(cols, qa, 42) if cols >= 6 * qa else synth.activation(cols, 42, 0)
    q, d = quantize_f16_gpu(x, qa)
    q_ref, d_ref, _ = oracle.quantize_q8(x, qa, f16_scale=True)
    assert np.array_equal(q, q_ref) and same_bits(d, d_ref)
    wd = bq.Weights.upload(fmt, w, rows, cols)
    y = t.full((rows,), float("nan"), dtype=t.float32, device="cuda")
    (bq.bq_q1_0_matvec if fmt == Q1 else bq.bq_q2_0_matvec)(wd, stage_act(q, d, qa), y)
    t.cuda.synchronize()
    ref = oracle.matvec(fmt, w, rows, cols, q_ref, d_ref, qa, threads=THREADS)[0]
    assert same_bits(y.cpu().numpy(), ref)


@pytest.mark.parametrize("fmt", [Q1, Q2])
def test_q8_0_decode_token_sweep(fmt):
    """All 253 products of a decode token with qa 32, f16-valued scales."""
    _check_sweep(fmt, synth.decode_sweep_shapes(), seed=64 + fmt, qa=32, f16_scale=True)
