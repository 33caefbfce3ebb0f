"""A decode token as a chain of dependent launches: every group's activation
is the quantized output of the previous group (per layer {q, k, v}, {o},
{gate, up}, {down}, then the LM head; the attention and gated-activation
steps between them are replaced by the nearest output of the right length).
The chain on the GPU must equal the same chain computed by the CPU oracle
alone, bit for bit, through all 145 quantizations and 253 products; a chain
captured in a graph must replay to the same bits."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import log, torch
from pins import same_bits

pytestmark = pytest.mark.gpu

THREADS = 16


def chain_wiring(n_layers):
    """[(products, source)] written out from the rule above (kept apart from the
    package's own wiring, which the test compares against it)."""
    out, prev = [], -1
    for layer in range(n_layers):
        b = 7 * layer
        out += [([b, b + 1, b + 2], prev), ([b + 3], b), ([b + 4, b + 5], b + 3), ([b + 6], b + 5)]
        prev = b + 6
    out.append(([7 * n_layers], prev))
    return out


def oracle_chain(fmt, canon, shapes, x0, wiring, qa=128):
    ys = [None] * len(shapes)
    for prods, src in wiring:
        q, d, _ = oracle.quantize_q8(x0 if src < 0 else ys[src], qa)
        for p in prods:
            _, rows, cols = shapes[p]
            ys[p] = oracle.matvec(fmt, canon[p], rows, cols, q, d, qa, threads=THREADS)[0]
    return ys


def _stage(fmt, n_layers, seed, fused=True):
    from ternary_quantized_gemv_amd.staging import StagedChain, chain_groups
    assert chain_groups(n_layers) == chain_wiring(n_layers)
    shapes = synth.decode_sweep_shapes(n_layers)
    canon = [synth.blocks(fmt, r, c, seed, i) for i, (_, r, c) in enumerate(shapes)]
    x0 = synth.activation(shapes[0][2], seed, 999)
    return StagedChain(fmt, canon, shapes, x0, fused=fused), canon, shapes, x0


@pytest.mark.parametrize("fused", [True, False], ids=["fused", "quantize+sweep"])
@pytest.mark.parametrize("fmt,n_layers", [(1, 36), (2, 4)])
def test_chain_against_oracle(fmt, n_layers, fused):
    t = torch()
    log(f"chain fmt={fmt} layers={n_layers} fused={fused}: staging")
    ch, canon, shapes, x0 = _stage(fmt, n_layers, 71 + fmt, fused)
    try:
        ch.run()
        t.cuda.synchronize()
        y = ch.y.cpu().numpy()
        assert np.all(np.isfinite(y))
        ys = oracle_chain(fmt, canon, shapes, x0, chain_wiring(n_layers))
        bad = 0
        for i, (name, _, _) in enumerate(shapes):
            nbad = int(np.count_nonzero(y[ch.yoff[i]:ch.yoff[i + 1]].view(np.uint32) != ys[i].view(np.uint32)))
            if nbad:
                log(f"  {name}: {nbad} outputs differ")
            bad += nbad
        log(f"chain fmt={fmt}: {y.size} outputs over {len(ch.stages)} groups, {bad} differ")
        assert bad == 0
    finally:
        ch.close()


@pytest.mark.parametrize("fused", [True, False], ids=["fused", "quantize+sweep"])
def test_chain_graph_replay(fused):
    """Capture one chain in a graph; every replay, with eager work and
    synchronisation between replays, gives the eager chain's bits."""
    t = torch()
    ch, _, _, _ = _stage(1, 2, 81, fused)
    try:
        ch.run()
        t.cuda.synchronize()
        ref = ch.y.cpu().numpy()
        side = t.cuda.Stream()
        side.wait_stream(t.cuda.current_stream())
        with t.cuda.stream(side):
            ch.run()  # warm-up on the capture stream
        t.cuda.current_stream().wait_stream(side)
        t.cuda.synchronize()
        g = t.cuda.CUDAGraph()
        with t.cuda.graph(g):
            ch.run()
        for rep in range(3):
            ch.y.fill_(float("nan"))
            t.cuda.synchronize()
            g.replay()
            t.cuda.synchronize()
            assert same_bits(ch.y.cpu().numpy(), ref), f"replay {rep}"
            ch.run()  # eager work between replays
            t.cuda.synchronize()
            assert same_bits(ch.y.cpu().numpy(), ref)
        log("chain graph: 3 replays equal the eager chain")
    finally:
        ch.close()
