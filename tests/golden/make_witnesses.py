"""Writes ``witnesses.json``: tiny hand-built inputs whose exact outputs follow
from binary arithmetic worked out by hand below (no oracle, no GPU involved).

Each witness isolates one step of the dot-product order that the bankML page
"gpu/ -- the video-card component" gives in its section "kernels.rs -- the Q1_0
kernels": the product of the first sub-block, the fused inner chain, the fused
outer step, the lane grouping and the final pairwise tree.  A mistake in any of
those steps moves the result off the value derived here.

Run: python tests/golden/make_witnesses.py
"""
from __future__ import annotations

import json
import os
import struct

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
CITE_GPU = 'bankML "gpu/ -- the video-card component", section "kernels.rs -- the Q1_0 kernels"'


def f32_hex(v: float) -> str:
    return struct.pack("<f", v).hex()


def f16_bits(v: float) -> int:
    return int(np.array([v], dtype=np.float16).view(np.uint16)[0])


ONE_PLUS_ULP = float(np.float32(1.0) + np.float32(2.0**-23))  # 1 + 2^-23, exact in f32


def q1_block(scale_bits: int, plus: list[int]) -> list[int]:
    """One canonical Q1_0 block: weights listed in ``plus`` are +1, the rest -1."""
    payload = [0] * 16
    for k in plus:
        payload[k >> 3] |= 1 << (k & 7)
    return [scale_bits & 0xFF, scale_bits >> 8] + payload


def q2_block(scale_bits: int, codes: dict[int, int]) -> list[int]:
    """One canonical Q2_0 block: code 1 (weight 0) except where ``codes`` says."""
    c = [1] * 64
    for k, v in codes.items():
        c[k] = v
    payload = [c[4 * i] | c[4 * i + 1] << 2 | c[4 * i + 2] << 4 | c[4 * i + 3] << 6 for i in range(16)]
    return [scale_bits & 0xFF, scale_bits >> 8] + payload


def witnesses():
    out = []

    # W1 -- the inner chain is fused and the first product is rounded.
    # Sub-block 0, lane 0: s0 = +3 (q[0] = 3, weight +1); sub-block 1, lane 0:
    # s1 = -3 (q[32] = 3, weight -1).  d1 = 1 + 2^-23 for both (qa = 32).
    # RN(d1*3): exact 3 + 3*2^-23 lies halfway between 3 + 2^-22 and 3 + 2^-21
    # (spacing 2^-22 in [2,4)); ties-to-even picks 3 + 2^-21.
    # ab = RN(d1*(-3) + 3 + 2^-21) = RN(-3 - 3*2^-23 + 3 + 4*2^-23) = 2^-23.
    # Later sub-blocks add d1*0.  acc0 = fma(1, 2^-23, +0) = 2^-23; other lanes 0.
    # An unfused chain gives RN(RN(P0) + RN(P1)) = 0, an exact sum gives 0.
    q = np.zeros(128, np.int8)
    q[0], q[32] = 3, 3
    out.append(dict(
        name="W1_inner_chain_fused", fmt=1, cols=128, qa=32,
        blocks=[q1_block(f16_bits(1.0), [0])],
        q=q.tolist(), d=[f32_hex(ONE_PLUS_ULP)] * 4,
        expected=f32_hex(2.0**-23),
        derivation="RN(d1*3) = 3+2^-21; RN(d1*(-3) + 3+2^-21) = 2^-23; y = 2^-23",
        cite=CITE_GPU))

    # W2 -- the outer step acc = fma(d0, ab, acc) is fused.
    # Two blocks, qa = 128, d1 = 1 + 2^-23, d0 = 1 + 2^-10 (an f16 value).
    # Block 0 lane 0: s = -1 (q[0] = 1, weight -1) -> ab0 = -(1 + 2^-23);
    #   acc = RN(d0*ab0) = -(1 + 2^-10 + 2^-23)   [exact 1 + 2^-10 + 2^-23 + 2^-33]
    # Block 1 lane 0: s = +1 (q[128] = 1, weight +1) -> ab1 = 1 + 2^-23;
    #   acc = RN(d0*ab1 + acc) = RN(2^-33) = 2^-33.   Unfused: 0.
    q = np.zeros(256, np.int8)
    q[0], q[128] = 1, 1
    d0 = f16_bits(1.0 + 2.0**-10)
    out.append(dict(
        name="W2_outer_step_fused", fmt=1, cols=256, qa=128,
        blocks=[q1_block(d0, []), q1_block(d0, [0])],
        q=q.tolist(), d=[f32_hex(ONE_PLUS_ULP)] * 2,
        expected=f32_hex(2.0**-33),
        derivation="acc after block 0 = -(1+2^-10+2^-23); fma(1+2^-10, 1+2^-23, acc) = 2^-33",
        cite=CITE_GPU))

    # W3 -- the final tree ((a0+a4)+(a2+a6)) + ((a1+a5)+(a3+a7)).
    # Block 0 (d0 = 2^12, d1 = 2^12): lane 0 gets s = 1 -> a0 = 2^24.
    # Block 1 (d0 = 1, d1 = 1): lanes 1, 2, 4, 6 get s = 1 (first element of
    # each lane group in sub-block 0: weights 132, 136, 144, 152).
    # a = [2^24, 1, 1, 0, 1, 0, 1, 0].
    # a0+a4 = 2^24+1 -> 2^24 (tie, even); a2+a6 = 2; -> 2^24+2 (exact);
    # a1+a5 = 1, a3+a7 = 0 -> 1; 2^24+2 + 1 = 2^24+3 -> tie -> 2^24+4 (even).
    # Left-to-right summation gives 2^24, adjacent pairs give 2^24+2.
    q = np.zeros(256, np.int8)
    q[0] = 1
    for k in (132, 136, 144, 152):
        q[k] = 1
    out.append(dict(
        name="W3_final_tree", fmt=1, cols=256, qa=128,
        blocks=[q1_block(f16_bits(4096.0), [0]), q1_block(f16_bits(1.0), [4, 8, 16, 24])],
        q=q.tolist(), d=[f32_hex(4096.0), f32_hex(1.0)],
        expected=f32_hex(2.0**24 + 4),
        derivation="a=[2^24,1,1,0,1,0,1,0]; tree -> 2^24+4",
        cite=CITE_GPU))

    # W4 -- lane L holds weights 4L..4L+3 of its sub-block (reading R3).
    # a0 = 2^24 as in W3.  Block 1: weight 132 (lane 1) and weight 149 (lane 5),
    # both +1 with q = 1.  a = [2^24, 1, 0, 0, 0, 1, 0, 0].
    # (a0+a4)+(a2+a6) = 2^24; (a1+a5)+(a3+a7) = 2; total 2^24+2 (exact).
    # With lanes taken as stride-8 (weight 4 -> lane 4), a4 = 1 would be lost
    # against 2^24 and the result would be 2^24+1 -> 2^24.
    q = np.zeros(256, np.int8)
    q[0], q[132], q[149] = 1, 1, 1
    out.append(dict(
        name="W4_lane_grouping", fmt=1, cols=256, qa=128,
        blocks=[q1_block(f16_bits(4096.0), [0]), q1_block(f16_bits(1.0), [4, 21])],
        q=q.tolist(), d=[f32_hex(4096.0), f32_hex(1.0)],
        expected=f32_hex(2.0**24 + 2),
        derivation="a=[2^24,1,0,0,0,1,0,0]; tree -> 2^24+2",
        cite=CITE_GPU))

    # W5 -- int8 negation wraps: weight -1 times q = -128 contributes -128.
    # One block, d0 = d1 = 1; lane 0 of sub-block 0: q = [-128, -128, 5, 0] with
    # weights [-1, +1, -1, +1] -> s = -128 + -128 + -5 + 0 = -261.
    # Every other q is 0.  y = -261.
    q = np.zeros(128, np.int8)
    q[0], q[1], q[2] = -128, -128, 5
    out.append(dict(
        name="W5_negation_wrap", fmt=1, cols=128, qa=128,
        blocks=[q1_block(f16_bits(1.0), [1, 3])],
        q=q.tolist(), d=[f32_hex(1.0)],
        expected=f32_hex(-261.0),
        derivation="(-1)*(-128) wraps to -128: s = -128-128-5 = -261",
        cite=CITE_GPU + '; section "How it is verified" (-128 quants)'))

    # W6 -- Q2_0, same inner chain as W1 on its two 32-weight sub-blocks.
    # Code 2 (+1) on weight 0 with q[0] = 3; code 0 (-1) on weight 32 with
    # q[32] = 3; every other weight code 1 (0).  d1 = 1 + 2^-23 (qa = 32),
    # d0 = 1.  y = 2^-23 as in W1.
    q = np.zeros(64, np.int8)
    q[0], q[32] = 3, 3
    out.append(dict(
        name="W6_q2_inner_chain", fmt=2, cols=64, qa=32,
        blocks=[q2_block(f16_bits(1.0), {0: 2, 32: 0})],
        q=q.tolist(), d=[f32_hex(ONE_PLUS_ULP)] * 2,
        expected=f32_hex(2.0**-23),
        derivation="as W1 with ternary codes: y = 2^-23",
        cite=CITE_GPU + " (order reused for Q2_0, reading R5)"))

    # W7 -- Q2_0 code map: code c means weight c-1.  d0 = d1 = 1.
    # Lane 0: codes [0, 1, 2, 2] with q = [7, 11, 13, -128] -> -7 + 0 + 13 - 128.
    # Lane 3 of sub-block 1 (weights 44..47): codes [2, 0, 1, 0], q = [1, 2, 3, 4]
    # -> 1 - 2 + 0 - 4 = -5.  y = -122 + -5 = -127.
    q = np.zeros(64, np.int8)
    q[0:4] = [7, 11, 13, -128]
    q[44:48] = [1, 2, 3, 4]
    out.append(dict(
        name="W7_q2_code_map", fmt=2, cols=64, qa=64,
        blocks=[q2_block(f16_bits(1.0), {0: 0, 1: 1, 2: 2, 3: 2, 44: 2, 45: 0, 46: 1, 47: 0})],
        q=q.tolist(), d=[f32_hex(1.0)],
        expected=f32_hex(-127.0),
        derivation="w = c-1: (-7 + 0 + 13 - 128) + (1 - 2 + 0 - 4) = -127",
        cite="reading R2 (the pages give Q2_0's size only)"))
    return out


if __name__ == "__main__":
    path = os.path.join(HERE, "witnesses.json")
    with open(path, "w") as f:
        json.dump(witnesses(), f, indent=1)
    print("wrote", path)
