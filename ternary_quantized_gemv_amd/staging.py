"""Stage many products on the GPU and run them as one decode-token sweep.

A convenience over the C ABI binding: packs each canonical matrix with bq_pack,
copies both planes to the device once, lays the float32 activation vectors end
to end in one device buffer (so one bq_quantize_act_q8 call quantizes them
all: quantization works block by block and every vector length is a multiple
of qa), and builds one bq_sweep plan.  A token is then two launches: the
quantizer over all activations and the sweep.
"""
from __future__ import annotations

import numpy as np

from . import Act, Weights, bq_quantize_act_q8, bq_sweep_create, bq_token_sweep, BLOCK_LEN


class StagedSweep:
    def __init__(self, fmt: int, canon, shapes, x, qa: int = 128, keep_host: bool = True):
        """fmt: BQ_Q1_0 / BQ_Q2_0; canon: list of uint8 [rows, cols/QK, 18];
        shapes: list of (name, rows, cols); x: list of float32 [cols] (or one
        concatenated float32 array)."""
        import torch

        self.fmt, self.qa = fmt, qa
        self.shapes = [(str(n), int(r), int(c)) for n, r, c in shapes]
        for _, _, cols in self.shapes:
            if cols % qa or cols % BLOCK_LEN[fmt]:
                raise ValueError("every cols must be a multiple of qa and of the block length")
        self.koff = np.concatenate([[0], np.cumsum([c for _, _, c in self.shapes])]).astype(np.int64)
        self.yoff = np.concatenate([[0], np.cumsum([r for _, r, _ in self.shapes])]).astype(np.int64)
        self.ktotal = int(self.koff[-1])
        self.rows_total = int(self.yoff[-1])
        self.weights = []
        self.weight_bytes = 0
        self.canon = [] if keep_host else None
        for c, (_, rows, cols) in zip(canon, self.shapes):
            self.weights.append(Weights.upload(fmt, c, rows, cols))
            self.weight_bytes += c.size
            if keep_host:
                self.canon.append(c)
        xa = np.concatenate([np.asarray(v, np.float32).ravel() for v in x]) if isinstance(x, (list, tuple)) \
            else np.asarray(x, np.float32).ravel()
        if xa.size != self.ktotal:
            raise ValueError("activation length does not match the shapes")
        self.x = xa
        self.xd = torch.from_numpy(xa).to("cuda")
        self.q = torch.empty(self.ktotal, dtype=torch.int8, device="cuda")
        self.d = torch.empty(self.ktotal // qa, dtype=torch.float32, device="cuda")
        self.y = torch.full((self.rows_total,), float("nan"), dtype=torch.float32, device="cuda")
        self.entries = []
        for i, (_, rows, cols) in enumerate(self.shapes):
            k0, k1 = int(self.koff[i]), int(self.koff[i + 1])
            a = Act(self.q[k0:k1], self.d[k0 // qa:k1 // qa], cols, qa, 1)
            self.entries.append((self.weights[i], a, self.y[int(self.yoff[i]):int(self.yoff[i + 1])]))
        self.plan = bq_sweep_create(self.entries)

    # ------------------------------------------------------------- running
    def quantize(self, stream=None):
        bq_quantize_act_q8(self.xd, self.qa, self.q, self.d, stream)

    def sweep(self, stream=None):
        bq_token_sweep(self.plan, stream)

    def run(self, stream=None):
        self.quantize(stream)
        self.sweep(stream)

    # ----------------------------------------------------------- accounting
    def sweep_bytes(self) -> int:
        """Algorithmic bytes of one sweep launch: packed weights (18 bytes a
        block) + int8 quants + f32 activation scales read, f32 outputs written."""
        return self.weight_bytes + self.ktotal + 4 * (self.ktotal // self.qa) + 4 * self.rows_total

    def quantize_bytes(self) -> int:
        """Algorithmic bytes of the quantizer launch: f32 in, int8 + f32 scales out."""
        return 4 * self.ktotal + self.ktotal + 4 * (self.ktotal // self.qa)

    def output(self, i: int):
        return self.y[int(self.yoff[i]):int(self.yoff[i + 1])]

    def close(self):
        self.plan.destroy()
