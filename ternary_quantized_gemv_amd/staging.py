"""Stage many products on the GPU and run them as one decode-token sweep.

A convenience over the C ABI binding: packs each canonical matrix with bq_pack,
copies both planes to the device once, lays the float32 activation vectors end
to end in one device buffer (so one bq_quantize_act_q8 call quantizes them
all: quantization works block by block and every vector length is a multiple
of qa), and builds one bq_sweep plan.  A token is then two launches: the
quantizer over all activations and the sweep -- or one, sweep_fused(), whose
plan (bq_sweep_create_x) quantizes the f32 vectors inside the launch.
"""
from __future__ import annotations

import numpy as np

from . import (Act, GroupCall, Weights, bq_quantize_act_q8, bq_quantize_act_q8_f16, bq_sweep_create,
               bq_sweep_create_x, bq_token_sweep, BLOCK_LEN)


class StagedSweep:
    def __init__(self, fmt: int, canon, shapes, x, qa: int = 128, keep_host: bool = True,
                 f16_scale: bool = False):
        """fmt: BQ_Q1_0 / BQ_Q2_0; canon: list of uint8 [rows, cols/QK, 18];
        shapes: list of (name, rows, cols); x: list of float32 [cols] (or one
        concatenated float32 array); f16_scale: quantize with f16-valued
        scales (bq_quantize_act_q8_f16, the q8_0 flavour)."""
        import torch

        self.fmt, self.qa, self.f16_scale = fmt, qa, f16_scale
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
        self.plan_x = None

    # ------------------------------------------------------------- running
    def quantize(self, stream=None):
        (bq_quantize_act_q8_f16 if self.f16_scale else bq_quantize_act_q8)(self.xd, self.qa, self.q, self.d, stream)

    def sweep(self, stream=None):
        bq_token_sweep(self.plan, stream)

    def run(self, stream=None):
        self.quantize(stream)
        self.sweep(stream)

    def sweep_fused(self, stream=None):
        """The token in one launch from the f32 activations (f32 scales only):
        the same bits in y as run()."""
        if self.f16_scale:
            raise ValueError("the in-launch quantizer writes f32 scales (the q8_0 flavour needs run())")
        if self.plan_x is None:
            ents = [(w, self.xd[int(self.koff[i]):int(self.koff[i + 1])], y) for i, (w, _, y) in enumerate(self.entries)]
            self.plan_x = bq_sweep_create_x(ents, self.qa)
        bq_token_sweep(self.plan_x, stream)

    # ----------------------------------------------------------- accounting
    def sweep_bytes(self) -> int:
        """Algorithmic bytes of one sweep launch: packed weights (18 bytes a
        block) + int8 quants + f32 activation scales read, f32 outputs written."""
        return self.weight_bytes + self.ktotal + 4 * (self.ktotal // self.qa) + 4 * self.rows_total

    def fused_bytes(self) -> int:
        """Algorithmic bytes of one sweep_fused launch: packed weights + the
        f32 activations read, f32 outputs written."""
        return self.weight_bytes + 4 * self.ktotal + 4 * self.rows_total

    def quantize_bytes(self) -> int:
        """Algorithmic bytes of the quantizer launch: f32 in, int8 + f32 scales out."""
        return 4 * self.ktotal + self.ktotal + 4 * (self.ktotal // self.qa)

    def output(self, i: int):
        return self.y[int(self.yoff[i]):int(self.yoff[i + 1])]

    def close(self):
        self.plan.destroy()
        if self.plan_x is not None:
            self.plan_x.destroy()


# ------------------------------------------------------------------ chain
def chain_groups(n_layers: int, lm_head: bool = True):
    """The dependency order of one decode token over the products of
    synth.decode_sweep_shapes(n_layers): per layer {q, k, v}, {o}, {gate, up},
    {down}, then {lm_head}.  Returns [(product indices, source index)]: the
    group's input is the output of product `source` (-1: the token's input
    vector).  The products' own data dependencies (attention, the gated
    activation) are replaced by the nearest output of the right length:
    o takes q's output, gate and up take o's, down takes up's, and the next
    layer (or the LM head) takes down's."""
    groups = []
    prev = -1
    for layer in range(n_layers):
        base = 7 * layer
        q, k, v, o, gate, up, down = range(base, base + 7)
        groups.append(([q, k, v], prev))
        groups.append(([o], q))
        groups.append(([gate, up], o))
        groups.append(([down], up))
        prev = down
    if lm_head:
        groups.append(([7 * n_layers], prev))
    return groups


class StagedChain:
    """One decode token as a chain of dependent launches over the groups of
    chain_groups(), all on one stream.  fused=True: one bq_group_matvec launch
    per group, which quantizes the group's input (the previous group's f32
    output) inside the kernel.  fused=False: a bq_quantize_act_q8 launch into
    an int8 buffer, then a sweep launch over the group's products."""

    def __init__(self, fmt: int, canon, shapes, x0, qa: int = 128, n_layers: int = None, fused: bool = True):
        import torch

        self.fmt, self.qa, self.fused = fmt, qa, fused
        self.shapes = [(str(n), int(r), int(c)) for n, r, c in shapes]
        n_layers = (len(self.shapes) - 1) // 7 if n_layers is None else n_layers
        self.groups = chain_groups(n_layers, lm_head=len(self.shapes) == 7 * n_layers + 1)
        self.yoff = np.concatenate([[0], np.cumsum([r for _, r, _ in self.shapes])]).astype(np.int64)
        self.weights = [Weights.upload(fmt, c, r, k) for c, (_, r, k) in zip(canon, self.shapes)]
        self.weight_bytes = int(sum(c.size for c in canon))
        self.x0 = torch.from_numpy(np.asarray(x0, np.float32).ravel()).to("cuda")
        self.y = torch.full((int(self.yoff[-1]),), float("nan"), dtype=torch.float32, device="cuda")
        self.stages = []
        for prods, src in self.groups:
            cols = self.shapes[prods[0]][2]
            if any(self.shapes[p][2] != cols for p in prods):
                raise ValueError("a group's products must share their input length")
            xin = self.x0 if src < 0 else self.output(src)
            if xin.numel() != cols:
                raise ValueError("a group's input length must match its products")
            if fused:
                self.stages.append(GroupCall([self.weights[p] for p in prods], xin, qa,
                                             [self.output(p) for p in prods]))
            else:
                q = torch.empty(cols, dtype=torch.int8, device="cuda")
                d = torch.empty(cols // qa, dtype=torch.float32, device="cuda")
                a = Act(q, d, cols, qa, 1)
                plan = bq_sweep_create([(self.weights[p], a, self.output(p)) for p in prods])
                self.stages.append((xin, q, d, plan))

    def output(self, i: int):
        return self.y[int(self.yoff[i]):int(self.yoff[i + 1])]

    def run(self, stream=None):
        if self.fused:
            for call in self.stages:
                call.launch(stream)
            return
        for xin, q, d, plan in self.stages:
            bq_quantize_act_q8(xin, self.qa, q, d, stream)
            bq_token_sweep(plan, stream)

    def launches(self) -> int:
        return len(self.stages) * (1 if self.fused else 2)

    def token_bytes(self) -> int:
        """Algorithmic bytes of one token: weights, every group's f32 input
        read once and every output written; unfused, also the int8 quants and
        scales written by the quantizer and read by each product."""
        n = 0
        for prods, _ in self.groups:
            cols = self.shapes[prods[0]][2]
            n += 4 * cols
            if not self.fused:
                n += cols + 4 * (cols // self.qa)                          # quantizer writes
                n += len(prods) * (cols + 4 * (cols // self.qa))           # products read the activation
        return self.weight_bytes + n + 4 * int(self.yoff[-1])

    def close(self):
        if not self.fused:
            for _, _, _, plan in self.stages:
                plan.destroy()
        self.stages = []
