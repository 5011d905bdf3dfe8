"""Block verification over a stack of MoE layers ("A drafter that leaves the
answer unchanged", "Run Kimi 3.1 locally on one GPU").

The engine on the pages verifies drafted tokens in one multi-row pass (at
most 16 rows: the token being decoded followed by the drafts).  A draft is
accepted while it equals the model's greedy choice at its position; the
output is always the model's own greedy sequence.  Experts are fetched once
per block, and each block row must reproduce the one-row step exactly; the
pages show this by FNV-1a hashing every position's logits on both sides,
and this harness does the same.

``Stack`` is the harness's model: no attention, so a row depends only on its
own token.  Per row, with h the fp32 residual stream and n(.) the RMS
normalisation (pre-norm residual blocks, so h grows only linearly):

    h  = Q8_0 row ``token`` of the head matrix            (tied embedding)
    for each layer l:
        h += n(h) . S_l^T      (Q8_0 spine matmul, d x d, at most 8 rows a call)
        h += MoE_l(bf16(n(h))) (moe_layer_mxfp4: router, top-k, experts, combine)
    logits = n(h) . H^T        (Q8_0 head, vocabulary x d)
    next token = argmax(logits)

Every step is a C-ABI call into the library's kernels; this module only
sequences them and holds the buffers.  Everything runs on torch's current
stream (select another with ``torch.cuda.stream``).
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

from . import (MOE_LAYOUT_ROWS, MOE_LAYOUT_TILES, Experts, MoELayer, moe_argmax_rows, moe_fnv1a_rows,
               moe_residual_bf16, moe_rmsnorm, q8_0_matmul, q8_0_pack, q8_0_rows)

Q8_ROWS = 8  # the Q8_0 matmul takes up to 8 rows per call
EPS = 1e-6


@dataclass
class Q8Matrix:
    wq: torch.Tensor  # int8 [N x K], device
    ws: torch.Tensor  # fp16 bits [N x K/32] (int16), device
    layout: int = MOE_LAYOUT_ROWS  # order of wq (q8_0_pack converts)

    def tiled(self) -> "Q8Matrix":
        """A copy with wq in tile order (N % 16 == 0)."""
        dst = torch.empty_like(self.wq)
        q8_0_pack(self.wq, dst, MOE_LAYOUT_TILES)
        return Q8Matrix(dst, self.ws, MOE_LAYOUT_TILES)


class Stack:
    def __init__(self, layers: list[tuple[Experts, torch.Tensor]], spines: list[Q8Matrix], head: Q8Matrix, k: int,
                 max_rows: int = 16, device="cuda"):
        if len(layers) != len(spines) or not layers:
            raise ValueError("one spine matrix per layer")
        d = layers[0][0].d
        self.d, self.vocab, self.k, self.max_rows = d, head.wq.shape[0], k, max_rows
        self.spines, self.head = spines, head
        self.mls = [MoELayer(ex, k, max_rows, w_router=wr, device=device) for ex, wr in layers]
        f32 = dict(dtype=torch.float32, device=device)
        self.h = torch.empty((max_rows, d), **f32)
        self.a = torch.empty((max_rows, d), **f32)
        self.n = torch.empty((max_rows, d), **f32)
        self.hb = torch.empty((max_rows, d), dtype=torch.bfloat16, device=device)
        self.logits = torch.empty((max_rows, self.vocab), **f32)
        self.tok = torch.empty(max_rows, dtype=torch.int32, device=device)
        self.next = torch.empty(max_rows, dtype=torch.int32, device=device)
        self.hashes = torch.empty(max_rows, dtype=torch.int64, device=device)

    def _q8(self, X, m: Q8Matrix, Y):
        for r in range(0, X.shape[0], Q8_ROWS):
            q8_0_matmul(X[r:r + Q8_ROWS], m.wq, m.ws, Y[r:r + Q8_ROWS], layout=m.layout)

    def run(self, tokens: torch.Tensor) -> torch.Tensor:
        """Logits [M x vocab] of M rows, row m fed token tokens[m] (int32, on
        the device); also leaves each row's greedy next token in self.next."""
        M = tokens.numel()
        if M < 1 or M > self.max_rows:
            raise ValueError("1..max_rows rows")
        self.tok[:M].copy_(tokens)
        h, a, n, hb = self.h[:M], self.a[:M], self.n[:M], self.hb[:M]
        q8_0_rows(self.tok[:M], self.head.wq, self.head.ws, h, layout=self.head.layout)
        for ml, spine in zip(self.mls, self.spines):
            moe_rmsnorm(h, n, None, EPS)
            self._q8(n, spine, a)
            moe_residual_bf16(h, a, None)
            moe_rmsnorm(h, None, hb, EPS)
            v = ml.forward(hb)
            moe_residual_bf16(h, v["out"], None)
        moe_rmsnorm(h, n, None, EPS)
        self._q8(n, self.head, self.logits[:M])
        moe_argmax_rows(self.logits[:M], self.next)
        return self.logits[:M]

    def hash_rows(self, M: int) -> list[int]:
        """FNV-1a of the last run's logits rows (bits as unsigned ints)."""
        moe_fnv1a_rows(self.logits[:M], self.hashes)
        return [int(v) & 0xFFFFFFFFFFFFFFFF for v in self.hashes[:M].cpu().tolist()]


def plain_steps(stack: Stack, token: int, n: int, hashes: bool = True):
    """n plain decode steps from ``token``: returns the n tokens the model
    chooses and, with ``hashes``, each step's logits hash."""
    out, hs = [], []
    cur = torch.tensor([token], dtype=torch.int32, device=stack.tok.device)
    for _ in range(n):
        stack.run(cur)
        if hashes:
            hs.append(stack.hash_rows(1)[0])
        cur = stack.next[:1].clone()
        out.append(cur)
    return [int(t.item()) for t in out], hs


def verify_block(stack: Stack, token: int, drafts: list[int], hashes: bool = True):
    """One block: row 0 = ``token``, rows 1.. = the drafts.  The model's
    choice after row i is g_i; draft i+1 is kept while g_i equals it.
    Returns (emitted tokens = the kept drafts' g's plus the model's token after
    the last kept row, number of drafts kept, per-row logits hashes)."""
    rows = [token] + list(drafts)
    t = torch.tensor(rows, dtype=torch.int32, device=stack.tok.device)
    stack.run(t)
    hs = stack.hash_rows(len(rows)) if hashes else []
    g = stack.next[:len(rows)].cpu().tolist()
    kept = 0
    while kept < len(drafts) and g[kept] == drafts[kept]:
        kept += 1
    return g[:kept + 1], kept, hs
