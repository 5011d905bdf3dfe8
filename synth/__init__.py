"""Seeded synthetic inputs for the MXFP4 mixture-of-experts layer and the
Q8_0 spine matmul.

This module is shared by the tests, the benchmark and the smoke check, and it
feeds both the CPU oracle and the GPU library.  It draws random bytes and
numbers and packs them into the storage formats; it contains none of the
layer's arithmetic (no dequantisation, routing, bucketing, FFN or combine).

Workloads (shapes from "Run Kimi 3.1 locally on one GPU", argonautlabs.ai:
top-16 routing over 896 experts, section "Read the experts the router needs";
blocks of 2..16 rows, section "A drafter that leaves the answer unchanged";
270- and 1,533-token prompt passes, section "Decode and prefill are different
measurements"; 17,547,264-byte MXFP4 experts, section "One GPU, three storage
tiers"; 2 shared experts from the model table of the computingforgeeks guide
"Run Kimi K3 and K3.1 Pro Locally"):

* tiny:    d=256, f=128, 16 experts, top-2, no shared expert, x fp32 N(0,1),
           W_r N(0, 0.05), E8M0 exponents uniform in [-6, -2];
* kimi:    d=7168, f=1536, 896 routed + 2 shared, top-16, x bf16 N(0,1),
           W_r N(0, 0.02), E8M0 exponents uniform in [-8, -4];
* block:   row 0 is x0 ~ N(0,1), row i>0 is x0 + N(0, 0.3^2), then bf16;
* q8_0:    int8 uniform in [-127, 127], fp16 scale ~ U(1e-3, 1e-2), X fp32 N(0,1);
* prefill: logits = log p_{pi(e)} + Gumbel(0,1) with p_r proportional to
           r^-1.1 over a seeded permutation pi (Zipf popularity; Gumbel-top-k
           draws k distinct experts with those probabilities).
The second argument of N(.,.) is a standard deviation.  Code bytes are
uniform over 0..255, so both nibbles are uniform E2M1 codes.
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class LayerShape:
    name: str
    d: int
    f: int
    n_routed: int
    n_shared: int
    k: int
    exp_lo: int
    exp_hi: int
    wr_std: float
    x_dtype: str  # "f32" or "bf16"

    @property
    def n_experts(self) -> int:
        return self.n_routed + self.n_shared

    @property
    def sections(self) -> tuple[int, int, int, int, int, int]:
        """Byte sizes of gate codes, gate scales, up codes, up scales, down
        codes, down scales (gate/up are [f x d], down is [d x f])."""
        c, s = self.f * self.d // 2, self.f * self.d // 32
        return (c, s, c, s, c, s)

    @property
    def stride(self) -> int:
        return sum(self.sections)


TINY = LayerShape("tiny", 256, 128, 16, 0, 2, -6, -2, 0.05, "f32")
KIMI = LayerShape("kimi", 7168, 1536, 896, 2, 16, -8, -4, 0.02, "bf16")

# (K, N) of the three spine matrices; M in {1, 2, 4, 8}
Q8_0_SHAPES = ((7168, 7168), (7168, 18432), (7168, 163840))
BLOCK_SIGMA = 0.3
ZIPF_S = 1.1


def rng(seed: int, *tags: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), *[int(t) for t in tags]])))


# stream tags keep every tensor's draws independent of the others
_T_EXPERT, _T_ROUTER, _T_X, _T_BLOCK, _T_Q8, _T_ZIPF, _T_MISC = 11, 12, 13, 14, 15, 16, 17


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def expert_record(shape: LayerShape, seed: int, e: int) -> np.ndarray:
    """Expert e's record: uniform code bytes, E8M0 scale bytes 127+U{lo..hi}."""
    g = rng(seed, _T_EXPERT, e)
    parts = []
    for i, n in enumerate(shape.sections):
        if i % 2 == 0:
            parts.append(g.integers(0, 256, size=n, dtype=np.uint8))
        else:
            parts.append((127 + g.integers(shape.exp_lo, shape.exp_hi + 1, size=n)).astype(np.uint8))
    return np.concatenate(parts)


def expert_records(shape: LayerShape, seed: int, ids, workers: int = 8):
    """Yield (e, record) for each id, generated in a thread pool."""
    ids = list(ids)
    with ThreadPoolExecutor(max_workers=workers) as ex:
        for e, rec in zip(ids, ex.map(lambda i: expert_record(shape, seed, i), ids)):
            yield e, rec


def router_weight(shape: LayerShape, seed: int) -> np.ndarray:
    g = rng(seed, _T_ROUTER)
    return (g.standard_normal((shape.n_routed, shape.d), dtype=np.float32) * np.float32(shape.wr_std)).astype(np.float32)


def rows_x(shape: LayerShape, seed: int, M: int) -> np.ndarray:
    """M independent rows ~ N(0,1): float32, or bfloat16 bits for bf16 layers."""
    x = rng(seed, _T_X, M).standard_normal((M, shape.d), dtype=np.float32)
    return bf16_bits(x) if shape.x_dtype == "bf16" else x


def block_x(shape: LayerShape, seed: int, B: int, sigma: float = BLOCK_SIGMA) -> np.ndarray:
    """A verification block: row 0 = x0 ~ N(0,1); row i>0 = x0 + N(0, sigma^2)."""
    g = rng(seed, _T_BLOCK, B)
    x0 = g.standard_normal(shape.d, dtype=np.float32)
    x = np.repeat(x0[None, :], B, axis=0)
    if B > 1:
        x[1:] += g.standard_normal((B - 1, shape.d), dtype=np.float32) * np.float32(sigma)
    return bf16_bits(x) if shape.x_dtype == "bf16" else x


def zipf_logits(shape: LayerShape, seed: int, M: int, s: float = ZIPF_S) -> np.ndarray:
    """Router logits whose top-k draws follow Zipf(s) popularity over a seeded
    permutation of the routed experts (Gumbel-top-k)."""
    g = rng(seed, _T_ZIPF, M)
    E = shape.n_routed
    pi = g.permutation(E)  # pi[e] = popularity rank (0-based) of expert e
    logp = -s * np.log(np.arange(1, E + 1, dtype=np.float64))
    gumbel = -np.log(-np.log(g.random((M, E))))
    return (logp[pi][None, :] + gumbel).astype(np.float32)


def random_logits(seed: int, M: int, E: int, scale: float = 1.0) -> np.ndarray:
    return (rng(seed, _T_MISC, M, E).standard_normal((M, E), dtype=np.float32) * np.float32(scale)).astype(np.float32)


def q8_0_weight(seed: int, K: int, N: int):
    """(int8 [N x K] uniform in [-127,127], fp16 scale bits [N x K/32] ~ U(1e-3,1e-2))."""
    g = rng(seed, _T_Q8, K, N)
    wq = g.integers(-127, 128, size=(N, K), dtype=np.int8)
    ws = g.uniform(1e-3, 1e-2, size=(N, K // 32)).astype(np.float16).view(np.uint16)
    return wq, ws


def q8_0_x(seed: int, M: int, K: int) -> np.ndarray:
    return rng(seed, _T_Q8, M, K, 1).standard_normal((M, K), dtype=np.float32)


def device_experts(shape: LayerShape, seed: int, device="cuda", ids=None):
    """All expert records of a layer (or only ``ids``, others left zero) in one
    device uint8 tensor of n_experts * stride bytes; generated on the host one
    record at a time and copied up."""
    import torch

    base = torch.zeros(shape.n_experts * shape.stride, dtype=torch.uint8, device=device)
    todo = range(shape.n_experts) if ids is None else ids
    for e, rec in expert_records(shape, seed, todo):
        base[e * shape.stride:(e + 1) * shape.stride].copy_(torch.from_numpy(rec), non_blocking=False)
    return base
