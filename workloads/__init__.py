"""Seeded synthetic inputs for the MX-quantised MoE expert block.

This module is shared by the GPU path's callers (tests, bench) and by the CPU oracle. It holds
random draws and bit-level rounding of those draws to the input storage type (bf16) only. It holds
none of the block's arithmetic: no routing, no sort, no MX quantisation, no GEMM. Weights are
handed out as fp32 draws; each side turns them into MX codes with its own quantiser.

Workloads are one GPU's share of the serving shapes described in "Lần theo điểm nghẽn: Tối ưu
MiniMax M3 trên AMD Instinct MI355X" (decode batches at concurrency 32/128 with the expert
intermediate split by TP4/TP2, one 8K-token prefill) and in "Ling-3.0-flash: Tối ưu hóa độ trễ
giải mã lên 54% trên 4 GPU Blackwell" (a 512-expert MoE at batch 1 and a 6-token verify window).
The pages measure on serving benchmarks that are not available here; these seeded draws stand in
for the MoE inputs those benchmarks would produce.

Draw recipe (per workload, seed s):
  * x      : [T, H]  N(0, 1) in fp32, rounded to bf16 (round to nearest even).
  * logits : [T, E]  N(0, 1) in fp32, plus (for Zipf workloads) a per-expert bias
             b_e = -1.1 * ln(e + 1) added in fp32, then rounded to bf16. Softmax routing then picks
             expert e with odds proportional to (e + 1)^-1.1, i.e. Zipf(s = 1.1) popularity.
  * gate   : [E, H]  N(0, 1/H) in fp32, rounded to bf16 (for the router gate in front of the
             routing step; logits = x . gate^T are then about N(0, 1)).
  * weights: for each expert e in 0..E (E is the shared expert) an independent stream gives
             W13 [2I, H] (gate rows 0..I-1, then up rows I..2I-1) and then W2 [H, I],
             N(0, 0.02) in fp32 (standard normal times 0.02 in fp32). bf16 workloads round them to
             bf16; MX workloads quantise them (each side with its own quantiser).
"""
from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, replace

import numpy as np

__all__ = [
    "Workload", "WORKLOADS", "get", "bf16_bits_from_f32", "f32_from_bf16_bits", "draw_gate",
    "draw_x", "draw_logits", "draw_expert", "draw_all_experts",
]


@dataclass(frozen=True)
class Workload:
    name: str
    T: int           # tokens
    H: int           # hidden size (K of gate_up, N of down)
    E: int           # routed experts; the shared expert has id E
    top_k: int       # routed experts per token
    I: int           # per-GPU expert intermediate size (N/2 of gate_up, K of down)
    w_fmt: str       # "bf16" | "mxfp8" | "mxfp4"
    act_fmt: str     # "bf16" | "mxfp8" | "mxfp4" (MXFP4 with MXFP4 weights only)
    zipf: bool       # add the Zipf(1.1) popularity bias to the router logits
    seed: int = 0
    description: str = ""

    @property
    def slots(self) -> int:
        return self.T * (self.top_k + 1)

    def with_T(self, T: int) -> "Workload":
        return replace(self, T=T, name=f"{self.name.rsplit('_T', 1)[0]}_T{T}")


def _wide(T: int, act: str = "mxfp8") -> Workload:
    tag = "mxfp4" if act == "mxfp8" else "w4a4"
    return Workload(f"wide512_{tag}_T{T}", T, 2048, 512, 8, 512, "mxfp4", act, True,
                    description="512 routed experts top-8 + shared, hidden 2048, intermediate 512, "
                                f"MXFP4 weights, {act.upper()} activations, Zipf(1.1) routing")


WORKLOADS = {
    w.name: w for w in [
        Workload("tiny_bf16", 16, 256, 8, 2, 128, "bf16", "bf16", False,
                 description="tiny bf16 block (no quantisation): 8 routed experts top-2 + shared"),
        Workload("decode_mxfp8", 32, 3072, 128, 8, 384, "mxfp8", "mxfp8", False,
                 description="decode batch 32, TP4 share (I=384), MXFP8 weights and activations"),
        Workload("prefill_mxfp8", 8192, 3072, 128, 8, 384, "mxfp8", "mxfp8", True,
                 description="one 8K-token prefill, TP4 share, MXFP8, Zipf(1.1) expert popularity"),
        Workload("decode_mxfp4", 128, 3072, 128, 8, 768, "mxfp4", "mxfp8", False,
                 description="decode batch 128, TP2 share (I=768), MXFP4 weights, MXFP8 activations"),
        _wide(1), _wide(6), _wide(4096),
        # W4A4: both MFMA operands E2M1 (the activations and the intermediate quantised to MXFP4)
        Workload("decode_w4a4", 128, 3072, 128, 8, 768, "mxfp4", "mxfp4", False,
                 description="decode batch 128, TP2 share (I=768), MXFP4 weights and activations"),
        _wide(4096, "mxfp4"),
    ]
}


def get(name: str) -> Workload:
    return WORKLOADS[name]


# ---------------------------------------------------------------- storage rounding of draws
def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even); returns the uint16 bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    return ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)


def f32_from_bf16_bits(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to fp32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# ---------------------------------------------------------------- streams
_X, _LOGITS, _W, _GATE = 0, 1, 2, 3


def _rng(seed: int, *key: int) -> np.random.Generator:
    return np.random.Generator(np.random.SFC64(np.random.SeedSequence(seed, spawn_key=key)))


def draw_x(w: Workload) -> np.ndarray:
    """Activations as bf16 bit patterns, [T, H] uint16."""
    z = _rng(w.seed, _X).standard_normal((w.T, w.H), dtype=np.float32)
    return bf16_bits_from_f32(z)


def zipf_bias(E: int) -> np.ndarray:
    return np.array([-1.1 * math.log(e + 1.0) for e in range(E)], dtype=np.float32)


def draw_logits(w: Workload) -> np.ndarray:
    """Router logits as bf16 bit patterns, [T, E] uint16."""
    z = _rng(w.seed, _LOGITS).standard_normal((w.T, w.E), dtype=np.float32)
    if w.zipf:
        z = (z + zipf_bias(w.E)[None, :]).astype(np.float32)
    return bf16_bits_from_f32(z)


def draw_gate(w: Workload) -> np.ndarray:
    """Router gate weights as bf16 bit patterns, [E, H] uint16: N(0, 1/H) in fp32 (standard normal
    times 1/sqrt(H)), so that with N(0, 1) activations the logits are about N(0, 1), the logit
    distribution of the drawn-logits workloads."""
    z = _rng(w.seed, _GATE).standard_normal((w.E, w.H), dtype=np.float32)
    return bf16_bits_from_f32(z * np.float32(1.0 / math.sqrt(w.H)))


def draw_expert(w: Workload, e: int):
    """fp32 draws for expert e (0..E; E is the shared expert): (W13 [2I, H], W2 [H, I]).

    For bf16 workloads the draws are returned already rounded to bf16 (as fp32 values)."""
    if not 0 <= e <= w.E:
        raise IndexError(e)
    g = _rng(w.seed, _W, e)
    w13 = g.standard_normal((2 * w.I, w.H), dtype=np.float32) * np.float32(0.02)
    w2 = g.standard_normal((w.H, w.I), dtype=np.float32) * np.float32(0.02)
    if w.w_fmt == "bf16":
        w13 = f32_from_bf16_bits(bf16_bits_from_f32(w13))
        w2 = f32_from_bf16_bits(bf16_bits_from_f32(w2))
    return w13, w2


def draw_all_experts(w: Workload, threads: int = 8, callback=None):
    """Draw every expert (0..E) in parallel. With `callback(e, w13, w2)` the arrays are handed
    over one expert at a time (and not kept); otherwise a list of (w13, w2) is returned."""
    out = [None] * (w.E + 1) if callback is None else None
    threads = max(1, threads)
    with ThreadPoolExecutor(threads) as ex:
        futs = {}
        nxt = 0
        for e in range(w.E + 1):
            while nxt <= w.E and nxt < e + 2 * threads:    # bounded look-ahead
                futs[nxt] = ex.submit(draw_expert, w, nxt)
                nxt += 1
            a, b = futs.pop(e).result()
            if callback is None:
                out[e] = (a, b)
            else:
                callback(e, a, b)
    return out


# ---------------------------------------------------------------- exact-arithmetic draws
def draw_exact_block(T: int, H: int, E: int, top_k: int, I: int, seed: int = 0):
    """Inputs on which every step of the block is exact in fp32, for bit-for-bit parity checks of
    the GEMM operand and scale layouts (the integer-exact construction).

    Every value is a small integer times a power of two, chosen so that its MX block maximum makes
    it land on the E4M3 and E2M1 grids exactly (no rounding at Q1 or at weight quantisation):
      * x[t, h]: one of 0, +-1, +-2 times 2^p (p in -1..1, per 32-block), except x[t, 0] = 16 (its
        block keeps p = 0). bf16-exact.
      * logits: for each token top_k distinct experts get 1.0, the others one of -1, -0.5, 0, 0.5;
        the selected logits are equal, so every routed weight is exp(0) / top_k (top_k a power of
        two keeps it exact) and ties order the selection by expert index.
      * W13 gate row n < I: 4 at column 0, and 4 further columns with +-2^p (p in -1..0 per
        block); with x[t, 0] = 16 the gate pre-activation is then 64 +- 16 >= 48, where
        SiLU(g) = g / (1 + e^-g) equals g in fp32 and fp64 (e^-48 < 2^-53).
      * W13 up row: 16 columns with one of +-1, +-2 times 2^p (p in -1..1 per block); in every
        32-block holding a nonzero, the largest magnitude is 1 or 2 times 2^p.
      * W2 row: about one column in eight with one of +-1, +-2 times 2^p.
    Returns (x bf16 bits [T, H], logits bf16 bits [T, E], [(w13 fp32 [2I, H], w2 fp32 [H, I])]
    for experts 0..E)."""
    if top_k & (top_k - 1):
        raise ValueError("top_k must be a power of two for exact routing weights")
    rng = _rng(seed, 9)
    nb = H // 32

    def block_pow(rows, blocks, lo, hi):
        return np.repeat(2.0 ** rng.integers(lo, hi + 1, size=(rows, blocks)), 32, axis=1)

    x = rng.integers(-2, 3, size=(T, H)).astype(np.float64) * block_pow(T, nb, -1, 1)
    x[:, :32] = rng.integers(-2, 3, size=(T, 32))
    x[:, 0] = 16.0
    lg = rng.choice(np.array([-1.0, -0.5, 0.0, 0.5]), size=(T, E))
    for t in range(T):
        lg[t, rng.choice(E, size=top_k, replace=False)] = 1.0
    experts = []
    for _ in range(E + 1):
        w13 = np.zeros((2 * I, H))
        gp = block_pow(I, nb, -1, 0)
        for n in range(I):
            w13[n, 0] = 4.0
            cols = rng.choice(np.arange(1, H), size=4, replace=False)
            w13[n, cols] = rng.choice([-1.0, 1.0], size=4) * gp[n, cols]
        up = block_pow(I, nb, -1, 1)
        for n in range(I):
            cols = rng.choice(H, size=16, replace=False)
            w13[I + n, cols] = rng.choice([-2.0, -1.0, 1.0, 2.0], size=16) * up[n, cols]
        w2 = np.zeros((H, I))
        dp = block_pow(H, I // 32, -1, 1)
        mask = rng.random((H, I)) < 0.125
        w2[mask] = rng.choice([-2.0, -1.0, 1.0, 2.0], size=int(mask.sum())) * dp[mask]
        experts.append((w13.astype(np.float32), w2.astype(np.float32)))
    return (bf16_bits_from_f32(x.astype(np.float32)), bf16_bits_from_f32(lg.astype(np.float32)),
            experts)
