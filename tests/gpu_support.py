"""Shared set-up for the GPU parity tests: seeded inputs on the device, weights prepared by the
library's own kernels, and the oracle's view of the same draws (quantised by the oracle itself)."""
from __future__ import annotations

import functools

import numpy as np
import torch

import workloads
from mx_quantized_grouped_amd import binding as B
from mx_quantized_grouped_amd.weights import ExpertLoader
from oracle import moe

DEV = "cuda"


def bf16_tensor(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(bits.astype(np.uint16).view(np.int16)).to(DEV).view(torch.bfloat16)


def f64(bits: np.ndarray) -> np.ndarray:
    return workloads.f32_from_bf16_bits(bits).astype(np.float64)


def shape_of(w: workloads.Workload, logits_dtype="bf16") -> B.Shape:
    return B.Shape.of(w.T, w.H, w.E, w.top_k, w.I, w.w_fmt, logits_dtype)


def packed_weights(name: str):
    """Prepacked device weights of a workload (independent of T), built with mxmoe_quantize and
    mxmoe_prepack from the seeded fp32 draws. Cached: workloads that differ only in T share one
    weight set."""
    w = workloads.get(name)
    key = (w.H, w.E, w.I, w.w_fmt, w.seed)
    if key not in _PACKED:
        if len(_PACKED) >= 3:
            _PACKED.pop(next(iter(_PACKED)))
        loader = ExpertLoader(shape_of(w), DEV)
        workloads.draw_all_experts(w, threads=8, callback=loader.add_expert)
        packed = loader.finish(keep_canonical=True)
        torch.cuda.synchronize()
        _PACKED[key] = (loader, packed)
    return _PACKED[key]


_PACKED: dict = {}


def oracle_weights(w: workloads.Workload) -> moe.ExpertWeights:
    return moe.ExpertWeights.from_draws(lambda e: workloads.draw_expert(w, e), w.E, w.H, w.I,
                                        w.w_fmt)


@functools.lru_cache(maxsize=16)
def inputs(name: str):
    w = workloads.get(name)
    xb, lb = workloads.draw_x(w), workloads.draw_logits(w)
    return w, xb, lb


def sample_tokens(T: int, n: int, seed: int = 0) -> np.ndarray:
    if T <= n:
        return np.arange(T)
    rng = np.random.default_rng(seed)
    mid = rng.choice(np.arange(1, T - 1), size=n - 2, replace=False)
    return np.unique(np.concatenate([[0, T - 1], mid]))


@functools.lru_cache(maxsize=16)
def oracle_result(name: str, n_sample: int):
    w, xb, lb = inputs(name)
    toks = sample_tokens(w.T, n_sample)
    r = moe.moe_block(f64(xb), f64(lb), oracle_weights(w), w.top_k, w.act_fmt, tokens=toks)
    return r


def tolerance_ok(stats: dict) -> bool:
    # The block's output tolerance: max |err| <= 2e-2 * max |ref| and sum|err| / sum|ref| <= 5e-3.
    return stats["max_rel"] <= 2e-2 and stats["mean_rel"] <= 5e-3
