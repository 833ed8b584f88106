"""Seeded synthetic inputs for the attention workloads.

This module is shared by the HIP path's tests and benchmark and by the CPU
oracle's tests.  It holds no attention arithmetic: only a counter-based
random generator, the fp32 -> bf16 rounding that places the draws on the
device, the exact bf16 -> fp64 widening the oracle consumes, and the table of
workload shapes.

Generator (stated from its published definitions, no library RNG):
  * SplitMix64 (Steele, Lea, Flood, "Fast splittable pseudorandom number
    generators", OOPSLA 2014): element ``n`` of a stream with seed ``s`` is
    ``mix64(s + (n + 1) * 0x9E3779B97F4A7C15)``.
  * Box-Muller: two uniforms ``u1, u2`` in (0, 1] built from the top 53 bits
    of consecutive draws give ``sqrt(-2 ln u1) * (cos, sin)(2 pi u2)``;
    even elements take the cosine, odd ones the sine.
  * fp32 -> bf16 is round-to-nearest-even on the fp32 bit pattern (the same
    rule ``torch.Tensor.to(torch.bfloat16)`` applies; a CPU test checks it).

Per-tensor seeds: ``0xFA000000 + 16 * workload_id + tensor_id`` with
tensor_id Q=0, K=1, V=2, dO=3.
"""
from __future__ import annotations

import concurrent.futures as cf
import os

import numpy as np

GOLDEN = np.uint64(0x9E3779B97F4A7C15)
M1 = np.uint64(0xBF58476D1CE4E5B9)
M2 = np.uint64(0x94D049BB133111EB)

TENSOR_ID = {"q": 0, "k": 1, "v": 2, "do": 3, "lengths": 15}

# Workloads of the attention pages' evaluation, with the shapes they are
# quoted on.  ``id`` feeds the seed.  ``boost`` = (period, factor): every
# period-th query row is multiplied by factor before rounding to bf16, which
# makes scores of those rows large so that the running max keeps moving.
WORKLOADS = {
    "smoke_d64_s256": dict(id=1, B=1, H=2, S=256, d=64, causal=(False,), bwd=False, boost=None),
    "fwd_b4_h16_s4096": dict(id=2, B=4, H=16, S=4096, d=128, causal=(False,), bwd=False, boost=None),
    "causal_boost_b2_h16_s8192": dict(id=3, B=2, H=16, S=8192, d=128, causal=(True,), bwd=False,
                                      boost=(64, 8.0)),
    "causal_fwdbwd_b2_h16_s16384": dict(id=4, B=2, H=16, S=16384, d=128, causal=(True,), bwd=True,
                                        boost=None),
    "long_b1_h16_s32768": dict(id=5, B=1, H=16, S=32768, d=128, causal=(False, True), bwd=True,
                               boost=None),
}


def seed_for(workload_id: int, tensor: str) -> int:
    return 0xFA000000 + 16 * int(workload_id) + TENSOR_ID[tensor]


def _mix64(z: np.ndarray) -> np.ndarray:
    z = (z ^ (z >> np.uint64(30))) * M1
    z = (z ^ (z >> np.uint64(27))) * M2
    return z ^ (z >> np.uint64(31))


def splitmix64(seed: int, start: int, count: int) -> np.ndarray:
    """Draws ``start .. start+count-1`` of the SplitMix64 stream ``seed``."""
    idx = np.arange(start + 1, start + count + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        state = np.uint64(seed & 0xFFFFFFFFFFFFFFFF) + idx * GOLDEN
        return _mix64(state)


def _normal_pairs(seed: int, p0: int, p1: int, out: np.ndarray, n: int) -> None:
    raw = splitmix64(seed, 2 * p0, 2 * (p1 - p0)).reshape(-1, 2)
    u = ((raw >> np.uint64(11)).astype(np.float64) + 1.0) * (2.0 ** -53)
    r = np.sqrt(-2.0 * np.log(u[:, 0]))
    t = (2.0 * np.pi) * u[:, 1]
    pair = np.empty((p1 - p0, 2), dtype=np.float64)
    pair[:, 0] = r * np.cos(t)
    pair[:, 1] = r * np.sin(t)
    e0, e1 = 2 * p0, min(n, 2 * p1)
    out[e0:e1] = pair.reshape(-1)[: e1 - e0].astype(np.float32)


def normal_f32(seed: int, n: int, chunk: int = 1 << 21) -> np.ndarray:
    """``n`` N(0,1) draws as float32 (Box-Muller over SplitMix64 pairs).
    Chunks are independent slices of the same stream, filled by a thread
    pool (numpy releases the GIL); the result does not depend on ``chunk``."""
    out = np.empty(n, dtype=np.float32)
    npairs = (n + 1) // 2
    spans = [(p0, min(npairs, p0 + chunk)) for p0 in range(0, npairs, chunk)]
    if len(spans) <= 1:
        for p0, p1 in spans:
            _normal_pairs(seed, p0, p1, out, n)
        return out
    workers = min(len(spans), os.cpu_count() or 1, 16)
    with cf.ThreadPoolExecutor(max_workers=workers) as ex:
        list(ex.map(lambda sp: _normal_pairs(seed, sp[0], sp[1], out, n), spans))
    return out


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    with np.errstate(over="ignore"):
        return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float64."""
    return bf16_bits_to_f32(b).astype(np.float64)


def make_tensor_f32(workload_id: int, tensor: str, shape, boost=None) -> np.ndarray:
    """fp32 host draws for one tensor of shape [B, H, S, d]."""
    B, H, S, d = shape
    x = normal_f32(seed_for(workload_id, tensor), B * H * S * d).reshape(B, H, S, d)
    if boost is not None and tensor == "q":
        period, factor = boost
        x[:, :, ::period, :] *= np.float32(factor)
    return x


def make_tensor_bf16(workload_id: int, tensor: str, shape, boost=None) -> np.ndarray:
    """bf16 bit patterns (uint16) for one tensor of shape [B, H, S, d]."""
    return f32_to_bf16_bits(make_tensor_f32(workload_id, tensor, shape, boost))


def workload_inputs(name: str, tensors=("q", "k", "v", "do"), S=None, B=None, H=None):
    """bf16 bits for the named workload; B/H/S may be overridden (smaller
    cases with the same distribution and seeds)."""
    w = WORKLOADS[name]
    shape = (B or w["B"], H or w["H"], S or w["S"], w["d"])
    return {t: make_tensor_bf16(w["id"], t, shape, w["boost"]) for t in tensors}


# Packed variable-length prefill batches (forward only, causal): n sequence
# lengths, each `unit` times a SplitMix64 draw uniform in 1..max_units, so a
# mix of short and long prompts; tensors are [total, H, d] (token-major).
VARLEN_WORKLOADS = {
    "prefill_varlen_h16_d128": dict(id=6, n=16, unit=128, max_units=128, H=16, d=128, causal=True),
}


def varlen_lengths(name: str) -> np.ndarray:
    w = VARLEN_WORKLOADS[name]
    u = splitmix64(seed_for(w["id"], "lengths"), 0, w["n"])
    return (w["unit"] * (1 + (u % np.uint64(w["max_units"])))).astype(np.int64)


def varlen_inputs(name: str, tensors=("q", "k", "v")):
    """(lengths, bf16 bits [total, H, d] per tensor) for the named batch."""
    w = VARLEN_WORKLOADS[name]
    lens = varlen_lengths(name)
    total = int(lens.sum())
    shape = (total, w["H"], w["d"])
    bits = {t: f32_to_bf16_bits(normal_f32(seed_for(w["id"], t), total * w["H"] * w["d"]).reshape(shape))
            for t in tensors}
    return lens, bits


def default_scale(d: int) -> float:
    return 1.0 / float(np.sqrt(d))
