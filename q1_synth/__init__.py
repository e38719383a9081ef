"""Seeded synthetic inputs for the packed Q1 (1-bit affine, group 128) path.

This module is shared by the CPU oracle tests, the GPU parity tests, the
benchmark and the smoke check.  It only draws random numbers and stores them in
the formats the method consumes; it performs none of the method's arithmetic
(no unpacking, no dequantisation, no products).

Formats (Higgs PR #212 "Support Bonsai-27B affine Q1", section "What";
rMLX issue #207, section "The good news -- packing is standard"):

* packed weights: uint32 ``[N, K/32]``; each word holds 32 consecutive weights
  of one row, weight ``32*j + i`` in bit ``i`` of word ``j`` (LSB first);
* scales (and biases, for affine tensors): one value per 128-weight group along
  K, shape ``[N, K/128]``, stored as fp16 or bf16 bit patterns (uint16);
* activations: bf16 bit patterns (uint16), shape ``[M, K]``;
* token ids: int32.

The real Bonsai checkpoints are not available, so every tensor is drawn from
the distributions listed below with ``numpy.random.Generator(PCG64(seed))``,
always in the order bits, scales, biases, activations, ids.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch

GROUP = 128
META_F16 = "f16"
META_BF16 = "bf16"


def _to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 values -> bf16 bit patterns (uint16), rounding by torch's own
    float32->bfloat16 conversion (round to nearest even)."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def _to_f16_bits(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32).astype(np.float16).view(np.uint16).copy()


def meta_bits(a: np.ndarray, meta: str) -> np.ndarray:
    """Round float values to the metadata dtype and return the bit patterns."""
    if meta == META_F16:
        return _to_f16_bits(a)
    if meta == META_BF16:
        return _to_bf16_bits(a)
    raise ValueError(f"unknown metadata dtype {meta!r}")


def bf16_bits(a: np.ndarray) -> np.ndarray:
    return _to_bf16_bits(a)


@dataclasses.dataclass
class Q1Weight:
    """One packed Q1 matrix, host copy."""

    packed: np.ndarray            # uint32 [N, K/32]
    scales: np.ndarray            # uint16 bit patterns [N, K/128]
    biases: Optional[np.ndarray]  # uint16 bit patterns [N, K/128] or None (symmetric)
    meta: str                     # "f16" | "bf16"
    N: int
    K: int

    @property
    def symmetric(self) -> bool:
        return self.biases is None

    @property
    def metric_bytes(self) -> int:
        """Bytes of packed words plus metadata that one pass must read."""
        n = self.packed.nbytes + self.scales.nbytes
        if self.biases is not None:
            n += self.biases.nbytes
        return n


def draw_weight(rng: np.random.Generator, N: int, K: int, meta: str, symmetric: bool,
                scale_sigma: float = 0.02, bias_sigma: float = 0.01) -> Q1Weight:
    """Uniform random bits (i.i.d. Bernoulli(1/2)), scales |N(0, scale_sigma)|,
    biases N(0, bias_sigma) (affine only), metadata rounded to ``meta``."""
    if K % GROUP != 0:
        raise ValueError("K must be a multiple of 128")
    G = K // GROUP
    packed = rng.integers(0, 1 << 32, size=(N, K // 32), dtype=np.uint64).astype(np.uint32)
    scales = meta_bits(np.abs(rng.normal(0.0, scale_sigma, size=(N, G))), meta)
    biases = None
    if not symmetric:
        biases = meta_bits(rng.normal(0.0, bias_sigma, size=(N, G)), meta)
    return Q1Weight(packed, scales, biases, meta, N, K)


def draw_x(rng: np.random.Generator, M: int, K: int, sigma: float = 1.0) -> np.ndarray:
    """Activations N(0, sigma) rounded to bf16, returned as uint16 bit patterns [M, K]."""
    return bf16_bits(rng.normal(0.0, sigma, size=(M, K)))


def draw_ids(rng: np.random.Generator, T: int, vocab: int) -> np.ndarray:
    return rng.integers(0, vocab, size=(T,), dtype=np.int64).astype(np.int32)


# --------------------------------------------------------------------------
# The five workloads.  Shapes follow the Bonsai-27B (Qwen3.5-style) dense
# projections: hidden 5120, intermediate 17408, vocabulary 152064.
# --------------------------------------------------------------------------

@dataclasses.dataclass
class Workload:
    name: str
    weights: dict            # name -> Q1Weight
    x: dict                  # name -> uint16 bf16 bits [M, K]
    ids: Optional[np.ndarray]
    out_dtype: str           # "f32" | "bf16"
    Ms: tuple


def workload(index: int, max_m: int = 8, seed_offset: int = 1000, small: bool = False) -> Workload:
    """Build workload ``index`` (1..5), seeded with ``seed_offset + index``.

    ``small=True`` shrinks N (never K) so the oracle can check every output in
    seconds while still covering several tiles and a ragged tail.
    """
    rng = np.random.Generator(np.random.PCG64(seed_offset + index))
    if index == 1:
        w = draw_weight(rng, 1024, 1024, META_F16, True)
        x = draw_x(rng, 2, 1024)
        return Workload("tiny_1024x1024_sym_f16", {"w": w}, {"x": x}, None, "f32", (1, 2))
    if index == 2:
        N = 1000 + 37 if small else 17408
        w = draw_weight(rng, N, 5120, META_F16, True)
        x = draw_x(rng, max_m, 5120)
        return Workload("ffn_up_5120x17408_sym_f16", {"w": w}, {"x": x}, None, "bf16", tuple(range(1, max_m + 1)))
    if index == 3:
        N = 500 + 13 if small else 5120
        w = draw_weight(rng, N, 17408, META_BF16, False)
        x = draw_x(rng, 9, 17408)
        return Workload("ffn_down_17408x5120_affine_bf16", {"w": w}, {"x": x}, None, "bf16", tuple(range(1, 10)))
    if index == 4:
        V = 4096 + 77 if small else 152064
        w = draw_weight(rng, V, 5120, META_F16, True)
        x = draw_x(rng, 1, 5120)
        ids = draw_ids(rng, 64 if small else 4096, V)
        return Workload("lm_head_5120x152064_sym_f16", {"w": w}, {"x": x}, ids, "f32", (1,))
    if index == 5:
        H, I = 5120, 17408
        if small:
            I = 1024 + 128
        wg = draw_weight(rng, I, H, META_F16, True)
        wu = draw_weight(rng, I, H, META_F16, True)
        wd = draw_weight(rng, H if not small else 640, I, META_F16, True)
        x = draw_x(rng, 512 if not small else 40, H)
        return Workload("ffn_5120_17408_sym_f16", {"gate": wg, "up": wu, "down": wd}, {"x": x}, None, "bf16",
                        tuple(range(1, max_m + 1)))
    raise ValueError(f"no workload {index}")
