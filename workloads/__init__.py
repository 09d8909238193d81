"""Seeded synthetic inputs for the five workloads of the NF4 QLoRA linear path.

This module only draws random numbers and stores them in the tensors' storage
dtypes (fp32, or bf16 rounded from fp32 by torch's CPU conversion).  It holds
none of the method's arithmetic, and it is the only module that both the HIP
path's tests / bench and the oracle use.

Recipe (weights are near-normal, as the pages assume: P2 §4.1, P4 §三):
  * numpy ``Generator(PCG64(SeedSequence(20230523 + workload_index)))``;
  * one spawned child stream per tensor, per layer in the order
    W, outlier indices, A, B, X, dY;
  * normals are drawn in fp64, scaled, rounded to fp32; bf16 tensors are the
    round-to-nearest-even of those fp32 values;
  * outliers (workloads 1 and 2): round(1e-3 * numel) distinct flat indices,
    multiplied by 10 in fp32;
  * W ~ N(0, 0.02^2); A ~ N(0, 0.02^2); B ~ N(0, 0.01^2); X, dY ~ N(0, 1).
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

SEED_BASE = 20230523


@dataclass(frozen=True)
class Workload:
    index: int
    name: str
    layers: tuple            # ((name, N, K), ...): N = out_features, K = in_features
    tokens: tuple            # M values
    rank: int
    alpha: float
    weight_dtype: str        # "f32" or "bf16": dtype handed to the quantizer
    outliers: bool
    backward: bool
    extra: dict = field(default_factory=dict)


_MLP7B = (("gate", 11008, 4096), ("up", 11008, 4096), ("down", 4096, 11008))
_ATTN7B = tuple((n, 4096, 4096) for n in ("q", "k", "v", "o"))
_ATTN65B = tuple((n, 8192, 8192) for n in ("q", "k", "v", "o"))
_MLP65B = (("gate", 22016, 8192), ("up", 22016, 8192), ("down", 8192, 22016))

WORKLOADS = {
    1: Workload(1, "tiny single linear 256x256", (("w", 256, 256),), (32,), 8, 16.0,
                "f32", True, True),
    2: Workload(2, "llama-7b q_proj 4096x4096 dequant-GEMV", (("q", 4096, 4096),), (1, 16),
                16, 32.0, "f32", True, False),
    3: Workload(3, "llama-7b MLP (gate, up 4096->11008; down 11008->4096)", _MLP7B, (4096,),
                64, 16.0, "f32", False, True),
    4: Workload(4, "llama-7b decoder block, 7 linears", _ATTN7B + _MLP7B, (8192,), 64, 16.0,
                "bf16", False, True, {"bulk_params": 6.7e9}),
    5: Workload(5, "65b-shaped layer, 7 linears", _ATTN65B + _MLP65B, (2048,), 64, 16.0,
                "bf16", False, True, {"bulk_params": 65e9}),
}


def _streams(w: Workload):
    ss = np.random.SeedSequence(SEED_BASE + w.index)
    kids = ss.spawn(6 * len(w.layers))
    return [np.random.Generator(np.random.PCG64(k)) for k in kids]


class Inputs:
    """Lazily drawn tensors of one workload.  ``layer`` indexes ``w.layers``."""

    def __init__(self, index: int):
        self.w = WORKLOADS[index]
        self._gens = _streams(self.w)

    def _gen(self, layer: int, slot: int):
        # a fresh copy of the child stream, so every call returns the same data
        g = self._gens[6 * layer + slot]
        return np.random.Generator(np.random.PCG64(g.bit_generator.seed_seq))

    def shape(self, layer: int):
        _, n, k = self.w.layers[layer]
        return n, k

    def weight_f32(self, layer: int) -> np.ndarray:
        n, k = self.shape(layer)
        W = (self._gen(layer, 0).standard_normal((n, k)) * 0.02).astype(np.float32)
        if self.w.outliers:
            numel = n * k
            cnt = int(round(1e-3 * numel))
            idx = self._gen(layer, 1).choice(numel, cnt, replace=False)
            flat = W.reshape(-1)
            flat[idx] = flat[idx] * np.float32(10.0)
        return W

    def weight(self, layer: int) -> np.ndarray:
        """The weight as handed to the quantizer: fp32, or bf16 bits (uint16)."""
        W = self.weight_f32(layer)
        return W if self.w.weight_dtype == "f32" else to_bf16_bits(W)

    def lora_A(self, layer: int) -> np.ndarray:
        _, k = self.shape(layer)
        return to_bf16_bits(self._gen(layer, 2).standard_normal((self.w.rank, k)) * 0.02)

    def lora_B(self, layer: int) -> np.ndarray:
        n, _ = self.shape(layer)
        return to_bf16_bits(self._gen(layer, 3).standard_normal((n, self.w.rank)) * 0.01)

    def X(self, layer: int, M: int) -> np.ndarray:
        _, k = self.shape(layer)
        return to_bf16_bits(self._gen(layer, 4).standard_normal((M, k)))

    def dY(self, layer: int, M: int) -> np.ndarray:
        n, _ = self.shape(layer)
        return to_bf16_bits(self._gen(layer, 5).standard_normal((M, n)))


def to_bf16_bits(a) -> np.ndarray:
    """fp64/fp32 array -> fp32 (nearest) -> bf16 bit patterns via torch."""
    import torch

    f32 = np.ascontiguousarray(np.asarray(a, dtype=np.float32))
    t = torch.from_numpy(f32).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_f32(b) -> np.ndarray:
    """bf16 bit patterns -> fp32 values (exact widening)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def random_bf16(shape, seed: int, scale: float = 1.0) -> np.ndarray:
    """Extra seeded N(0, scale^2) bf16 tensors for edge-case tests."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed)))
    return to_bf16_bits(g.standard_normal(shape) * scale)


def random_f32(shape, seed: int, scale: float = 1.0) -> np.ndarray:
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed)))
    return (g.standard_normal(shape) * scale).astype(np.float32)


def device_normal(torch, shape, seed: int, scale: float = 1.0, bf16: bool = True):
    """Seeded N(0, scale^2) drawn on the GPU with torch's counter-based Philox
    generator (fp32 draws, scaled, then rounded to bf16 unless bf16=False):
    the large inputs of the 7B-block and 65B-layer workloads and of the bulk
    quantization, where host generation would dominate the run.  The same
    (shape, seed) gives the same tensor on every call."""
    g = torch.Generator(device="cuda").manual_seed(int(seed))
    t = torch.randn(*shape, generator=g, device="cuda", dtype=torch.float32).mul_(scale)
    return t.to(torch.bfloat16) if bf16 else t


# Bulk quantization tensor lists (the totals the 7B-block and 65B workloads
# name; the two 32000-row embedding-shaped matrices only pad the totals):
# 32 x the seven 7B-block linears + 2 x 32000x4096 = 6.738e9 parameters;
# 80 x the seven 65B-layer linears + 2 x 32000x8192 = 65.29e9 parameters.
def bulk_tensors(index: int):
    w = WORKLOADS[index]
    reps, emb = (32, (32000, 4096)) if index == 4 else (80, (32000, 8192))
    out = []
    for rep in range(reps):
        for name, n, k in w.layers:
            out.append((f"layer{rep}.{name}", n, k))
    out += [("embed", emb[0], emb[1]), ("lm_head", emb[0], emb[1])]
    return out
