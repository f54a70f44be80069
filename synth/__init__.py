"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module holds no arithmetic of the codec: it only draws random numbers,
rounds them to BF16 with torch's own cast, and describes the workloads (their
shapes, value distributions and the codebook model a user would pick for them).
Both the oracle and the HIP path consume the exact bytes produced here.

The workloads stand in for the pages' training runs (a 162M-parameter
NanoGPT and Qwen3-4B fine-tuning, explainer "LCT paper - Lossless Huffman
coding of BF16 training tensors", results table), whose data and trained
weights are not available: the shapes follow those models and the values
follow the distributions named for each tensor.  Per-tensor seed is
1000 * config + tensor index; host draws use numpy's PCG64, device draws use
torch's CUDA generator.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

GAUSSIAN, LAPLACE, POWERLAW = 0, 1, 2
CLEAN, MEDIUM, HIGH = 0, 1, 2


def to_bf16_bits(a) -> np.ndarray:
    """float64/float32 array -> BF16 bit patterns (uint16), round-to-nearest-even."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


@dataclass
class Model:
    """Codebook model a user picks for a tensor: family, scale, shape (t's dof)."""
    family: int
    scale: float
    shape: float = 0.0


@dataclass
class TensorSpec:
    name: str
    shape: tuple
    seed: int
    kind: str                 # generator kind
    args: dict = field(default_factory=dict)

    @property
    def numel(self) -> int:
        n = 1
        for d in self.shape:
            n *= d
        return n


# ------------------------------------------------------------------ draws

def draw(spec: TensorSpec) -> np.ndarray:
    """Host draw of one tensor as BF16 bit patterns (uint16, flat)."""
    g = rng(spec.seed)
    n = spec.numel
    k = spec.kind
    a = spec.args
    if k == "normal":
        v = g.normal(0.0, a["sigma"], n)
    elif k == "laplace":
        v = g.laplace(0.0, a["b"], n)
    elif k == "student_t":
        v = a["scale"] * g.standard_t(a["dof"], n)
    elif k == "shifted_normal":
        chunk = a["chunk"]
        ks = g.integers(a["kmin"], a["kmax"] + 1, size=-(-n // chunk))
        v = g.normal(0.0, 1.0, n) * np.repeat(np.ldexp(1.0, ks), chunk)[:n]
    elif k == "silu":
        x = g.normal(0.0, 1.0, n)
        v = x / (1.0 + np.exp(-x))
    elif k == "outlier_normal":
        v = g.normal(0.0, 1.0, n)
        hit = g.random(n) < a["frac"]
        v[hit] *= a["mult"]
    elif k == "uniform_bits":
        return g.integers(0, 1 << 16, size=n, dtype=np.uint16)
    else:
        raise ValueError(k)
    return to_bf16_bits(v)


def draw_device(spec: TensorSpec, device="cuda") -> torch.Tensor:
    """Device draw of a Gaussian tensor (for sets too large for host generation).
    Returns a flat torch.bfloat16 tensor; deterministic for a given seed."""
    if spec.kind != "normal":
        raise ValueError("device draws are only used for Gaussian parameter sets")
    gen = torch.Generator(device=device)
    gen.manual_seed(spec.seed)
    v = torch.randn(spec.numel, generator=gen, device=device, dtype=torch.float32)
    v.mul_(spec.args["sigma"])
    return v.to(torch.bfloat16)


# ------------------------------------------------------------------ workloads

def config1():
    """2^20 elements ~ N(0, 0.02^2); CLEAN; Gaussian(0.02) model."""
    return [(TensorSpec("w", (1 << 20,), 1000, "normal", {"sigma": 0.02}),
             Model(GAUSSIAN, 0.02))]


def config2(n=1 << 26):
    """Three 2^26-element tensors: Laplace(0.01), 0.01*t(3), N(0,1)*2^k per 2^20 chunk."""
    return [
        (TensorSpec("laplace", (n,), 2000, "laplace", {"b": 0.01}), Model(LAPLACE, 0.01)),
        (TensorSpec("student_t3", (n,), 2001, "student_t", {"dof": 3.0, "scale": 0.01}),
         Model(POWERLAW, 0.01, 3.0)),
        (TensorSpec("shifted", (n,), 2002, "shifted_normal",
                    {"chunk": 1 << 20, "kmin": -12, "kmax": 4}), Model(GAUSSIAN, 1.0)),
    ]


def gpt162m_shapes():
    """12 layers, d=768: qkv, attention out, MLP in/out; token embedding and untied head."""
    shapes = []
    for layer in range(12):
        shapes += [(f"h{layer}.qkv", (768, 2304)), (f"h{layer}.proj", (768, 768)),
                   (f"h{layer}.fc", (768, 3072)), (f"h{layer}.fc_proj", (3072, 768))]
    shapes += [("wte", (50304, 768)), ("lm_head", (50304, 768))]
    return shapes


def config3():
    """GPT-style 162M parameter set: W ~ N(0, 0.02^2), M ~ N(0, 1e-3^2), eta = 1e-3."""
    w, m = [], []
    for i, (name, shp) in enumerate(gpt162m_shapes()):
        w.append(TensorSpec("W." + name, shp, 3000 + 2 * i, "normal", {"sigma": 0.02}))
        m.append(TensorSpec("M." + name, shp, 3000 + 2 * i + 1, "normal", {"sigma": 1e-3}))
    return w, m, Model(GAUSSIAN, 0.02), Model(GAUSSIAN, 1e-3), 1e-3


def config4():
    """One Qwen3-4B-shaped layer's activations at batch 1, seq 3500."""
    seq, hid, ffn = 3500, 2560, 9728
    return [
        (TensorSpec("silu_gate", (seq, ffn), 4000, "silu"), Model(LAPLACE, 0.25)),
        (TensorSpec("residual", (seq, hid), 4001, "outlier_normal", {"frac": 1e-3, "mult": 50.0}),
         Model(GAUSSIAN, 1.0)),
        (TensorSpec("uniform_bits", (seq, hid), 4002, "uniform_bits"), Model(GAUSSIAN, 1.0)),
    ]


def qwen3_4b_shapes():
    """Qwen3-4B-shaped parameter set with tied embeddings (36 layers, hidden 2560,
    FFN 9728, 32 q heads / 8 kv heads of dim 128, vocab 151936): 4,022,468,096."""
    hid, ffn, nq, nkv, hd, vocab = 2560, 9728, 32, 8, 128, 151936
    shapes = [("embed", (vocab, hid))]
    for layer in range(36):
        p = f"l{layer}."
        shapes += [(p + "q", (hid, nq * hd)), (p + "k", (hid, nkv * hd)),
                   (p + "v", (hid, nkv * hd)), (p + "o", (nq * hd, hid)),
                   (p + "gate", (hid, ffn)), (p + "up", (hid, ffn)), (p + "down", (ffn, hid)),
                   (p + "ln1", (hid,)), (p + "ln2", (hid,)),
                   (p + "q_norm", (hd,)), (p + "k_norm", (hd,))]
    shapes.append(("final_norm", (hid,)))
    return shapes


def config5():
    """Qwen3-4B-shaped set, flat: W ~ N(0, 0.02^2), M ~ N(0, 1e-3^2), eta = 1e-3."""
    n = sum(int(np.prod(s)) for _, s in qwen3_4b_shapes())
    w = TensorSpec("W.flat", (n,), 5000, "normal", {"sigma": 0.02})
    m = TensorSpec("M.flat", (n,), 5001, "normal", {"sigma": 1e-3})
    return w, m, Model(GAUSSIAN, 0.02), Model(GAUSSIAN, 1e-3), 1e-3


def mode_layout(mode: int):
    """(block_elems, cap_words) of the three modes: CLEAN 65536 / 25 words,
    MEDIUM 32768 / 12, HIGH 32768 / 11."""
    return {CLEAN: (65536, 25), MEDIUM: (32768, 12), HIGH: (32768, 11)}[mode]
