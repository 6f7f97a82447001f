"""Workload registry and seeded generators for synthetic linear layers and calibration activations.

The pages evaluate on real checkpoints (Llama 1B-13B, Qwen 0.5B-32B) and real calibration text
(AAAC summary, section 4); neither is available here, so these generators stand in for them with
the same matrix shapes:

* weights   W = bf16(0.02 * z * (1 + 19 m)),  z ~ N(0, 1),  m ~ Bernoulli(0.001)
              (N(0, 0.02) with 0.1 % of the entries scaled by 20, rounded to bf16);
* activations X[t, k] = c_k * Z / sqrt((E1 + E2) / 2),  c_k = exp(N(0, 1)) per column,
              Z ~ N(0, 1), E1, E2 ~ Exp(1), so Z / sqrt(chi2_4 / 4) is Student-t with 4 degrees
              of freedom (chi2_4 = 2 (E1 + E2)).

Every tensor has its own torch.Generator seeded with
``0xAAAC * 10**6 + cfg * 10**4 + layer * 16 + tensor_id``; activations are drawn in chunks of
8192 tokens from one generator, in order (Z, E1, E2 per chunk). Values depend on the device the
generator runs on (CPU and GPU streams differ), so one test always draws both sides' inputs from
the same device and copies them.
"""

from __future__ import annotations

import dataclasses
from typing import Iterator, List, Optional

import torch

# tensor ids inside one layer
Q, K, V, O, GATE, UP, DOWN = 0, 1, 2, 3, 4, 5, 6
X_ATTN, X_O, X_MLP, X_DOWN = 8, 9, 10, 11

CHUNK_TOKENS = 8192


@dataclasses.dataclass(frozen=True)
class MatrixSpec:
    name: str
    rows: int          # out features
    cols: int          # in features (the reduction axis of the importance)
    tensor_id: int
    x_id: int          # which activation stream feeds this matrix

    @property
    def numel(self) -> int:
        return self.rows * self.cols


@dataclasses.dataclass(frozen=True)
class QuantConfig:
    cfg_id: int
    name: str
    g: int             # scale group (consecutive weights along a row)
    S: int             # selection group (divides g)
    n: int             # table entries
    iters: int         # assign+refine iterations
    tokens: int        # calibration tokens per activation stream
    matrices: tuple
    layers: int = 1

    @property
    def numel_per_layer(self) -> int:
        return sum(m.numel for m in self.matrices)

    def x_streams(self):
        """(x_id, K) for every activation stream of one layer, in tensor-id order."""
        seen = {}
        for m in self.matrices:
            if m.x_id not in seen:
                seen[m.x_id] = m.cols
            elif seen[m.x_id] != m.cols:
                raise ValueError("matrices sharing an activation stream must share C")
        return sorted(seen.items())


def _decoder(hidden: int, kv: int, mlp: int) -> tuple:
    return (
        MatrixSpec("q_proj", hidden, hidden, Q, X_ATTN),
        MatrixSpec("k_proj", kv, hidden, K, X_ATTN),
        MatrixSpec("v_proj", kv, hidden, V, X_ATTN),
        MatrixSpec("o_proj", hidden, hidden, O, X_O),
        MatrixSpec("gate_proj", mlp, hidden, GATE, X_MLP),
        MatrixSpec("up_proj", mlp, hidden, UP, X_MLP),
        MatrixSpec("down_proj", hidden, mlp, DOWN, X_DOWN),
    )


CONFIGS = {
    1: QuantConfig(1, "single 2048x2048 linear, INT4 g=128", 128, 128, 16, 8, 512,
                   (MatrixSpec("linear", 2048, 2048, Q, X_ATTN),)),
    2: QuantConfig(2, "Llama-3-8B-shaped decoder layer, INT4 g=128, selector in scale sign bit",
                   128, 128, 16, 10, 128 * 2048, _decoder(4096, 1024, 14336)),
    3: QuantConfig(3, "8B-shaped decoder layer, NVFP4-style g=16, 15-entry tables",
                   16, 16, 15, 10, 128 * 2048, _decoder(4096, 1024, 14336)),
    4: QuantConfig(4, "13B-shaped MLP, g=128, selection group S=16 in a 1-bit map",
                   128, 16, 16, 10, 256 * 2048,
                   (MatrixSpec("gate_proj", 13824, 5120, GATE, X_MLP),
                    MatrixSpec("up_proj", 13824, 5120, UP, X_MLP),
                    MatrixSpec("down_proj", 5120, 13824, DOWN, X_DOWN))),
    5: QuantConfig(5, "32B-shaped model, 64 decoder layers streamed, INT4 g=128",
                   128, 128, 16, 10, 256 * 2048, _decoder(5120, 1024, 27648), layers=64),
}


def config(cfg_id: int) -> QuantConfig:
    return CONFIGS[cfg_id]


def seed_for(cfg_id: int, layer: int, tensor_id: int) -> int:
    # C2 and C3 are the same layer quantized two ways: they share seeds.
    base_cfg = 2 if cfg_id == 3 else cfg_id
    return 0xAAAC * 10**6 + base_cfg * 10**4 + layer * 16 + tensor_id


def make_weight(rows: int, cols: int, seed: int, device="cpu",
                out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """bf16 [rows, cols] weight: N(0, 0.02) with 0.1 % of the entries scaled x20."""
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    z = torch.randn(rows, cols, generator=gen, device=device, dtype=torch.float32)
    m = torch.rand(rows, cols, generator=gen, device=device, dtype=torch.float32) < 0.001
    z.mul_(0.02)
    z.mul_(torch.where(m, 20.0, 1.0))
    del m
    w = z.to(torch.bfloat16)
    if out is not None:
        out.copy_(w)
        return out
    return w


def activation_chunks(tokens: int, cols: int, seed: int, device="cpu",
                      chunk: int = CHUNK_TOKENS) -> Iterator[torch.Tensor]:
    """Yield fp32 [<=chunk, cols] calibration activations, Student-t(4) rows with a
    LogNormal(0, 1) scale per column, in token order from one generator."""
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    c = torch.randn(cols, generator=gen, device=device, dtype=torch.float32).exp_()
    done = 0
    while done < tokens:
        t = min(chunk, tokens - done)
        z = torch.randn(t, cols, generator=gen, device=device, dtype=torch.float32)
        e = torch.empty(t, cols, device=device, dtype=torch.float32).exponential_(generator=gen)
        e2 = torch.empty(t, cols, device=device, dtype=torch.float32).exponential_(generator=gen)
        e.add_(e2).mul_(0.5).sqrt_()
        del e2
        z.div_(e).mul_(c)
        del e
        yield z
        done += t


def make_activations(tokens: int, cols: int, seed: int, device="cpu",
                     chunk: int = CHUNK_TOKENS) -> torch.Tensor:
    """All chunks of one activation stream, concatenated into one fp32 [tokens, cols] tensor."""
    out = torch.empty(tokens, cols, device=device, dtype=torch.float32)
    row = 0
    for x in activation_chunks(tokens, cols, seed, device, chunk):
        out[row:row + x.shape[0]].copy_(x)
        row += x.shape[0]
    return out


def layer_matrices(cfg: QuantConfig, layer: int = 0, device="cpu") -> List[torch.Tensor]:
    return [make_weight(m.rows, m.cols, seed_for(cfg.cfg_id, layer, m.tensor_id), device)
            for m in cfg.matrices]
