"""Workload definitions and seeded generators (no method arithmetic).

Workloads (shapes follow the GPT-2-small / GPT-2-XL hidden weights that the
Muon speedruns train, plus a single large square matrix and one Newton-Muon
layer):

  tiny    one 256x512 float32 matrix, G ~ N(0,1), M0 = 0, W ~ N(0,0.02)
  square  one 4096x4096 bfloat16 matrix, G = rank-32 factor product with a
          1/k spectrum plus N(0,1e-3) noise (fresh per step), M0 ~ N(0,1e-2),
          W ~ N(0,0.02); 10 consecutive steps
  gpt2s   12 layers x {Q,K,V,O 768x768, up 3072x768, down 768x3072} bfloat16,
          G = s_i * N(0,1e-2) with s_i ~ U(0.1,10) per matrix, M0 = 0
  gpt2xl  48 layers x {Q,K,V,O 1600x1600, up 6400x1600, down 1600x6400}
          bfloat16, G = rank-64 factor product + N(0,1e-3) noise, M0 = 0
  nmuon   one layer at d=768 with Newton-Muon: packed QKV 2304x768 (three
          768-row blocks), O 768x768, up 3072x768 sharing one S; down
          768x3072 with four S blocks; activations 16384x768 bfloat16 drawn
          N(0, Q diag(lambda) Q^T), lambda log-uniform in [1e-3, 1], Q Haar.
"""

from __future__ import annotations

import dataclasses
from typing import List, Optional

import numpy as np

F32 = "f32"
BF16 = "bf16"

_WL_ID = {"tiny": 1, "square": 2, "gpt2s": 3, "gpt2xl": 4, "nmuon": 5, "conv": 6, "gpt2s_aux": 7}
_KIND_ID = {"grad": 1, "mom": 2, "weight": 3, "acts": 4, "scale": 5,
            "gfac": 6, "gnoise": 7, "sigma": 8}


def rng_for(wl: str, layer: int, kind: str, step: int = 0) -> np.random.Generator:
    """Independent PCG64 stream per (workload, layer/matrix, kind, step)."""
    ss = np.random.SeedSequence([_WL_ID[wl], int(layer), _KIND_ID[kind], int(step)])
    return np.random.Generator(np.random.PCG64(ss))


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float64/float32 data to bfloat16 (nearest, ties to even) and
    return uint16 bit patterns.  Rounds from float32, which is exact for the
    bf16 grid decision only when the float32 value is not itself a rounded
    tie; inputs here are random draws, so this is a storage encoder, not a
    reference rounding."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    u = u + np.uint64(0x7FFF) + lsb
    return (u >> np.uint64(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclasses.dataclass(frozen=True)
class TensorSpec:
    name: str
    layer: int
    index: int            # global matrix index inside the workload (seed key)
    rows: int
    cols: int
    dtype: str            # F32 or BF16 (param and grad)
    split_rows: int = 0   # >0: orthogonalise row blocks of this height
    precond: int = -1     # preconditioner slot, -1 = none
    precond_blocks: int = 1
    kind: str = "muon"    # "muon" (hidden matrix) or "adamw" (embedding, gain, bias)
    shape: tuple = ()     # the parameter's own shape when it is not rows x cols (vectors)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    tensors: List[TensorSpec]
    steps: int = 1
    lr: float = 0.02
    weight_decay: float = 0.01
    momentum: float = 0.95
    ns_steps: int = 5
    grad_law: str = "gauss"     # "gauss", "gauss_scaled", "lowrank"
    grad_std: float = 1.0
    grad_rank: int = 0
    noise_std: float = 0.0
    mom0_std: float = 0.0
    act_rows: int = 0
    act_dim: int = 0


def _gpt2_layer(layer: int, base: int, d: int, dtype: str) -> List[TensorSpec]:
    return [
        TensorSpec("q", layer, base + 0, d, d, dtype),
        TensorSpec("k", layer, base + 1, d, d, dtype),
        TensorSpec("v", layer, base + 2, d, d, dtype),
        TensorSpec("attn_out", layer, base + 3, d, d, dtype),
        TensorSpec("mlp_up", layer, base + 4, 4 * d, d, dtype),
        TensorSpec("mlp_down", layer, base + 5, d, 4 * d, dtype),
    ]


def workload(name: str, layers: Optional[int] = None) -> Workload:
    """Build a workload description.  `layers` trims the GPT-2 sets (used by
    small parity cases); None means the full set."""
    if name == "tiny":
        return Workload("tiny", [TensorSpec("w", 0, 0, 256, 512, F32)],
                        grad_law="gauss", grad_std=1.0)
    if name == "square":
        return Workload("square", [TensorSpec("w", 0, 0, 4096, 4096, BF16)],
                        steps=10, grad_law="lowrank", grad_rank=32,
                        noise_std=1e-3, mom0_std=1e-2)
    if name == "gpt2s":
        n = 12 if layers is None else layers
        ts = [t for l in range(n) for t in _gpt2_layer(l, 6 * l, 768, BF16)]
        return Workload("gpt2s", ts, grad_law="gauss_scaled", grad_std=1e-2)
    if name == "gpt2xl":
        n = 48 if layers is None else layers
        ts = [t for l in range(n) for t in _gpt2_layer(l, 6 * l, 1600, BF16)]
        return Workload("gpt2xl", ts, grad_law="lowrank", grad_rank=64,
                        noise_std=1e-3)
    if name == "gpt2s_aux":
        # the GPT-2-small hidden matrices (Muon) plus every other parameter
        # of the model (AdamW): token and position embeddings (the head is
        # tied to the token embedding), per layer two layer-norm gains and
        # biases and the four linear biases, and the final layer norm
        d = 768
        ts = [t for l in range(12) for t in _gpt2_layer(l, 6 * l, d, BF16)]
        idx = 1000
        aux = [("wte", 50257, d, ()), ("wpe", 1024, d, ())]
        for l in range(12):
            for nm, n in (("ln1_g", d), ("ln1_b", d), ("attn_b", 3 * d), ("proj_b", d), ("ln2_g", d),
                          ("ln2_b", d), ("fc_b", 4 * d), ("fcproj_b", d)):
                aux.append((f"{nm}{l}", 1, n, (n,)))
        aux += [("lnf_g", 1, d, (d,)), ("lnf_b", 1, d, (d,))]
        for k, (nm, r, c, shp) in enumerate(aux):
            ts.append(TensorSpec(nm, -1, idx + k, r, c, BF16, kind="adamw", shape=shp))
        return Workload("gpt2s_aux", ts, grad_law="gauss_scaled", grad_std=1e-2)
    if name == "conv":
        # convolution filters of a small CIFAR-10-style network as the 2-D
        # views Muon orthogonalises, out x (in*kh*kw): three blocks of two
        # 3x3 convolutions (widths 64, 256, 256); the first (input) layer is
        # left to the auxiliary optimiser and is not part of the set
        shapes = [(64, 32 * 9), (64, 64 * 9), (256, 64 * 9), (256, 256 * 9), (256, 256 * 9),
                  (256, 256 * 9)]
        ts = [TensorSpec(f"conv{i}", i, i, r, c, BF16) for i, (r, c) in enumerate(shapes)]
        return Workload("conv", ts, grad_law="gauss_scaled", grad_std=1e-2)
    if name == "nmuon":
        d = 768
        ts = [TensorSpec("qkv", 0, 0, 3 * d, d, BF16, split_rows=d, precond=0),
              TensorSpec("attn_out", 0, 1, d, d, BF16, precond=0),
              TensorSpec("mlp_up", 0, 2, 4 * d, d, BF16, precond=0),
              TensorSpec("mlp_down", 0, 3, d, 4 * d, BF16, precond=1,
                         precond_blocks=4)]
        return Workload("nmuon", ts, grad_law="gauss_scaled", grad_std=1e-2,
                        act_rows=16384, act_dim=d)
    raise KeyError(name)


WORKLOADS = ("tiny", "square", "gpt2s", "gpt2xl", "conv", "nmuon", "gpt2s_aux")


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == F32:
        return x.astype(np.float32)
    return to_bf16_bits(x)


def gradient(wl: Workload, t: TensorSpec, step: int = 0) -> np.ndarray:
    """Gradient of tensor t at step `step`, in its stored dtype."""
    r, c = t.rows, t.cols
    if wl.grad_law == "gauss":
        g = rng_for(wl.name, t.index, "grad", step).standard_normal((r, c)) * wl.grad_std
    elif wl.grad_law == "gauss_scaled":
        s = rng_for(wl.name, t.index, "scale", step).uniform(0.1, 10.0)
        g = rng_for(wl.name, t.index, "grad", step).standard_normal((r, c)) * (wl.grad_std * s)
    elif wl.grad_law == "lowrank":
        k = wl.grad_rank
        rf = rng_for(wl.name, t.index, "gfac", step)
        L = rf.standard_normal((r, k))
        R = rf.standard_normal((c, k))
        spec = 1.0 / np.arange(1, k + 1)
        g = (L * spec) @ R.T / np.sqrt(k)
        g += rng_for(wl.name, t.index, "gnoise", step).standard_normal((r, c)) * wl.noise_std
    else:
        raise KeyError(wl.grad_law)
    return _store(g, t.dtype)


def momentum0(wl: Workload, t: TensorSpec) -> np.ndarray:
    """Initial momentum buffer (float32)."""
    if wl.mom0_std == 0.0:
        return np.zeros((t.rows, t.cols), np.float32)
    return (rng_for(wl.name, t.index, "mom").standard_normal((t.rows, t.cols))
            * wl.mom0_std).astype(np.float32)


def weight(wl: Workload, t: TensorSpec) -> np.ndarray:
    """Initial weight, N(0, 0.02), in the stored dtype."""
    w = rng_for(wl.name, t.index, "weight").standard_normal((t.rows, t.cols)) * 0.02
    return _store(w, t.dtype)


def activations(wl: Workload, slot_block: int) -> np.ndarray:
    """N x d bfloat16 activations for one preconditioner block, drawn
    N(0, Q diag(lam) Q^T) with lam log-uniform in [1e-3, 1] and Q Haar
    (QR of a Gaussian with the sign fix of R's diagonal)."""
    d, n = wl.act_dim, wl.act_rows
    rs = rng_for(wl.name, slot_block, "sigma")
    lam = np.exp(rs.uniform(np.log(1e-3), np.log(1.0), d))
    q, rr = np.linalg.qr(rs.standard_normal((d, d)))
    q = q * np.sign(np.diag(rr))
    z = rng_for(wl.name, slot_block, "acts").standard_normal((n, d))
    x = (z * np.sqrt(lam)) @ q.T
    return to_bf16_bits(x)
