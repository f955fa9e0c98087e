"""Seeded synthetic inputs shared by the CPU oracle, the GPU parity tests and the bench.

This module only draws and lays out inputs: random Q/K/V/dO, position ids, the
fp32 cos/sin tables a FLUX-style caller hands to rotary attention, and key-padding
masks.  It holds none of the attention arithmetic (no rotation, no scores, no
softmax); both the oracle and the HIP path consume exactly the tensors built here.

Sources for the recipes (pages are cited by title and section):
  * "Metal Flash Attention" (SimpleTuner docs), section "Fused RoPE + SDPA":
    tensors are BHSD; cos/sin tables are pair-duplicated (entry 2i equals entry
    2i+1), shaped [S, D], [1, S, D] or per-sample [B, S, D], and normalised to fp32;
    the models differ only in how the caller builds the tables.
  * same page, section "FLUX Sequence Lengths": FLUX.1 attention is
    B,H,S,D = 1,24,S,128.
  * same page, section "Enable In SimpleTuner": bool masks (True = attend), additive
    masks, batched [B,H,Sq,Skv] and broadcast [B,1,1,Skv] shapes.

Readings where the pages are silent:
  * RoPE frequencies: omega_p = theta ** (-2p/d) for pair p < d/2 of an axis of
    width d, angle = position * omega_p, computed in float64 and rounded to fp32
    once.  Multi-axis tables concatenate the per-axis pairs in axis order.
  * FLUX packing: text tokens first with ids (0,0,0); image token (r, c) of a G x G
    grid follows row-major with ids (0, r, c).
  * Random numbers: numpy PCG64 seeded from SeedSequence([seed, stream]); draws are
    float32 N(0, 1), cast to bf16/fp16 by round-to-nearest-even on the host.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

# Independent random streams per tensor role, so that changing one tensor's shape
# never changes another tensor's values.
STREAM_Q, STREAM_K, STREAM_V, STREAM_DO, STREAM_LEN, STREAM_TAB, STREAM_NORM = 1, 2, 3, 4, 5, 6, 7
STREAM_LAYER = 100  # + 2 * layer (K) and + 2 * layer + 1 (V) of a chain

_TORCH_DTYPES = {
    "f32": torch.float32,
    "f16": torch.float16,
    "bf16": torch.bfloat16,
}


def rng(seed: int, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, stream])))


def normal(seed: int, stream: int, shape, dtype: str = "bf16", std: float = 1.0) -> torch.Tensor:
    """N(0, std^2) drawn in float32 and cast (RNE) to `dtype` on the CPU."""
    x = rng(seed, stream).standard_normal(size=tuple(shape), dtype=np.float32)
    if std != 1.0:
        x = x * np.float32(std)
    return torch.from_numpy(x).to(_TORCH_DTYPES[dtype])


def norm_weights(seed: int, dim: int):
    """Per-dimension RMSNorm weights for Q and K: fp32 [dim] each, 1 + 0.25 N(0, 1) (learned
    weights stay near their initial value of one)."""
    x = rng(seed, STREAM_NORM).standard_normal(size=(2, dim), dtype=np.float32)
    w = torch.from_numpy(np.float32(1.0) + np.float32(0.25) * x)
    return w[0].clone(), w[1].clone()


def rope_angles(positions: np.ndarray, dim: int, theta: float) -> np.ndarray:
    """Angles [S, dim/2] in float64 for one axis of width `dim`."""
    assert dim % 2 == 0
    p = np.arange(dim // 2, dtype=np.float64)
    omega = theta ** (-2.0 * p / dim)
    return np.asarray(positions, dtype=np.float64)[:, None] * omega[None, :]


def rope_tables(ids: np.ndarray, axes_dim, theta: float = 10000.0):
    """Pair-duplicated fp32 cos/sin tables [S, D] from integer position ids [S, n_axes].

    D = sum(axes_dim).  Per axis a, pairs of width axes_dim[a] use ids[:, a].
    """
    ids = np.asarray(ids)
    if ids.ndim == 1:
        ids = ids[:, None]
    assert ids.shape[1] == len(axes_dim)
    ang = np.concatenate(
        [rope_angles(ids[:, a], d, theta) for a, d in enumerate(axes_dim)], axis=1
    )  # [S, D/2]
    ang = np.repeat(ang, 2, axis=1)  # pair duplication: column 2i and 2i+1 share an angle
    cos = torch.from_numpy(np.cos(ang).astype(np.float32))
    sin = torch.from_numpy(np.sin(ang).astype(np.float32))
    return cos, sin


def flux_ids(n_text: int, grid: int) -> np.ndarray:
    """[n_text + grid*grid, 3] ids: text (0,0,0) first, then image (0, r, c) row-major."""
    txt = np.zeros((n_text, 3), dtype=np.int64)
    r, c = np.meshgrid(np.arange(grid), np.arange(grid), indexing="ij")
    img = np.stack([np.zeros(grid * grid, dtype=np.int64), r.ravel(), c.ravel()], axis=1)
    return np.concatenate([txt, img], axis=0)


def key_padding_lengths(seed: int, batch: int, lo: int = 64, hi: int = 512) -> np.ndarray:
    """Valid text length per batch item, uniform integers in [lo, hi] inclusive."""
    return rng(seed, STREAM_LEN).integers(lo, hi + 1, size=batch)


def key_padding_mask(lengths, n_text: int, seq: int) -> torch.Tensor:
    """Bool [B, 1, 1, S]: text key j valid iff j < L_b; image keys (j >= n_text) always valid."""
    B = len(lengths)
    j = torch.arange(seq)
    m = torch.zeros(B, 1, 1, seq, dtype=torch.bool)
    for b, L in enumerate(lengths):
        m[b, 0, 0] = (j < int(L)) | (j >= n_text)
    return m


def expand_additive(bool_mask: torch.Tensor, heads: int, seq_q: int, dtype: str = "bf16") -> torch.Tensor:
    """The same pattern as an additive 0 / -inf mask expanded to [B, H, Sq, Skv] (contiguous)."""
    B, _, _, S = bool_mask.shape
    z = torch.zeros((), dtype=_TORCH_DTYPES[dtype])
    ninf = torch.full((), float("-inf"), dtype=_TORCH_DTYPES[dtype])
    m = torch.where(bool_mask, z, ninf)
    return m.expand(B, heads, seq_q, S).contiguous()


@dataclass
class Workload:
    """One synthetic problem: everything both sides need, on the CPU."""

    name: str
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    cos: torch.Tensor  # fp32 [1|B, S, D]
    sin: torch.Tensor
    mask: torch.Tensor | None = None
    mask_kind: str = "none"  # none | bool | additive
    causal: bool = False
    scale: float | None = None
    do: torch.Tensor | None = None
    quant_int8: bool = False
    meta: dict = field(default_factory=dict)

    @property
    def shape(self):
        return tuple(self.q.shape)


def tiny_fp32(seed: int = 1000) -> Workload:
    """Tiny fused RoPE+SDPA forward in fp32: B=1, H=2, S=128, D=64, 1-axis RoPE, no mask."""
    B, H, S, D = 1, 2, 128, 64
    cos, sin = rope_tables(np.arange(S), (D,), 10000.0)
    return Workload(
        "tiny_fp32_b1h2s128d64",
        normal(seed, STREAM_Q, (B, H, S, D), "f32"),
        normal(seed, STREAM_K, (B, H, S, D), "f32"),
        normal(seed, STREAM_V, (B, H, S, D), "f32"),
        cos[None], sin[None],
        meta={"axes": (D,), "theta": 10000.0},
    )


def flux(batch: int = 1, heads: int = 24, n_text: int = 512, grid: int = 64, dtype: str = "bf16",
         seed: int = 2000, with_grad: bool = False, kv_heads: int | None = None,
         per_sample_tables: bool = False) -> Workload:
    """FLUX-style joint text+image attention: S = n_text + grid^2, D = 128, 3-axis RoPE (16,56,56).

    kv_heads: K/V head count for grouped-query attention (default: heads).
    per_sample_tables: one table per batch item ([B, S, D]); item b's image ids are shifted by
    a seeded offset (r0_b, c0_b) in [0, 64), as for crops taken at different positions.
    """
    S = n_text + grid * grid
    D = 128
    if per_sample_tables:
        offs = rng(seed, STREAM_TAB).integers(0, 64, size=(batch, 2))
        tabs = []
        for b in range(batch):
            ids = flux_ids(n_text, grid)
            ids[n_text:, 1] += offs[b, 0]
            ids[n_text:, 2] += offs[b, 1]
            tabs.append(rope_tables(ids, (16, 56, 56), 10000.0))
        cos = torch.stack([t[0] for t in tabs])
        sin = torch.stack([t[1] for t in tabs])
    else:
        c, s = rope_tables(flux_ids(n_text, grid), (16, 56, 56), 10000.0)
        cos, sin = c[None], s[None]
    hkv = heads if kv_heads is None else kv_heads
    shape = (batch, heads, S, D)
    kv_shape = (batch, hkv, S, D)
    w = Workload(
        f"flux_b{batch}h{heads}kv{hkv}s{S}d{D}_{dtype}",
        normal(seed, STREAM_Q, shape, dtype),
        normal(seed, STREAM_K, kv_shape, dtype),
        normal(seed, STREAM_V, kv_shape, dtype),
        cos, sin,
        do=normal(seed, STREAM_DO, shape, dtype) if with_grad else None,
        meta={"axes": (16, 56, 56), "theta": 10000.0, "n_text": n_text, "grid": grid, "kv_heads": hkv},
    )
    return w


def causal_1axis(batch: int = 4, heads: int = 16, seq: int = 2048, dim: int = 128, dtype: str = "bf16",
                 seed: int = 4000, with_grad: bool = True) -> Workload:
    """Causal training shape: 1-axis RoPE theta=10000 over positions 0..S-1."""
    cos, sin = rope_tables(np.arange(seq), (dim,), 10000.0)
    shape = (batch, heads, seq, dim)
    return Workload(
        f"causal_b{batch}h{heads}s{seq}d{dim}_{dtype}",
        normal(seed, STREAM_Q, shape, dtype),
        normal(seed, STREAM_K, shape, dtype),
        normal(seed, STREAM_V, shape, dtype),
        cos[None], sin[None], causal=True,
        do=normal(seed, STREAM_DO, shape, dtype) if with_grad else None,
        meta={"axes": (dim,), "theta": 10000.0},
    )


def random_small(B, H, S, D, dtype="f32", seed=7, mask_kind="none", mask_shape=None, causal=False,
                 per_sample_tables=False, with_grad=False, std=1.0, theta=10000.0, p_keep=0.7,
                 kv_heads=None) -> Workload:
    """Small general case for parity tests: 1-axis RoPE, optional random mask of any broadcast
    shape, optional grouped-query K/V (kv_heads < H)."""
    r = rng(seed, 99)
    if per_sample_tables:
        offs = r.integers(0, 1000, size=B)
        tabs = [rope_tables(np.arange(S) + o, (D,), theta) for o in offs]
        cos = torch.stack([t[0] for t in tabs]); sin = torch.stack([t[1] for t in tabs])
    else:
        c, s = rope_tables(np.arange(S), (D,), theta)
        cos, sin = c[None], s[None]
    mask = None
    if mask_kind != "none":
        ms = tuple(mask_shape) if mask_shape is not None else (B, H, S, S)
        keep = torch.from_numpy(r.random(ms) < p_keep)
        if mask_kind == "bool":
            mask = keep
        elif mask_kind == "additive":
            vals = torch.from_numpy(r.standard_normal(ms).astype(np.float32))
            add = torch.where(keep, vals, torch.full((), float("-inf")))
            mask = add.to(_TORCH_DTYPES[dtype])
        else:
            raise ValueError(mask_kind)
    shape = (B, H, S, D)
    kv_shape = (B, H if kv_heads is None else kv_heads, S, D)
    return Workload(
        f"small_b{B}h{H}s{S}d{D}_{dtype}_{mask_kind}{'_causal' if causal else ''}",
        normal(seed, STREAM_Q, shape, dtype, std),
        normal(seed, STREAM_K, kv_shape, dtype, std),
        normal(seed, STREAM_V, kv_shape, dtype),
        cos, sin, mask=mask, mask_kind=mask_kind, causal=causal,
        do=normal(seed, STREAM_DO, shape, dtype) if with_grad else None,
    )



@dataclass
class Chain:
    """A chain of attention layers with no projections between them: layer l attends with
    query x_l and its own keys/values (K_l, V_l), and its output is the next query,
    x_{l+1} = attention(R(x_l), R(K_l), V_l).  Everything both sides need, on the CPU."""

    x0: torch.Tensor
    ks: list
    vs: list
    cos: torch.Tensor
    sin: torch.Tensor

    @property
    def layers(self):
        return len(self.ks)


def zimage_chain(layers: int = 12, batch: int = 1, heads: int = 30, n_text: int = 32, grid: int = 64,
                 dtype: str = "bf16", seed: int = 6000) -> Chain:
    """The pages' chain benchmark at the Z-Image DiT attention shape (B, H, S, D) =
    (1, 30, 4128, 128), bf16: S = 32 caption tokens + a 64 x 64 image grid.  The pages give the
    shape but not the model's position ids or frequencies ("the caller adapts" the tables), so
    the FLUX-style 3-axis tables (16, 56, 56), theta = 10000, are used: text ids (0, 0, 0),
    image ids (0, r, c)."""
    S = n_text + grid * grid
    D = 128
    cos, sin = rope_tables(flux_ids(n_text, grid), (16, 56, 56), 10000.0)
    shape = (batch, heads, S, D)
    ks = [normal(seed, STREAM_LAYER + 2 * l, shape, dtype) for l in range(layers)]
    vs = [normal(seed, STREAM_LAYER + 2 * l + 1, shape, dtype) for l in range(layers)]
    return Chain(normal(seed, STREAM_Q, shape, dtype), ks, vs, cos[None], sin[None])
