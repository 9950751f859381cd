"""Seeded synthetic KV-cache tensors for the SplitZip codec tests and benchmark.

This module only draws input data.  It holds none of the codec's arithmetic:
no exponent split, no codebook, no escape logic.  Both the GPU path's tests and
the CPU oracle's tests take their inputs from here.

The SplitZip pages measure on KV activations of Qwen, Llama and Phi models and
on BF16 activations captured from real models (technical summary, Metodologia /
Informacion Clave and Contribuciones Clave 2; the authors' abstract).  Those tensors are not available, so seeded
synthetic tensors with the same layout and a similar exponent distribution
stand in for them:

* layout ``[layers, 2 (K/V), tokens, kv_heads, head_dim]``, row-major, head_dim
  fastest;
* values ``N(0, 1) * s`` where each (layer, K/V, head, dim) channel has its own
  scale ``s = exp(sigma * N(0, 1))`` (a log-normal), and a Bernoulli(p) subset
  of channels is multiplied by an outlier factor ``f``;
* rounded to BF16 (or FP8 E5M2) with round-to-nearest-even by a direct
  float32 cast.

Seeds: layer ``l`` of workload number ``w`` draws its data with seed
``1000 * w + l``; its calibration sample uses ``seed + 500000``.

Large tensors are drawn layer by layer with ``torch.Generator`` on the target
device (the same seed gives the same bytes on the same device type; CPU and GPU
draws differ, so a test always hands one draw to both sides).  Channel scales
are drawn with numpy on the host and are identical everywhere.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

BF16 = 1
E5M2 = 2


@dataclass
class Spec:
    """Recipe of one workload."""
    name: str
    number: int                  # seed namespace
    dtype: int                   # BF16 or E5M2
    layers: int
    tokens: int
    heads: int
    head_dim: int = 128
    sigma: float = 1.0           # log-normal sigma of the channel scales
    outlier_p: float = 0.02
    outlier_f: float = 20.0
    calib_tokens: int = 1024
    calib: str = "per_layer"     # per_layer | rerun | sigma1 | same_generator
    kind: str = "gaussian"       # gaussian | const_exponent | uniform_bits | special_mix
    per_layer_codebooks: bool = True
    note: str = ""

    @property
    def layer_elems(self) -> int:
        return 2 * self.tokens * self.heads * self.head_dim

    @property
    def n(self) -> int:
        return self.layers * self.layer_elems


SPECS = {
    # Smallest instance: one layer's K and V, [1, 2, 1024, 8, 128] = 4 MiB.
    # Calibrated on a full re-draw of the same distribution (new scales too).
    "kv_layer_bf16": Spec("kv_layer_bf16", 1, BF16, 1, 1024, 8, calib="rerun",
                          per_layer_codebooks=False),
    # Llama-3-8B-shaped prefill KV, [32, 2, 8192, 8, 128] = 1 GiB, per-layer
    # codebooks calibrated on 1024 fresh tokens that share the layer's scales.
    "llama3_8b_kv_bf16": Spec("llama3_8b_kv_bf16", 2, BF16, 32, 8192, 8),
    # Long context, heavier tail, [28, 2, 32768, 4, 128] = 1.75 GiB.
    # Scales log-normal with variance 2 (sigma = sqrt 2), 5% channels x100;
    # calibrated on a narrower sigma = 1 draw.
    "long_ctx_heavy_tail_bf16": Spec("long_ctx_heavy_tail_bf16", 3, BF16, 28, 32768, 4,
                                     sigma=math.sqrt(2.0), outlier_p=0.05, outlier_f=100.0,
                                     calib="sigma1"),
    # Edge cases, 134,217,728 BF16 values (256 MiB) each, one codebook:
    # [1, 2, 65536, 8, 128].
    "edge_const_exponent": Spec("edge_const_exponent", 41, BF16, 1, 65536, 8,
                                kind="const_exponent", calib="same_generator",
                                per_layer_codebooks=False),
    "edge_uniform_bits": Spec("edge_uniform_bits", 42, BF16, 1, 65536, 8,
                              kind="uniform_bits", calib="same_generator",
                              per_layer_codebooks=False),
    "edge_special_values": Spec("edge_special_values", 43, BF16, 1, 65536, 8,
                                kind="special_mix", calib="same_generator",
                                per_layer_codebooks=False),
    # FP8 E5M2, Llama-3-70B-shaped, one GPU's share: [80, 2, 16384, 8, 128].
    "llama3_70b_kv_e5m2": Spec("llama3_70b_kv_e5m2", 5, E5M2, 80, 16384, 8),
}


def _channel_scales(seed: int, heads: int, head_dim: int, sigma: float, p: float, f: float) -> np.ndarray:
    """Per (K/V, head, dim) scale: log-normal times an outlier factor."""
    rng = np.random.default_rng(seed)
    s = np.exp(sigma * rng.standard_normal((2, heads, head_dim)))
    outlier = rng.random((2, heads, head_dim)) < p
    s = np.where(outlier, s * f, s)
    return s.astype(np.float32)


def _round_bits(x: torch.Tensor, dtype: int) -> torch.Tensor:
    """float32 -> BF16 / E5M2 bit patterns by round-to-nearest-even."""
    if dtype == BF16:
        return x.to(torch.bfloat16).view(torch.int16)
    return x.to(torch.float8_e5m2).view(torch.uint8)


def _gaussian_layer(seed: int, scales: np.ndarray, tokens: int, heads: int, head_dim: int,
                    dtype: int, device) -> torch.Tensor:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    z = torch.randn((2, tokens, heads, head_dim), generator=g, device=device, dtype=torch.float32)
    s = torch.from_numpy(scales).to(device).reshape(2, 1, heads, head_dim)
    return _round_bits(z * s, dtype).reshape(-1)


def _uniform_u16(seed: int, n: int, device) -> torch.Tensor:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return torch.randint(-32768, 32768, (n,), generator=g, device=device, dtype=torch.int32).to(torch.int16)


def _to_i16(v: torch.Tensor) -> torch.Tensor:
    """int32 values in [0, 65536) -> the int16 tensor with the same bits."""
    v = v.to(torch.int32)
    return (v - 65536 * (v >= 32768).to(torch.int32)).to(torch.int16)


def _edge_layer(kind: str, seed: int, n: int, device) -> torch.Tensor:
    """Edge-case BF16 bit patterns (int16 view)."""
    if kind == "uniform_bits":
        return _uniform_u16(seed, n, device)
    if kind == "const_exponent":
        u = _uniform_u16(seed, n, device).to(torch.int32) & 0xFFFF
        # random sign and mantissa, exponent field fixed at 127
        v = (u & 0x807F) | (127 << 7)
        return _to_i16(v)
    if kind == "special_mix":
        g = torch.Generator(device=device)
        g.manual_seed(seed)
        cat = torch.rand((n,), generator=g, device=device)
        bits = torch.randint(0, 65536, (n,), generator=g, device=device, dtype=torch.int32)
        sign = (bits & 1) << 15
        payload = ((bits >> 1) % 127) + 1          # 1..127, nonzero 7-bit payload
        scales = _channel_scales(seed + 7, 8, 128, 1.0, 0.02, 20.0).reshape(-1)
        s = torch.from_numpy(scales).to(device)
        idx = torch.arange(n, device=device) % s.numel()
        z = torch.randn((n,), generator=g, device=device)
        normal = (z * s[idx]).to(torch.bfloat16).view(torch.int16).to(torch.int32) & 0xFFFF
        out = normal
        out = torch.where(cat < 0.2, sign, out)                                  # +-0
        out = torch.where((cat >= 0.2) & (cat < 0.4), sign | payload, out)       # subnormal
        out = torch.where((cat >= 0.4) & (cat < 0.5), sign | 0x7F80, out)        # +-Inf
        out = torch.where((cat >= 0.5) & (cat < 0.6), sign | 0x7F80 | payload, out)  # NaN
        return _to_i16(out)
    raise ValueError(kind)


@dataclass
class Workload:
    spec: Spec
    data: torch.Tensor                    # flat int16 (BF16 bits) or uint8 (E5M2 bits)
    calib: list = field(default_factory=list)  # one flat sample tensor per codebook
    segment_elems: int = 0

    @property
    def n(self) -> int:
        return self.data.numel()

    @property
    def n_codebooks(self) -> int:
        return len(self.calib)

    @property
    def raw_bytes(self) -> int:
        return self.n * (2 if self.spec.dtype == BF16 else 1)


def _layer(spec: Spec, l: int, device, data: bool = True, calib: bool = True):
    """Data and calibration sample of layer ``l`` of a workload."""
    T, H, D = spec.tokens, spec.heads, spec.head_dim
    seed = 1000 * spec.number + l
    cseed = seed + 500000
    x = c = None
    if spec.kind == "gaussian":
        sc = _channel_scales(seed, H, D, spec.sigma, spec.outlier_p, spec.outlier_f)
        if data:
            x = _gaussian_layer(seed, sc, T, H, D, spec.dtype, device)
        if calib:
            if spec.calib == "per_layer":
                csc = sc
            elif spec.calib == "rerun":
                csc = _channel_scales(cseed, H, D, spec.sigma, spec.outlier_p, spec.outlier_f)
            elif spec.calib == "sigma1":
                csc = _channel_scales(cseed, H, D, 1.0, spec.outlier_p, spec.outlier_f)
            else:
                raise ValueError(spec.calib)
            ct = spec.calib_tokens if spec.calib != "rerun" else T
            c = _gaussian_layer(cseed, csc, ct, H, D, spec.dtype, device)
    else:
        n_l = spec.layer_elems
        if data:
            x = _edge_layer(spec.kind, seed, n_l, device)
        if calib:
            c = _edge_layer(spec.kind, cseed, min(n_l, 1 << 20), device)
    return x, c


def resize(name: str, layers: int | None = None, tokens: int | None = None) -> Spec:
    """The recipe of workload ``name``, optionally with fewer layers/tokens."""
    spec = Spec(**{**SPECS[name].__dict__})
    if layers is not None:
        spec.layers = layers
    if tokens is not None:
        spec.tokens = tokens
        if spec.kind == "gaussian":
            spec.calib_tokens = min(spec.calib_tokens, max(tokens, 16))
    return spec


def make(name: str, device="cpu", layers: int | None = None, tokens: int | None = None) -> Workload:
    """Draw workload ``name``; ``layers``/``tokens`` shrink it for small tests
    (the recipe and seeds stay the same)."""
    spec = resize(name, layers, tokens)
    parts = []
    calib = []
    for l in range(spec.layers):
        need_calib = spec.per_layer_codebooks or l == 0
        x, c = _layer(spec, l, device, calib=need_calib)
        parts.append(x)
        if need_calib:
            calib.append(c)
    flat = parts[0] if len(parts) == 1 else torch.cat(parts)
    seg = spec.layer_elems if (spec.per_layer_codebooks and spec.layers > 1) else 0
    return Workload(spec=spec, data=flat, calib=calib, segment_elems=seg)


def layer(name: str, l: int, device="cpu"):
    """Layer ``l`` of workload ``name`` on its own: (data, calibration sample)."""
    return _layer(resize(name), l, device)


def random_bits(n: int, dtype: int, seed: int, device="cpu", kind: str = "gaussian",
                sigma: float = 1.0) -> torch.Tensor:
    """Flat test tensor of ``n`` values: a channel-scaled Gaussian (1024
    channels) or uniformly random bit patterns."""
    if kind == "uniform_bits":
        if dtype == BF16:
            return _uniform_u16(seed, n, device)
        g = torch.Generator(device=device)
        g.manual_seed(seed)
        return torch.randint(0, 256, (n,), generator=g, device=device, dtype=torch.int32).to(torch.uint8)
    sc = _channel_scales(seed + 13, 4, 128, sigma, 0.02, 20.0).reshape(-1)
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    z = torch.randn((n,), generator=g, device=device)
    s = torch.from_numpy(sc).to(device)
    idx = torch.arange(n, device=device) % s.numel()
    return _round_bits(z * s[idx], dtype)


def to_numpy_bits(t: torch.Tensor) -> np.ndarray:
    """Host numpy view of a bit-pattern tensor (uint16 for BF16, uint8 for E5M2)."""
    a = t.detach().cpu().numpy()
    return a.view(np.uint16) if a.dtype == np.int16 else a
