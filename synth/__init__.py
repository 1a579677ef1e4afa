"""Seeded synthetic inputs shaped like the activations the pages describe.

This module only draws data: it holds none of the quantization arithmetic and
imports neither the oracle nor the GPU library, so both sides can take their
inputs from it.

Outlier model (page "4.2 W8A8 量化与 SmoothQuant" section 1.1, page
"SmoothQuant大模型平滑量化技术" background section): about 1 % of the input
channels carry values roughly 100x larger than the rest, and a channel that is
an outlier is one for every token.  So a fixed set of channels is chosen once
per configuration and multiplied, on every token of the runtime batch and of
every calibration chunk, by a per-channel factor drawn once.

Everything is drawn with ``torch`` generators in fp32 and rounded to bf16
(round to nearest even) where a configuration says bf16.  A CPU generator and
a GPU generator with the same seed give different streams, so a test always
draws once and hands the same tensor to both sides.
"""
from __future__ import annotations

import hashlib
from dataclasses import dataclass, field

import torch


@dataclass(frozen=True)
class Config:
    name: str
    M: int                  # runtime tokens
    K: int                  # input channels
    N: int                  # output channels
    x_dtype: str            # "f32" or "bf16"
    body: str               # "normal" (N(0,1)) or "t4" (Student-t, 4 degrees of freedom)
    n_out: int              # number of outlier channels
    out_lo: float           # outlier factor ~ U[out_lo, out_hi] per channel (lo == hi: fixed)
    out_hi: float
    w_std: float            # W ~ N(0, w_std^2)
    calib_chunks: int       # calibration: chunks x chunk_tokens fresh draws (0 = X itself)
    chunk_tokens: int
    alphas: tuple = (0.5,)
    gran: str = "per_token"  # activation granularity
    w_prequant: bool = False  # weights arrive smoothed and quantized (decode shape)
    notes: str = ""
    seed_tag: int = 0        # salt of the workload's random streams

    @property
    def calib_tokens(self) -> int:
        return self.M if self.calib_chunks == 0 else self.calib_chunks * self.chunk_tokens

    @property
    def torch_dtype(self):
        return torch.float32 if self.x_dtype == "f32" else torch.bfloat16


TINY = "tiny_linear_64x256x256_f32"
ATTN_PROJ = "attn_proj_2048x4096x4096_bf16"
MLP_UP = "mlp_up_4096x4096x14336_bf16"
DECODE = "decode_16x8192x28672_bf16"
LARGE = "large_8192x12288x49152_bf16_t4"
ALL = (TINY, ATTN_PROJ, MLP_UP, DECODE, LARGE)

CONFIGS = {c.name: c for c in (
    Config(TINY, 64, 256, 256, "f32", "normal", 3, 100.0, 100.0, 0.02,
           0, 0, (0.5,), "per_tensor", seed_tag=1,
           notes="calibrates on X itself; per-tensor dynamic activation scale"),
    Config(ATTN_PROJ, 2048, 4096, 4096, "bf16", "normal", 41, 50.0, 150.0,
           0.02, 16, 512, (0.5,), seed_tag=2),
    Config(MLP_UP, 4096, 4096, 14336, "bf16", "normal", 41, 100.0, 100.0,
           0.02, 16, 512, (0.5,), seed_tag=3),
    Config(DECODE, 16, 8192, 28672, "bf16", "normal", 82, 100.0, 100.0,
           0.02, 16, 512, (0.5,), w_prequant=True, seed_tag=4),
    Config(LARGE, 8192, 12288, 49152, "bf16", "t4", 61, 200.0, 200.0,
           0.015, 512, 512, (0.4, 0.5, 0.6, 0.75), seed_tag=5,
           notes="calibration is 512 sequences x 512 tokens"),
)}


def seed_for(*parts) -> int:
    """Stable 63-bit seed from a tuple such as (42, config, tensor, chunk)."""
    h = hashlib.sha256("/".join(str(p) for p in parts).encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def _gen(device, *parts) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed_for(42, *parts))
    return g


def outlier_set(K: int, n_out: int, lo: float, hi: float, tag, device="cpu"):
    """(channel indices, per-channel factors) drawn once for a configuration."""
    g = _gen("cpu", tag, "outliers")
    idx = torch.randperm(K, generator=g)[:n_out].sort().values
    if hi > lo:
        fac = lo + (hi - lo) * torch.rand(n_out, generator=g)
    else:
        fac = torch.full((n_out,), float(lo))
    return idx.to(device), fac.to(device)


def body(rows: int, K: int, kind: str, gen: torch.Generator, device) -> torch.Tensor:
    """fp32 body of an activation matrix: N(0,1) or Student-t with 4 d.o.f.

    t4 = Z / sqrt(V / 4) with V ~ chi-square(4) = -2 (ln U1 + ln U2)."""
    z = torch.randn(rows, K, generator=gen, device=device, dtype=torch.float32)
    if kind == "normal":
        return z
    if kind != "t4":
        raise ValueError(kind)
    u = torch.rand(2, rows, K, generator=gen, device=device, dtype=torch.float32)
    u = 1.0 - u  # (0, 1]
    v = -2.0 * (torch.log(u[0]) + torch.log(u[1]))
    return z / torch.sqrt(v * 0.25)


def activations(rows: int, K: int, kind: str, out_idx, out_fac, dtype, gen, device) -> torch.Tensor:
    x = body(rows, K, kind, gen, device)
    if out_idx is not None and len(out_idx) > 0:
        x[:, out_idx.to(x.device)] *= out_fac.to(x.device)[None, :]
    return x.to(dtype)


def weights(K: int, N: int, std: float, dtype, gen, device) -> torch.Tensor:
    w = torch.randn(K, N, generator=gen, device=device, dtype=torch.float32)
    w.mul_(std)
    return w.to(dtype)


@dataclass
class Inputs:
    cfg: Config
    x: torch.Tensor                 # [M, K] runtime activations
    w: torch.Tensor                 # [K, N] weights
    calib: torch.Tensor             # [T, K] calibration tokens (contiguous chunks)
    out_idx: torch.Tensor = field(default=None)
    out_fac: torch.Tensor = field(default=None)


def make(cfg: Config | str, device="cpu", M=None, K=None, N=None, calib_chunks=None,
         chunk_tokens=None, variant=0, with_w=True) -> Inputs:
    """Draw one configuration's inputs (optionally at a reduced size with the
    same recipe).  ``variant`` selects an independent set of draws (the
    benchmark rotates several so timed reads come from HBM, not cache)."""
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    M = cfg.M if M is None else M
    K = cfg.K if K is None else K
    N = cfg.N if N is None else N
    chunks = cfg.calib_chunks if calib_chunks is None else calib_chunks
    ctok = cfg.chunk_tokens if chunk_tokens is None else chunk_tokens
    n_out = cfg.n_out if K == cfg.K else max(1, round(cfg.n_out * K / cfg.K))
    dt = cfg.torch_dtype
    out_idx, out_fac = outlier_set(K, n_out, cfg.out_lo, cfg.out_hi, (cfg.seed_tag, K), device)
    tag = (cfg.seed_tag, M, K, N, variant)
    x = activations(M, K, cfg.body, out_idx, out_fac, dt, _gen(device, *tag, "x"), device)
    w = weights(K, N, cfg.w_std, dt, _gen(device, *tag, "w"), device) if with_w else None
    if chunks == 0:
        calib = x
    else:
        calib = torch.empty(chunks * ctok, K, dtype=dt, device=device)
        for c in range(chunks):
            calib[c * ctok:(c + 1) * ctok] = activations(
                ctok, K, cfg.body, out_idx, out_fac, dt, _gen(device, *tag, "calib", c), device)
    return Inputs(cfg, x, w, calib, out_idx, out_fac)


def make_x(cfg: Config | str, device="cpu", variant=0, rows=None, with_outliers=True) -> torch.Tensor:
    """One more runtime batch x [rows (default M), K] of a configuration, with
    its outlier channels, from its own stream (``variant`` >= 1 gives batches
    independent of the one ``make`` draws); no weights, no calibration set."""
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    rows = cfg.M if rows is None else rows
    out_idx, out_fac = outlier_set(cfg.K, cfg.n_out, cfg.out_lo, cfg.out_hi, (cfg.seed_tag, cfg.K), device)
    if not with_outliers:
        out_idx = out_fac = None
    return activations(rows, cfg.K, cfg.body, out_idx, out_fac, cfg.torch_dtype,
                       _gen(device, cfg.seed_tag, rows, "extra-x", variant), device)


def to_numpy(t: torch.Tensor):
    """Host numpy view for the oracle: fp32 stays fp32, bf16 becomes uint16 bits."""
    t = t.detach().to("cpu").contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view("uint16")
    if t.dtype == torch.float32:
        return t.numpy()
    return t.numpy()
