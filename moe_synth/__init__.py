"""Seeded synthetic inputs for one GPU's share of a Mixture-of-Experts layer.

This module is the only code shared by the HIP path's callers (tests, bench)
and the CPU oracle. It draws random numbers and packs them into the storage
formats the layer consumes; it holds none of the layer's arithmetic (no
routing, no dispatch, no GEMM, no activation, no combine).

Workloads (shapes follow the problem statement of the MoE forward pass in
"Fine-grained Computation-Communication Overlap via Tile-level Signaling and
Scheduling for MoE", Section 2.1, and the MegaMoE description in "X-Stage: An
Overlooked Pipeline Stage ...", Section 2.2):

  tiny                 T=64,    d=128,  f=256,   E=4,   k=2, experts [0,4)
  deepseek_share_bf16  T=4096,  d=7168, f=2048,  E=256, k=8, experts [0,32)
  dit_skewed           T=32768, d=2048, f=1024,  E=64,  k=4, Zipf(1.2) prior
  mixtral              T=16384, d=4096, f=14336, E=8,   k=2
  deepseek_share_fp8   as deepseek_share_bf16, e4m3 + 128x128 fp32 block
                       scales, 8 destination segments (token t -> t mod 8)
  deepseek_share_w4a8  as deepseek_share_fp8, but W1 and W2 in MXFP4 (E2M1
                       elements, one E8M0 scale per 32 along K): the low-bit
                       weight variant the X-Stage evaluation runs beside W8A8

Draw order (one torch.Generator per call, seeded): X, then logits, then W1
expert by expert, then W2 expert by expert. All draws are fp32 standard
normals; weights are scaled by 0.02 (standard deviation). Only the local
experts' weights are drawn. The CUDA generator and the CPU generator give
different (each deterministic) streams: a caller generates once and hands the
same bits to both sides.

Storage formats produced here:
  bf16   : torch.bfloat16 tensors (torch's fp32 -> bf16 cast, round to nearest even)
  e4m3   : torch.uint8 bit patterns of OCP E4M3FN values plus fp32 block scales
           scale = amax(block) / 448 (1 if the block is all zero); code =
           torch's fp32 -> float8_e4m3fn cast of clamp(x / scale, -448, 448).
  mxfp4  : weights only. Per row, per 32 consecutive elements along K, the
           OCP MX conversion: shared exponent = floor(log2(amax)) - 2 (2 is
           the largest E2M1 exponent), stored as the E8M0 byte exponent + 127
           (127 for an all-zero block); elements = E2M1 of x / 2^exponent,
           round to nearest even, saturating at +-6. Two codes per byte, the
           even element in the low nibble: W1 [E_l, 2f, d/2] and W2
           [E_l, d, f/2] uint8, scales [E_l, 2f, d/32] and [E_l, d, f/32]
           uint8.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import torch

__all__ = ["MoEConfig", "CONFIGS", "generate", "make_config"]


@dataclasses.dataclass(frozen=True)
class MoEConfig:
    name: str
    T: int
    d: int
    f: int
    E_global: int
    k: int
    e_begin: int
    e_end: int
    dtype: str = "bf16"            # "bf16" or "fp8_e4m3"
    num_segments: int = 1
    zipf_s: float = 0.0            # > 0: logits get a -s*ln(e+1) Zipf prior
    seed: int = 0
    quant_block: int = 128

    @property
    def E_local(self) -> int:
        return self.e_end - self.e_begin

    @property
    def cap(self) -> int:
        """Upper bound on local (token, expert) assignments."""
        return self.T * min(self.k, self.E_local)

    def replace(self, **kw) -> "MoEConfig":
        return dataclasses.replace(self, **kw)


CONFIGS: Dict[str, MoEConfig] = {
    "tiny": MoEConfig("tiny", T=64, d=128, f=256, E_global=4, k=2, e_begin=0, e_end=4, seed=1),
    "deepseek_share_bf16": MoEConfig("deepseek_share_bf16", T=4096, d=7168, f=2048, E_global=256, k=8,
                                     e_begin=0, e_end=32, seed=2),
    "dit_skewed": MoEConfig("dit_skewed", T=32768, d=2048, f=1024, E_global=64, k=4, e_begin=0, e_end=64,
                            zipf_s=1.2, seed=3),
    "mixtral": MoEConfig("mixtral", T=16384, d=4096, f=14336, E_global=8, k=2, e_begin=0, e_end=8, seed=4),
    "deepseek_share_fp8": MoEConfig("deepseek_share_fp8", T=4096, d=7168, f=2048, E_global=256, k=8,
                                    e_begin=0, e_end=32, dtype="fp8_e4m3", num_segments=8, seed=2),
    "deepseek_share_w4a8": MoEConfig("deepseek_share_w4a8", T=4096, d=7168, f=2048, E_global=256, k=8,
                                     e_begin=0, e_end=32, dtype="w4a8_mxfp4", num_segments=8, seed=2),
}


def make_config(name: str, **overrides) -> MoEConfig:
    return CONFIGS[name].replace(**overrides)


def _normal(g: torch.Generator, shape, device, std: float = 1.0) -> torch.Tensor:
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x


def _quant_e4m3_blocks(x: torch.Tensor, br: int, bc: int):
    """Pack a 2-D fp32 tensor into e4m3 codes with one fp32 scale per (br x bc) block."""
    R, C = x.shape
    assert R % br == 0 and C % bc == 0, (R, C, br, bc)
    xb = x.reshape(R // br, br, C // bc, bc)
    amax = xb.abs().amax(dim=(1, 3))
    scale = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
    q = (xb / scale[:, None, :, None]).clamp_(-448.0, 448.0).to(torch.float8_e4m3fn)
    return q.reshape(R, C).view(torch.uint8), scale.contiguous()


# E2M1 rounding boundaries between consecutive magnitudes 0, 0.5, 1, 1.5, 2,
# 3, 4, 6; at the three marked ties the even code is the upper neighbour.
_E2M1_BOUNDS = (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0)
_E2M1_TIE_UP = (0.75, 1.75, 3.5)


def _quant_mxfp4_rows(x: torch.Tensor):
    """Pack a 2-D fp32 tensor [R, K] into MXFP4: (packed codes [R, K/2],
    E8M0 scale bytes [R, K/32])."""
    R, K = x.shape
    assert K % 32 == 0, K
    xb = x.reshape(R, K // 32, 32)
    amax = xb.abs().amax(dim=2)
    e = torch.where(amax > 0, torch.floor(torch.log2(torch.where(amax > 0, amax, torch.ones_like(amax)))) - 2,
                    torch.zeros_like(amax))
    e = e.clamp_(-127, 127)
    y = (xb / torch.exp2(e)[:, :, None]).abs()
    bounds = torch.tensor(_E2M1_BOUNDS, dtype=y.dtype, device=y.device)
    code = torch.bucketize(y, bounds, right=False)
    for t in _E2M1_TIE_UP:
        code += (y == t).to(code.dtype)
    code = code | (torch.signbit(xb).to(code.dtype) << 3)
    code = code.reshape(R, K).to(torch.uint8)
    packed = code[:, 0::2] | (code[:, 1::2] << 4)
    return packed.contiguous(), (e + 127).to(torch.uint8).contiguous()


def generate(cfg: MoEConfig, device="cpu", seed: Optional[int] = None) -> Dict[str, torch.Tensor]:
    """Draw one workload's inputs on `device`.

    Returns a dict with
      logits [T, E_global] fp32
      X      [T, d]            bf16, or uint8 e4m3 codes (+ X_scale [T/qb, d/qb] fp32)
      W1     [E_l, 2f, d]      bf16, or uint8 e4m3 codes (+ W1_scale [E_l, 2f/qb, d/qb]),
                               or MXFP4: uint8 [E_l, 2f, d/2] (+ W1_scale uint8 [E_l, 2f, d/32])
      W2     [E_l, d, f]       bf16, or uint8 e4m3 codes (+ W2_scale [E_l, d/qb, f/qb]),
                               or MXFP4: uint8 [E_l, d, f/2] (+ W2_scale uint8 [E_l, d, f/32])
    """
    device = torch.device(device)
    g = torch.Generator(device=device)
    g.manual_seed(cfg.seed if seed is None else seed)
    T, d, f, E, El = cfg.T, cfg.d, cfg.f, cfg.E_global, cfg.E_local
    out: Dict[str, torch.Tensor] = {}

    x32 = _normal(g, (T, d), device)
    logits = _normal(g, (T, E), device)
    if cfg.zipf_s > 0:
        prior = -cfg.zipf_s * torch.log(torch.arange(1, E + 1, device=device, dtype=torch.float64))
        logits += prior.to(torch.float32)[None, :]
    out["logits"] = logits.contiguous()

    fp8 = cfg.dtype in ("fp8_e4m3", "w4a8_mxfp4")
    w4 = cfg.dtype == "w4a8_mxfp4"
    qb = cfg.quant_block
    if fp8:
        out["X"], out["X_scale"] = _quant_e4m3_blocks(x32, qb, qb)
    else:
        out["X"] = x32.to(torch.bfloat16)
    del x32

    for name, rows, cols in (("W1", 2 * f, d), ("W2", d, f)):
        if w4:
            codes = torch.empty((El, rows, cols // 2), dtype=torch.uint8, device=device)
            scales = torch.empty((El, rows, cols // 32), dtype=torch.uint8, device=device)
        elif fp8:
            codes = torch.empty((El, rows, cols), dtype=torch.uint8, device=device)
            scales = torch.empty((El, rows // qb, cols // qb), dtype=torch.float32, device=device)
        else:
            codes = torch.empty((El, rows, cols), dtype=torch.bfloat16, device=device)
        for e in range(El):
            w = _normal(g, (rows, cols), device, std=0.02)
            if w4:
                codes[e], scales[e] = _quant_mxfp4_rows(w)
            elif fp8:
                codes[e], scales[e] = _quant_e4m3_blocks(w, qb, qb)
            else:
                codes[e] = w.to(torch.bfloat16)
            del w
        out[name] = codes
        if fp8:
            out[name + "_scale"] = scales
    return out
