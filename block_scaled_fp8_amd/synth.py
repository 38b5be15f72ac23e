"""Seeded synthetic inputs for the routed MoE expert FFN.

This module only *draws* inputs.  It holds none of the arithmetic of the
method itself (no E4M3FN decoding, routing, sorting or expert FFN): the
CPU oracle under ``oracle/`` and the HIP library both consume the exact bytes
produced here.

Workload shapes follow the routed-expert geometry described on the pages:

* "Gated DeltaNet (+ FP8 MoE) -- AWS Neuron (NKI) kernels for Trainium2",
  section "FP8 MoE decode kernel (moe_fused_w8_35b)", Interface: hidden 2048,
  intermediate 512, 256 experts, top-8.
* "Add gfx950 Q256 fused MXFP4 prefill pipeline" (ROCm/aiter PR #5988),
  description: width 8192, intermediate 256, 512 routed experts, top-10 plus
  one shared expert.

Recipe (every draw is seeded; ``seed`` selects the stream):

* ``x``       bf16 [T, H]: N(0, 1) in fp32, rounded to nearest-even bf16.
* ``logits``  fp32 [T, E]: N(0, 1); the skewed prefill workload adds the
  per-expert bias ``2 * ln(1 / (e + 1))`` (computed in float64, rounded to fp32,
  added in fp32) so expert 0 is the most popular (Zipf-like load imbalance).
* weights: every expert matrix is drawn N(0, 0.02) (0.02 is the standard
  deviation) in fp32 and quantised with one fp32 scale per 128x128 block,
  ``scale = blockmax / 448`` (448 is the largest finite E4M3FN value), codes
  ``= E4M3FN_RNE(clamp(w / scale, -448, 448))``.  An all-zero block gets scale
  0 and all-zero codes.  The rounding onto the E4M3FN grid is torch's own
  ``float8_e4m3fn`` cast (round to nearest even); this is input preparation
  only and plays no part in what is checked.
* ``w13``  uint8 [E, 2I, H]: rows 0..I-1 are the gate projection, rows I..2I-1
  the up projection; ``w13_scale`` fp32 [E, 2I/128, H/128].  Non-gated
  (relu^2) experts draw the up projection alone, [E, I, H].
* ``w2``   uint8 [E, H, I]; ``w2_scale`` fp32 [E, H/128, I/128].
* MXFP4 weights (``weight_format="mxfp4"``, from the same draws): ``w13``
  uint8 [E, 2I, H/2] and ``w2`` [E, H, I/2], two E2M1 codes a byte (element
  2j in the low nibble of byte j), with uint8 E8M0 scales [E, 2I, H/32] and
  [E, H, I/32], one per 32 consecutive elements of a row (``quantize_mx``).
* shared expert (optional): the same format for one expert, drawn after the
  routed experts.
* ``wg``  bf16 [E, H] router gate weights (for the router projection):
  N(0, 0.02) in fp32 rounded to nearest-even bf16; with x ~ N(0, 1) the
  projected logits have standard deviation 0.02 * sqrt(H) (0.9 at H = 2048).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

BLOCK = 128
E4M3FN_MAX = 448.0


@dataclass(frozen=True)
class MoeConfig:
    name: str
    T: int          # tokens
    H: int          # hidden width
    I: int          # expert intermediate width (moe_inter)
    E: int          # routed experts
    k: int          # experts per token
    shared: bool = False
    skew: bool = False
    desc: str = field(default="", compare=False)

    @property
    def routes(self) -> int:
        return self.T * self.k


CONFIGS = {
    c.name: c
    for c in (
        MoeConfig("tiny", T=4, H=256, I=128, E=8, k=2,
                  desc="tiny MoE FFN, top-2 of 8 experts"),
        MoeConfig("decode64", T=64, H=2048, I=512, E=256, k=8,
                  desc="decode batch of 64 tokens, top-8 of 256 experts"),
        MoeConfig("decode512", T=512, H=2048, I=512, E=256, k=8,
                  desc="high-batch decode, 512 tokens, top-8 of 256"),
        MoeConfig("prefill8k_skew", T=8192, H=2048, I=512, E=256, k=8, skew=True,
                  desc="prefill of 8192 tokens with Zipf-skewed routing"),
        MoeConfig("prefill16k_wide", T=16384, H=8192, I=256, E=512, k=10, shared=True,
                  desc="wide prefill, 16384 tokens, top-10 of 512 plus one shared expert"),
    )
}
CONFIG_ORDER = ["tiny", "decode64", "decode512", "prefill8k_skew", "prefill16k_wide"]


def _gen(seed: int, tag: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed((int(seed) * 1_000_003 + int(tag) * 7919) & 0x7FFF_FFFF_FFFF)
    return g


def quantize_blocks(w: torch.Tensor):
    """fp32 [..., R, C] -> (uint8 codes [..., R, C], fp32 scales [..., R/128, C/128])."""
    *lead, R, C = w.shape
    assert R % BLOCK == 0 and C % BLOCK == 0, (R, C)
    blk = w.reshape(*lead, R // BLOCK, BLOCK, C // BLOCK, BLOCK)
    amax = blk.abs().amax(dim=(-3, -1))
    scale = amax / E4M3FN_MAX
    safe = torch.where(scale > 0, scale, torch.ones_like(scale))
    q = (blk / safe[..., :, None, :, None]).clamp(-E4M3FN_MAX, E4M3FN_MAX)
    codes = q.to(torch.float8_e4m3fn).view(torch.uint8).reshape(*lead, R, C)
    return codes.contiguous(), scale.contiguous()


# E2M1 magnitudes by code (codes 0..7; bit 3 is the sign)
_E2M1_GRID = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)


def quantize_mx(w: torch.Tensor):
    """fp32 [..., R, C] -> MXFP4: (uint8 [..., R, C/2] with element 2j in the
    low nibble of byte j and 2j+1 in the high nibble, uint8 E8M0 scales
    [..., R, C/32]).  Per block of 32 consecutive elements of a row: shared
    exponent X = floor(log2(max|w|)) - 2 (2 = the largest E2M1 exponent), the
    scale byte X + 127 clamped to 0..254, then each w / 2^X rounded to the
    nearest E2M1 value (ties to the even code), saturating at +-6.  An all-zero
    block gets scale byte 0 and zero codes."""
    *lead, R, C = w.shape
    assert C % 32 == 0, C
    blk = w.reshape(*lead, R, C // 32, 32)
    amax = blk.abs().amax(dim=-1)
    X = torch.floor(torch.log2(torch.where(amax > 0, amax, torch.ones_like(amax)))) - 2
    sbyte = torch.where(amax > 0, (X + 127).clamp(0, 254), torch.zeros_like(X))
    X = sbyte - 127
    q = (blk / torch.exp2(X)[..., None]).clamp(-6.0, 6.0)
    a = q.abs()
    grid = torch.tensor(_E2M1_GRID, dtype=torch.float32, device=w.device)
    lo = (torch.searchsorted(grid, a.contiguous(), right=True) - 1).clamp(0, 7)
    hi = (lo + 1).clamp(max=7)
    d_lo, d_hi = a - grid[lo], grid[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = torch.where(pick_hi, hi, lo) | torch.where(torch.signbit(q), 8, 0)
    code = code.to(torch.uint8).reshape(*lead, R, C)
    packed = (code[..., 0::2] | (code[..., 1::2] << 4)).contiguous()
    return packed, sbyte.to(torch.uint8).contiguous()


def _draw_expert_weights(n: int, rows: int, cols: int, seed: int, tag: int, device,
                         chunk_elems: int = 1 << 28, weight_format: str = "e4m3_128"):
    """n matrices [rows, cols] ~ N(0, 0.02), quantised; drawn in chunks of experts."""
    mx = weight_format == "mxfp4"
    codes = torch.empty((n, rows, cols // 2 if mx else cols), dtype=torch.uint8, device=device)
    scales = torch.empty((n, rows, cols // 32) if mx else (n, rows // BLOCK, cols // BLOCK),
                         dtype=torch.uint8 if mx else torch.float32, device=device)
    per = max(1, chunk_elems // (rows * cols))
    for e0 in range(0, n, per):
        e1 = min(n, e0 + per)
        g = _gen(seed, tag * 65536 + e0, device)
        w = torch.randn((e1 - e0, rows, cols), generator=g, device=device,
                        dtype=torch.float32) * 0.02
        c, s = quantize_mx(w) if mx else quantize_blocks(w)
        codes[e0:e1] = c
        scales[e0:e1] = s
        del w, c, s
    return codes, scales


def skew_bias(E: int) -> torch.Tensor:
    """Per-expert logit bias 2*ln(1/(rank+1)) with rank(e) = e, as fp32."""
    return torch.tensor([2.0 * math.log(1.0 / (e + 1)) for e in range(E)],
                        dtype=torch.float64).to(torch.float32)


def make_activations(cfg: MoeConfig, seed: int, device="cpu"):
    g = _gen(seed, 1, device)
    x = torch.randn((cfg.T, cfg.H), generator=g, device=device,
                    dtype=torch.float32).to(torch.bfloat16)
    g = _gen(seed, 2, device)
    logits = torch.randn((cfg.T, cfg.E), generator=g, device=device, dtype=torch.float32)
    if cfg.skew:
        logits = logits + skew_bias(cfg.E).to(device)
    return x.contiguous(), logits.contiguous()


def make_weights(cfg: MoeConfig, seed: int, device="cpu", activation="swiglu",
                 weight_format="e4m3_128"):
    """Block-scaled expert weights: "e4m3_128" (E4M3FN codes, fp32 128x128
    block scales) or "mxfp4" (quantize_mx: E2M1 codes two a byte, E8M0 scales
    per 32 elements of a row), from the same N(0, 0.02) draws.  Activation
    "relu2" draws non-gated experts, whose first matrix is the up projection
    alone ([I, H])."""
    n13 = cfg.I if activation == "relu2" else 2 * cfg.I
    f = dict(weight_format=weight_format)
    w13, w13_scale = _draw_expert_weights(cfg.E, n13, cfg.H, seed, 3, device, **f)
    w2, w2_scale = _draw_expert_weights(cfg.E, cfg.H, cfg.I, seed, 4, device, **f)
    out = dict(w13=w13, w13_scale=w13_scale, w2=w2, w2_scale=w2_scale)
    if cfg.shared:
        s13, s13s = _draw_expert_weights(1, n13, cfg.H, seed, 5, device, **f)
        s2, s2s = _draw_expert_weights(1, cfg.H, cfg.I, seed, 6, device, **f)
        out["shared"] = dict(w13=s13[0], w13_scale=s13s[0], w2=s2[0], w2_scale=s2s[0])
    else:
        out["shared"] = None
    return out


def make_gate_weights(E: int, H: int, seed: int, device="cpu"):
    """Router gate weights [E, H] bf16 ~ N(0, 0.02)."""
    g = _gen(seed, 7, device)
    w = torch.randn((E, H), generator=g, device=device, dtype=torch.float32) * 0.02
    return w.to(torch.bfloat16).contiguous()


def make_case(cfg: MoeConfig | str, seed: int = 0, device="cpu", activation="swiglu",
              weight_format="e4m3_128"):
    """All inputs of one workload: x, logits and the block-scaled weights."""
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    x, logits = make_activations(cfg, seed, device)
    case = dict(cfg=cfg, x=x, logits=logits, weight_format=weight_format)
    case.update(make_weights(cfg, seed, device, activation, weight_format))
    return case


def random_ids(T: int, k: int, E: int, seed: int, device="cpu", distinct=True):
    """Caller-style expert ids [T, k] int32 (distinct per token unless asked)."""
    g = _gen(seed, 11, "cpu")
    if distinct:
        ids = torch.stack([torch.randperm(E, generator=g)[:k] for _ in range(T)]) if T else \
            torch.empty((0, k), dtype=torch.int64)
    else:
        ids = torch.randint(0, E, (T, k), generator=g)
    return ids.to(torch.int32).to(device)


def random_affinities(T: int, k: int, seed: int, device="cpu"):
    g = _gen(seed, 12, "cpu")
    a = torch.rand((T, k), generator=g, dtype=torch.float32) + 0.05
    return (a / a.sum(dim=1, keepdim=True)).to(device)
