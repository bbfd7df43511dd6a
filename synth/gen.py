"""Seeded synthetic workloads for one Kimi-K3-style LatentMoE layer.

Shapes follow the pages' statement of the layer: latent tokens of width 3584,
896 routed experts, 16 active per token (page 1, "从Kimi K3到MiniMax-H3", §一;
page 3, "Kimi K3 Day-0 适配剖析", §一 spec table). The pages give no expert
intermediate size, no weight distribution and no routing skew, so those are
parameters of the recipe below.

Recipe (every tensor has its own seeded stream, so an expert's weights do not
depend on how many other experts are drawn):

* tokens x ~ N(0, 1), drawn in fp32 and rounded to bf16 (round-to-nearest-even);
* router W_r ~ N(0, 1/d) in fp32, optional per-expert bias b:
  - ``normal``: b_e = 1.5 * N(0, 1)  (skews load; one expert-parallel rank's share),
  - ``zipf``:   b_e = -1.1 * ln(rank_e), rank a seeded permutation of 1..E
                (Zipf(1.1) popularity as a log-rank bias on the logits);
* expert e: W_gate, W_up [I, d] ~ N(0, 1/d) and W_down [d, I] ~ N(0, 1/I), drawn in
  fp32 and stored as MXFP4 (OCP Microscaling v1.0): per 32-element block along the
  contraction dim one E8M0 scale 2^(floor(log2 amax) - 2) and 32 E2M1 codes
  rounded to nearest, ties to even, magnitudes above 6 saturating to 6.

Storage layout of one weight matrix [N, K] (K = contraction dim): codes
[N, K/2] uint8 with element 2i in bits 0-3 and element 2i+1 in bits 4-7 of
byte i; scales [N, K/32] uint8 (E8M0 exponent, bias 127). Experts are stacked
on a leading axis.

The quantiser here is part of the input recipe (the layer only ever decodes);
the oracle carries its own, independently written, quantiser and the tests
check the two agree byte for byte.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from typing import Dict, Optional

import torch

D_LATENT = 3584
N_EXPERTS = 896
TOP_K = 16
MX_BLOCK = 32


@dataclass(frozen=True)
class LayerConfig:
    name: str
    T: int
    I: int
    d: int = D_LATENT
    E: int = N_EXPERTS
    k: int = TOP_K
    expert_begin: int = 0
    num_local: int = -1  # experts computed, ids expert_begin..; -1 means all E
    bias: Optional[str] = None  # None | "normal" | "zipf"
    seed: int = 0
    note: str = ""

    def __post_init__(self):
        if self.num_local < 0:
            object.__setattr__(self, "num_local", self.E - self.expert_begin)
        if not (0 <= self.expert_begin and self.expert_begin + self.num_local <= self.E):
            raise ValueError("local expert range outside [0, E)")

    def with_(self, **kw) -> "LayerConfig":
        return replace(self, **kw)


# The five workloads of the benchmark suite. The last, the largest that fits
# one GPU, is the headline workload.
CONFIGS: Dict[str, LayerConfig] = {
    "tiny": LayerConfig(
        "tiny", T=8, I=128,
        note="full structure at tiny width: T=8, I=128"),
    "decode": LayerConfig(
        "decode", T=64, I=1024,
        note="decode batch: T=64, bandwidth-bound weight streaming"),
    "prefill": LayerConfig(
        "prefill", T=8192, I=1024,
        note="prefill chunk: T=8192, ~146 rows per expert"),
    "ep_share": LayerConfig(
        "ep_share", T=16384, I=1024, num_local=112, bias="normal",
        note="one expert-parallel rank: experts 0..111 computed, skewed routing"),
    "long_skewed_prefill": LayerConfig(
        "long_skewed_prefill", T=65536, I=2048, bias="zipf",
        note="long prefill, Zipf(1.1) expert popularity"),
}
CONFIG_ORDER = ["tiny", "decode", "prefill", "ep_share", "long_skewed_prefill"]


# Stream ids: one per tensor kind; experts add their global id.
_S_TOKENS, _S_ROUTER, _S_BIAS = 1, 2, 3
_S_GATE, _S_UP, _S_DOWN = 10, 11, 12
_S_LORA = 20  # + 0..5: gate_a, gate_b, up_a, up_b, down_a, down_b


def _gen(device, seed: int, stream: int, sub: int = 0) -> torch.Generator:
    s = ((seed * 1_000_003 + stream) * 1_000_003 + sub) % (2**63 - 1)
    g = torch.Generator(device=device)
    g.manual_seed(s)
    return g


def make_tokens(cfg: LayerConfig, device="cpu", T: Optional[int] = None) -> torch.Tensor:
    """x [T, d] bf16 ~ N(0, 1) (fp32 draw, RNE to bf16)."""
    T = cfg.T if T is None else T
    g = _gen(device, cfg.seed, _S_TOKENS)
    x = torch.randn(T, cfg.d, generator=g, device=device, dtype=torch.float32)
    return x.to(torch.bfloat16)


def make_router(cfg: LayerConfig, device="cpu"):
    """W_r [E, d] fp32 ~ N(0, 1/d) and the optional bias [E] fp32."""
    g = _gen(device, cfg.seed, _S_ROUTER)
    w_r = torch.randn(cfg.E, cfg.d, generator=g, device=device, dtype=torch.float32)
    w_r.mul_(1.0 / math.sqrt(cfg.d))
    bias = None
    if cfg.bias == "normal":
        gb = _gen(device, cfg.seed, _S_BIAS)
        bias = 1.5 * torch.randn(cfg.E, generator=gb, device=device, dtype=torch.float32)
    elif cfg.bias == "zipf":
        gb = _gen("cpu", cfg.seed, _S_BIAS)
        rank = torch.randperm(cfg.E, generator=gb).to(torch.float64) + 1.0
        bias = (-1.1 * torch.log(rank)).to(torch.float32).to(device)
    elif cfg.bias is not None:
        raise ValueError(f"unknown bias kind {cfg.bias!r}")
    return w_r, bias


# ---------------------------------------------------------------------------
# MXFP4 encoding (input recipe)
# ---------------------------------------------------------------------------

def _pow2_f32(exp: torch.Tensor) -> torch.Tensor:
    """2**exp as fp32, built from its bit pattern (exact, exp in [-127, 127])."""
    e = exp.to(torch.int32)
    normal = (e + 127).clamp(min=1) << 23
    sub = torch.full_like(e, 1 << 22)  # 2**-127 is the one subnormal needed
    bits = torch.where(e > -127, normal, sub)
    return bits.view(torch.float32)


def quantize_mxfp4(w: torch.Tensor):
    """Encode w [N, K] fp32 as MXFP4: (codes [N, K/2] u8, scales [N, K/32] u8).

    Scale exponent: floor(log2 amax) - 2 taken exactly from frexp (never from a
    rounded log2), biased by 127 and clamped to [0, 254]; an all-zero block gets
    scale code 0 and zero codes. Magnitudes are rounded to the E2M1 grid
    {0, .5, 1, 1.5, 2, 3, 4, 6} to nearest with ties to the even code, values at
    or above 6 saturating to 6. The sign bit is the sign bit of the input.
    """
    assert w.dtype == torch.float32 and w.dim() == 2
    N, K = w.shape
    assert K % MX_BLOCK == 0
    blk = w.reshape(N, K // MX_BLOCK, MX_BLOCK)
    amax = blk.abs().amax(dim=-1)
    _, ex = torch.frexp(amax)  # amax = m * 2**ex with m in [0.5, 1)
    s = (ex.to(torch.int32) - 1 - 2 + 127).clamp(0, 254)
    s = torch.where(amax == 0, torch.zeros_like(s), s)
    q = blk * _pow2_f32(127 - s).unsqueeze(-1)  # exact: multiply by 2**(127 - s)
    a = q.abs()
    # Decision boundaries of round-to-nearest-even on the E2M1 magnitude grid:
    # a tie goes up where the upper grid point has the even code (0.75, 1.75, 3.5).
    mag = ((a > 0.25).to(torch.uint8) + (a >= 0.75).to(torch.uint8)
           + (a > 1.25).to(torch.uint8) + (a >= 1.75).to(torch.uint8)
           + (a > 2.5).to(torch.uint8) + (a >= 3.5).to(torch.uint8)
           + (a > 5.0).to(torch.uint8))
    code = mag | (torch.signbit(q).to(torch.uint8) << 3)
    code = torch.where((amax == 0).unsqueeze(-1), torch.zeros_like(code), code)
    code = code.reshape(N, K)
    packed = code[:, 0::2] | (code[:, 1::2] << 4)
    return packed.contiguous(), s.to(torch.uint8).contiguous()


def make_expert_weights(cfg: LayerConfig, device="cpu", experts=None) -> Dict[str, torch.Tensor]:
    """MXFP4 weights of the listed global experts (default: the local range).

    Returns gate/up codes [n, I, d/2], scales [n, I, d/32] and down codes
    [n, d, I/2], scales [n, d, I/32], all uint8 on ``device``.
    """
    if experts is None:
        experts = range(cfg.expert_begin, cfg.expert_begin + cfg.num_local)
    experts = list(experts)
    n, I, d = len(experts), cfg.I, cfg.d
    out = {
        "gate_codes": torch.empty(n, I, d // 2, dtype=torch.uint8, device=device),
        "gate_scales": torch.empty(n, I, d // MX_BLOCK, dtype=torch.uint8, device=device),
        "up_codes": torch.empty(n, I, d // 2, dtype=torch.uint8, device=device),
        "up_scales": torch.empty(n, I, d // MX_BLOCK, dtype=torch.uint8, device=device),
        "down_codes": torch.empty(n, d, I // 2, dtype=torch.uint8, device=device),
        "down_scales": torch.empty(n, d, I // MX_BLOCK, dtype=torch.uint8, device=device),
    }
    sg, sd = 1.0 / math.sqrt(d), 1.0 / math.sqrt(I)
    for i, e in enumerate(experts):
        for name, stream, shape, std in (("gate", _S_GATE, (I, d), sg),
                                         ("up", _S_UP, (I, d), sg),
                                         ("down", _S_DOWN, (d, I), sd)):
            g = _gen(device, cfg.seed, stream, e)
            w = torch.randn(*shape, generator=g, device=device, dtype=torch.float32)
            w.mul_(std)
            c, s = quantize_mxfp4(w)
            out[name + "_codes"][i].copy_(c)
            out[name + "_scales"][i].copy_(s)
            del w, c, s
    return out


LORA_NAMES = ("gate_a", "gate_b", "up_a", "up_b", "down_a", "down_b")


def make_lora(cfg: LayerConfig, rank: int, device="cpu") -> Dict[str, torch.Tensor]:
    """bf16 LoRA adapters of the local experts' three projections, rank r:
    gate_a / up_a [n, r, d] ~ N(0, 1/d), gate_b / up_b [n, I, r] ~ N(0, 1/r),
    down_a [n, r, I] ~ N(0, 1/I), down_b [n, d, r] ~ N(0, 1/r) (fp32 draws,
    RNE to bf16). The low-rank increment of the frozen base is B A."""
    n, I, d = cfg.num_local, cfg.I, cfg.d
    shapes = {"gate_a": (n, rank, d), "gate_b": (n, I, rank), "up_a": (n, rank, d),
              "up_b": (n, I, rank), "down_a": (n, rank, I), "down_b": (n, d, rank)}
    fan = {"gate_a": d, "gate_b": rank, "up_a": d, "up_b": rank, "down_a": I, "down_b": rank}
    out = {}
    for i, name in enumerate(LORA_NAMES):
        g = _gen(device, cfg.seed, _S_LORA + i, rank)
        w = torch.randn(*shapes[name], generator=g, device=device, dtype=torch.float32)
        out[name] = (w / math.sqrt(fan[name])).to(torch.bfloat16)
    return out


@dataclass
class LayerInputs:
    cfg: LayerConfig
    x: torch.Tensor
    w_router: torch.Tensor
    bias: Optional[torch.Tensor]
    weights: Dict[str, torch.Tensor] = field(default_factory=dict)

    def to(self, device) -> "LayerInputs":
        return LayerInputs(
            self.cfg, self.x.to(device), self.w_router.to(device),
            None if self.bias is None else self.bias.to(device),
            {k: v.to(device) for k, v in self.weights.items()})


def make_inputs(cfg: LayerConfig, device="cpu") -> LayerInputs:
    """All inputs of one layer call for ``cfg`` on ``device``.

    Different devices draw different random streams: compare a GPU result only
    with an oracle fed the very same bytes (copy them to the host).
    """
    x = make_tokens(cfg, device)
    w_r, bias = make_router(cfg, device)
    weights = make_expert_weights(cfg, device)
    return LayerInputs(cfg, x, w_r, bias, weights)
