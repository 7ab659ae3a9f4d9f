"""Seeded synthetic decode workloads for GDN heads (inputs only).

This module draws the inputs that both the GPU library and the CPU oracle
consume: initial fp32 states and per-token q, k, v, alpha, beta.  It holds
none of the quantized path's arithmetic (no windowed read, no record, no
fold, no quantization); its one piece of arithmetic is the dense prefill
that builds the initial states (below).  Every tensor it returns is an
input.  The shapes follow a Qwen3.5-9B-like hybrid
model: 24 GDN layers of 32 heads with a 128 x 128 state each ("Recurrent-state
quantization for linear attention: a first GPU kernel", Background).  The
recorded traces that page replays are not available, so these seeded
distributions stand in for them:

  q, k   ~ N(0, 1)^128, each L2-normalized per head and token
  v      ~ N(0, 1)^128
  beta   = sigmoid(z),         z ~ N(0, 1)
  alpha  = exp(-softplus(z)),  z ~ N(-3, 1)     (median 0.953); with
           per-channel decay (KDA) one independent draw per key channel

Initial states:
  "gauss":   N(0, 0.02^2) entries with 2 random rows and 2 random columns
             scaled x50 (outlier rows and columns, LeapQuant 1 Introduction).
  "prefill": the state a prompt leaves behind: 512 prefill tokens, drawn
             like the decode tokens but from a stream of their own, run
             through the dense fp32 recurrence from S = 0 (rows decayed by
             alpha, r = S^T k, u = beta (v - r), S += k u^T; with per-channel
             decay alpha scales each key row), then 1..4 distinct lines per
             head, each a row or a column with probability 1/2, scaled by
             U[20, 100].
  "hard":    "prefill" for heads < 24; heads 24..31 draw alpha from
             z ~ N(-6.9, 0.25) (alpha ~ 0.999), in the prefill as in decode,
             and, in place of the lines above, scale 2 rows and 2 columns
             x200 (a hard, slowly decaying late layer).

The prefill is the model's plain token step (the Gated DeltaNet recurrence of
"Recurrent-state quantization for linear attention: a first GPU kernel",
Background), written here with batched torch operations so that it can run on
either device; it is part of the input recipe, not of the quantized path, and
both sides of every comparison receive the tensor it produces.

Gated inputs (the raw projections that the gate arithmetic of the gated
entry points consumes) follow the Gated DeltaNet layer's parameterization:

  q, k, v ~ N(0, 1)^128 (q and k not normalized),  a, b ~ N(0, 1)
  per layer and model head: A_log = log(A), A ~ U[1, 16];
  dt_bias = softplus^-1(dt), log dt ~ U[log 1e-3, log 1e-1]

so that alpha = exp(-A softplus(a + dt_bias)) spreads over (0, 1) with most
heads decaying slowly.

Every draw comes from a torch generator seeded by a 64-bit mix of
(seed, stream, layer, token), so any (layer, token) slice can be regenerated
on demand, on the CPU or on the GPU.  The CPU and GPU generators produce
different numbers for the same seed; a comparison always hands both sides the
same tensor.
"""
import math
from dataclasses import dataclass, field

import torch

D = 128
MASK64 = (1 << 64) - 1


def _mix(*parts):
    """splitmix64 over the parts; a 63-bit torch seed."""
    x = 0x9E3779B97F4A7C15
    for p in parts:
        x = (x + (int(p) & MASK64) + 0x9E3779B97F4A7C15) & MASK64
        z = x
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK64
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK64
        x = z ^ (z >> 31)
    return x & ((1 << 63) - 1)


def _gen(device, *parts):
    g = torch.Generator(device=device)
    g.manual_seed(_mix(*parts))
    return g


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    layers: int
    heads: int
    tokens: int
    window: int = 16
    n_comp: int = 4
    in_dtype: str = "f32"          # "f32" or "bf16" for q, k, v
    init: str = "prefill"          # "gauss", "prefill" or "hard"
    seed: int = 0
    smoothing: bool = True
    sigma_floor: float = 1e-6
    decay: str = "scalar"          # "scalar" (GDN) or "channel" (KDA: alpha per key channel)
    notes: str = field(default="", compare=False)

    @property
    def heads_per_layer(self):
        return self.batch * self.heads

    def torch_dtype(self):
        return torch.bfloat16 if self.in_dtype == "bf16" else torch.float32


WORKLOADS = {
    "tiny": Workload("tiny", 1, 1, 4, 64, init="gauss", seed=0,
                     notes="1 request, 1 layer, 4 heads, 64 tokens (4 folds)"),
    "b32": Workload("b32", 32, 1, 32, 256, seed=1,
                    notes="single layer, batch 32, 256 tokens (16 folds)"),
    "b128": Workload("b128", 128, 24, 32, 512, seed=2,
                     notes="24 layers x 32 heads, batch 128, 512 tokens"),
    "b512": Workload("b512", 512, 24, 32, 1024, in_dtype="bf16", seed=3,
                     notes="24 layers x 32 heads, batch 512, 1024 tokens, bf16 q/k/v"),
    "tiny_kda": Workload("tiny_kda", 1, 1, 4, 64, init="gauss", seed=5, decay="channel",
                         notes="tiny with per-channel decay (KDA)"),
    "b512_kda": Workload("b512_kda", 512, 24, 32, 1024, in_dtype="bf16", seed=6, decay="channel",
                         notes="b512 shape with per-channel decay (KDA), bf16 q/k/v"),
    "long_kda": Workload("long_kda", 8, 3, 32, 4095, seed=7, decay="channel",
                         notes="batch 8, 3 layers x 32 heads, 4095 tokens, per-channel decay (KDA)"),
    "long": Workload("long", 8, 3, 32, 4095, init="hard", seed=4,
                     notes="batch 8, 3 layers x 32 heads, 4095 tokens (255 folds)"),
}

# stream ids
_S_INIT, _S_TOK, _S_HARD, _S_GTOK, _S_GPAR, _S_PRE = 1, 2, 3, 4, 5, 6

PREFILL_TOKENS = 512


def _normal(shape, g, device, mean=0.0, std=1.0):
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32) * std + mean


def _distinct(B, H, m, g, device):
    """m distinct indices in [0, 128) per head: [B, H, m] int64."""
    return torch.rand((B, H, D), generator=g, device=device).argsort(dim=-1)[..., :m].contiguous()


def initial_state(wl, layer, device="cpu", return_lines=False):
    """fp32 initial states of one layer: [batch, heads, 128, 128].

    With return_lines, also returns the planted outlier lines: for "gauss"
    (rows [B,H,2], cols [B,H,2]); otherwise (line [B,H,4], is_row [B,H,4],
    active [B,H,4]) for the regular heads' lines.
    """
    B, H = wl.batch, wl.heads
    g = _gen(device, wl.seed, _S_INIT, layer)
    if wl.init == "gauss":
        S = _normal((B, H, D, D), g, device, std=0.02)
        rows = _distinct(B, H, 2, g, device)
        cols = _distinct(B, H, 2, g, device)
        mult_r = torch.ones((B, H, D), device=device).scatter_(2, rows, 50.0)
        mult_c = torch.ones((B, H, D), device=device).scatter_(2, cols, 50.0)
        S = (S * mult_r.unsqueeze(-1) * mult_c.unsqueeze(-2)).contiguous()
        return (S, (rows, cols)) if return_lines else S
    S = prefill_state(wl, layer, device).reshape(B, H, D, D)
    # per-head outlier lines: count U{1..4}, axis with p = 1/2, scale U[20, 100]
    count = torch.randint(1, 5, (B, H), generator=g, device=device)
    axis = torch.randint(0, 2, (B, H, 4), generator=g, device=device)
    line = _distinct(B, H, 4, g, device)
    scale = torch.rand((B, H, 4), generator=g, device=device) * 80.0 + 20.0
    # distinct lines: a row and a column may share an index, two rows may not
    mult_r = torch.ones((B, H, D), device=device)
    mult_c = torch.ones((B, H, D), device=device)
    j = torch.arange(4, device=device).view(1, 1, 4)
    active = j < count.unsqueeze(-1)
    sr = torch.where(active & (axis == 0), scale, torch.ones_like(scale))
    sc = torch.where(active & (axis == 1), scale, torch.ones_like(scale))
    mult_r.scatter_(2, line, sr)
    mult_c.scatter_(2, line, sc)
    if wl.init == "hard":
        # heads 24..31: exactly 2 rows and 2 columns x200 replace the lines above
        gh = _gen(device, wl.seed, _S_HARD, layer)
        hl = _distinct(B, H, 4, gh, device)
        hr = torch.ones((B, H, D), device=device).scatter_(2, hl[..., :2], 200.0)
        hc = torch.ones((B, H, D), device=device).scatter_(2, hl[..., 2:], 200.0)
        mult_r[:, 24:] = hr[:, 24:]
        mult_c[:, 24:] = hc[:, 24:]
    S = (S * mult_r.unsqueeze(-1) * mult_c.unsqueeze(-2)).contiguous()
    return (S, (line, axis == 0, active)) if return_lines else S


def token_inputs(wl, layer, token, device="cpu", stream=_S_TOK):
    """Inputs of one decode token for one layer.

    Returns q, k, v as [batch, heads, 128] in the workload's input dtype and
    alpha, beta as fp32 [batch, heads]; with per-channel decay alpha is
    [batch, heads, 128], drawn per channel from the same distribution.
    `stream` separates the decode tokens from the prefill tokens.
    """
    B, H = wl.batch, wl.heads
    g = _gen(device, wl.seed, stream, layer, token)
    q = _normal((B, H, D), g, device)
    k = _normal((B, H, D), g, device)
    v = _normal((B, H, D), g, device)
    q = q / q.norm(dim=-1, keepdim=True)
    k = k / k.norm(dim=-1, keepdim=True)
    zb = _normal((B, H), g, device)
    za = _normal((B, H, D) if wl.decay == "channel" else (B, H), g, device, mean=-3.0)
    if wl.init == "hard":
        if wl.decay != "scalar":
            raise ValueError("the hard heads are defined for scalar decay")
        zh = _normal((B, H), g, device, mean=-6.9, std=0.25)
        za = za.clone()
        za[:, 24:] = zh[:, 24:]
    beta = torch.sigmoid(zb)
    alpha = torch.exp(-torch.nn.functional.softplus(za))
    dt = wl.torch_dtype()
    return (q.to(dt).contiguous(), k.to(dt).contiguous(), v.to(dt).contiguous(),
            alpha.contiguous(), beta.contiguous())


def prefill_state(wl, layer, device="cpu", tokens=PREFILL_TOKENS):
    """fp32 state [batch * heads, 128, 128] after `tokens` prefill tokens of
    the dense recurrence from zero, in token order.  The tokens come from
    token_inputs on the prefill stream (bf16 q/k/v widened exactly)."""
    N = wl.batch * wl.heads
    S = torch.zeros((N, D, D), dtype=torch.float32, device=device)
    for t in range(tokens):
        _, k, v, alpha, beta = token_inputs(wl, layer, t, device=device, stream=_S_PRE)
        k = k.reshape(N, D).to(torch.float32).contiguous()
        v = v.reshape(N, D).to(torch.float32)
        S.mul_(alpha.reshape((N, D, 1) if wl.decay == "channel" else (N, 1, 1)))
        r = torch.bmm(k.unsqueeze(1), S).squeeze(1)
        u = beta.reshape(N, 1) * (v - r)
        S.baddbmm_(k.unsqueeze(2), u.unsqueeze(1))
    return S


def gate_params(wl, layer, device="cpu"):
    """Gate parameters of one layer: A_log, dt_bias as fp32 [heads]."""
    g = _gen(device, wl.seed, _S_GPAR, layer)
    A = 1.0 + 15.0 * torch.rand(wl.heads, generator=g, device=device, dtype=torch.float64)
    u = torch.rand(wl.heads, generator=g, device=device, dtype=torch.float64)
    dt = torch.exp(math.log(1e-3) + u * (math.log(1e-1) - math.log(1e-3)))
    dt_bias = dt + torch.log(-torch.expm1(-dt))  # softplus(dt_bias) = dt
    return torch.log(A).float().contiguous(), dt_bias.float().contiguous()


def gated_token_inputs(wl, layer, token, device="cpu"):
    """Raw inputs of one decode token for the gated entry points: q, k, v as
    [batch, heads, 128] in the workload's input dtype (q, k not normalized)
    and the raw gate projections a, b as fp32 [batch, heads]."""
    B, H = wl.batch, wl.heads
    g = _gen(device, wl.seed, _S_GTOK, layer, token)
    q = _normal((B, H, D), g, device)
    k = _normal((B, H, D), g, device)
    v = _normal((B, H, D), g, device)
    a = _normal((B, H), g, device)
    b = _normal((B, H), g, device)
    dt = wl.torch_dtype()
    return q.to(dt).contiguous(), k.to(dt).contiguous(), v.to(dt).contiguous(), a.contiguous(), b.contiguous()


def widen(x):
    """Input tensor as fp32 (exact for bf16)."""
    return x.to(torch.float32)
