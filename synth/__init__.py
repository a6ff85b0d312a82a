"""Seeded synthetic inputs shared by the tests, the bench and the smoke check.

This module only draws numbers: it holds none of the method's arithmetic,
and neither the HIP library nor the oracle is imported here.  Every tensor is
a pure function of its seed (torch generators: CPU for small cases, the
device generator for large ones).  Floats are drawn in fp32, scaled and
rotated (RoPE) in fp32, then rounded to bf16 with round-to-nearest-even.

Workload shapes (the pages print no model dimensions; these follow the
Qwen3 family that the KVpop summary evaluates on, Sec. 4):
  tiny      B=1, Hq=2, Hkv=1, D=64,  S=256,   w=16,  s=4, budget=64
  qwen4b    B=1, Hq=32, Hkv=8, D=128, S=4096,  w=128, s=4, budget=1024, RoPE
  skewed    B=4, Hq=32, Hkv=8, D=128, S=16384, w=256, s=4, budget=1966,
            2% planted heavy-hitter keys per head
  qwen8b    B=1, Hq=32, Hkv=8, D=128, S=32768, w=256, s=4, budget=8192, RoPE,
            36 layers (seed per layer)
  decode    64 sequences, 36 layers, Hq=32, Hkv=8, D=128, prefix 32768
            compressed to budget 4096 (s=4, w=256), delay 16, 512 steps
"""
from dataclasses import dataclass, field

import torch

ROPE_THETA = 1.0e6


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    D: int
    S: int
    window: int
    n_sink: int
    budget: int
    rope: bool = False
    std: float = 1.0
    layers: int = 1
    extra: dict = field(default_factory=dict)


TINY = Workload("tiny", 1, 2, 1, 64, 256, 16, 4, 64, rope=False, std=1.0)
QWEN4B = Workload("qwen3-4b-layer", 1, 32, 8, 128, 4096, 128, 4, 1024, rope=True, std=0.5)
SKEWED = Workload("skewed-long", 4, 32, 8, 128, 16384, 256, 4, 1966, rope=False, std=1.0,
                  extra={"heavy_frac": 0.02, "heavy_norm": 4.0, "noise": 0.5, "q_bias": 0.3})
QWEN8B = Workload("qwen3-8b-prefill", 1, 32, 8, 128, 32768, 256, 4, 8192, rope=True, std=0.5,
                  layers=36)
DECODE = Workload("bounded-decode", 64, 32, 8, 128, 32768, 256, 4, 4096, rope=False, std=0.5,
                  layers=36, extra={"delay": 16, "steps": 512, "hidden": 64})

WORKLOADS = {w.name: w for w in (TINY, QWEN4B, SKEWED, QWEN8B, DECODE)}


def _gen(seed, device):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def normal(shape, seed, device="cpu", std=1.0):
    g = _gen(seed, device)
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x


def rope(x, theta=ROPE_THETA):
    """Rotary position embedding on [..., S, D] (rotate-half pairing i, i+D/2,
    frequency theta^(-2i/D), position = token index), computed in fp32."""
    S, D = x.shape[-2], x.shape[-1]
    half = D // 2
    inv = theta ** (-torch.arange(0, half, dtype=torch.float64, device=x.device) * 2.0 / D)
    ang = torch.arange(S, dtype=torch.float64, device=x.device)[:, None] * inv[None, :]
    cos = torch.cos(ang).to(torch.float32)
    sin = torch.sin(ang).to(torch.float32)
    x1, x2 = x[..., :half], x[..., half:]
    return torch.cat([x1 * cos - x2 * sin, x2 * cos + x1 * sin], dim=-1)


def bf16(x):
    return x.to(torch.bfloat16)


def attention_inputs(w: Workload, seed: int, device="cpu"):
    """Q [B,Hq,S,D], K, V [B,Hkv,S,D] as bf16 tensors on ``device``."""
    if w.extra.get("heavy_frac"):
        return skewed_inputs(w, seed, device)
    q = normal((w.B, w.Hq, w.S, w.D), seed * 3 + 0, device, w.std)
    k = normal((w.B, w.Hkv, w.S, w.D), seed * 3 + 1, device, w.std)
    v = normal((w.B, w.Hkv, w.S, w.D), seed * 3 + 2, device, w.std)
    if w.rope:
        q = rope(q)
        k = rope(k)
    return bf16(q), bf16(k), bf16(v)


def skewed_inputs(w: Workload, seed: int, device="cpu"):
    """Planted heavy hitters: per (b, KV head) a unit direction u; round(frac*S)
    positions drawn without replacement carry key = norm*u + noise; queries
    are N(0,1) plus q_bias*u of their KV head."""
    e = w.extra
    B, Hq, Hkv, S, D = w.B, w.Hq, w.Hkv, w.S, w.D
    G = Hq // Hkv
    g = _gen(seed * 7 + 5, device)
    u = torch.randn((B, Hkv, D), generator=g, device=device, dtype=torch.float32)
    u = u / u.norm(dim=-1, keepdim=True)
    n_heavy = int(round(e["heavy_frac"] * S))
    k = normal((B, Hkv, S, D), seed * 7 + 1, device, 1.0)
    noise = normal((B, Hkv, n_heavy, D), seed * 7 + 2, device, e["noise"])
    pos = torch.empty((B, Hkv, n_heavy), dtype=torch.long, device=device)
    for b in range(B):
        for h in range(Hkv):
            pos[b, h] = torch.randperm(S, generator=g, device=device)[:n_heavy]
    heavy = e["heavy_norm"] * u[:, :, None, :] + noise
    k.scatter_(2, pos[..., None].expand(B, Hkv, n_heavy, D), heavy)
    q = normal((B, Hq, S, D), seed * 7 + 3, device, 1.0)
    q = q + e["q_bias"] * u.repeat_interleave(G, dim=1)[:, :, None, :]
    v = normal((B, Hkv, S, D), seed * 7 + 4, device, 1.0)
    return bf16(q), bf16(k), bf16(v)


def scores(shape, seed, device="cpu", kind="normal"):
    """fp32 score arrays for retention tests.

    kind: 'normal'  N(0,1);
          'ties'    few distinct values (heavy ties);
          'special' normal with NaN, +-inf, -0.0 and +0.0 planted;
          'const'   all equal; 'ramp' score = position; 'nan' all NaN.
    """
    g = _gen(seed, device)
    S = shape[-1]
    if kind == "normal":
        return torch.randn(shape, generator=g, device=device)
    if kind == "ties":
        return torch.randint(0, 5, shape, generator=g, device=device).float() * 0.25
    if kind == "special":
        x = torch.randn(shape, generator=g, device=device)
        r = torch.rand(shape, generator=g, device=device)
        x = torch.where(r < 0.05, torch.full_like(x, float("nan")), x)
        x = torch.where((r >= 0.05) & (r < 0.08), torch.full_like(x, float("inf")), x)
        x = torch.where((r >= 0.08) & (r < 0.11), torch.full_like(x, float("-inf")), x)
        x = torch.where((r >= 0.11) & (r < 0.16), torch.full_like(x, -0.0), x)
        x = torch.where((r >= 0.16) & (r < 0.21), torch.zeros_like(x), x)
        return x
    if kind == "const":
        return torch.full(shape, 0.5, device=device)
    if kind == "ramp":
        return torch.arange(S, device=device, dtype=torch.float32).expand(shape).contiguous()
    if kind == "nan":
        return torch.full(shape, float("nan"), device=device)
    raise ValueError(kind)


def normalizers(B, Hq, S, seed, device="cpu"):
    """A seeded stand-in for per-query log-normalizers [B,Hq,S] (fp32):
    ln(d + 1) + 1.5 + N(0, 0.25^2), the size a causal row of small logits has.
    Lets the transposed pass be checked at full size on an input both sides
    are handed, without the dense pass."""
    d = torch.arange(S, dtype=torch.float32, device=device)
    base = torch.log1p(d) + 1.5
    return (base + normal((B, Hq, S), seed, device, std=0.25)).contiguous()


def mlp_weights(Hkv, D, hidden, seed, device="cpu"):
    """Random-init headwise scorer: W1 ~ N(0, 1/D), w2 ~ N(0, 1/hidden), zero biases."""
    w1 = normal((Hkv, hidden, D), seed * 5 + 1, device, D ** -0.5)
    w2 = normal((Hkv, hidden), seed * 5 + 2, device, hidden ** -0.5)
    b1 = torch.zeros((Hkv, hidden), device=device)
    b2 = torch.zeros((Hkv,), device=device)
    return w1, b1, w2, b2
