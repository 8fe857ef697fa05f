"""Seeded synthetic workloads for chunkwise causal linear attention.

This module only draws random inputs and describes workload shapes. It holds none of
the method's arithmetic, so both the fp64 oracle (under ``oracle/``) and the HIP path
(``chunkwise_causal_linear_amd``) can consume exactly the same tensors.

The five named workloads mirror the shapes the source pages time or describe:
  * plain causal linear attention with the elu+1 feature map and the z normaliser
    (textbook chapter 1.6, "linear attention" section and its parallel/recurrent code);
  * RetNet-style retention at hidden 1024 with 4 heads, batch 32, length 2048 (the
    fla-org getting-started guide's MultiScaleRetention example);
  * decayed and GLA-gated attention at batch 8, head dim 128, length 8192 / 16384 (the
    Triton fused-kernel blog post's H100 timing paragraph);
  * a million-token retention sequence (the FLA long-sequence blog post, ">1M tokens").

Every tensor is drawn from numpy's PCG64 with a fixed seed, one independent child
stream per (batch, head) pair (``SeedSequence.spawn``), so the result does not depend on
how many threads generate it. bf16 tensors are stored as raw ``uint16`` bit patterns,
rounded from fp32 to nearest-even.
"""
from __future__ import annotations

import concurrent.futures as _fut
import dataclasses
import math
import os
from typing import Optional

import numpy as np

DECAY_NONE, DECAY_GAMMA, DECAY_GATE, DECAY_TOKEN = "none", "gamma", "gate", "token"


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    T: int
    dk: int
    dv: int
    chunk: int
    dtype: str          # "f32" or "bf16" (q, k, v and out)
    decay: str          # DECAY_NONE | DECAY_GAMMA | DECAY_GATE | DECAY_TOKEN
    phi_elu1: bool      # feature map elu(x)+1 on q and k, else identity
    normalize: bool     # o = S phi(q) / (z^T phi(q))
    qk_scale: float     # q, k ~ N(0,1) * qk_scale
    init_sigma: float   # 0 -> no initial state, else fp32 N(0, sigma^2)
    gamma_exp: str = "" # how gamma_h is formed (documentation only)
    seed: int = 0

    @property
    def token_heads(self) -> int:
        return self.B * self.H * self.T

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


def _gammas_offset(H: int, step: float) -> np.ndarray:
    """gamma_h = 1 - 2^(-5 - h*step), computed in fp64, rounded once to fp32."""
    h = np.arange(H, dtype=np.float64)
    return (1.0 - np.exp2(-5.0 - h * step)).astype(np.float32)


WORKLOADS = {
    "plain_f32": Workload("plain_f32", 1, 1, 256, 64, 64, 64, "f32", DECAY_NONE, True, True,
                          1.0, 0.0, seed=1001),
    "retention_d256": Workload("retention_d256", 32, 4, 2048, 256, 256, 64, "bf16", DECAY_GAMMA,
                               False, False, 1.0 / math.sqrt(256), 0.0,
                               gamma_exp="1-2^(-5-h)", seed=1002),
    "decayed_d128": Workload("decayed_d128", 8, 16, 8192, 128, 128, 64, "bf16", DECAY_GAMMA,
                             False, False, 1.0 / math.sqrt(128), 0.0,
                             gamma_exp="1-2^(-5-h*8/H)", seed=1003),
    "gla_d128": Workload("gla_d128", 8, 16, 16384, 128, 128, 64, "bf16", DECAY_GATE,
                         False, False, 1.0 / math.sqrt(128), 0.0, seed=1004),
    "token_decay_d128": Workload("token_decay_d128", 8, 16, 16384, 128, 128, 64, "bf16",
                                 DECAY_TOKEN, False, False, 1.0 / math.sqrt(128), 0.0,
                                 seed=1006),
    "long_retention": Workload("long_retention", 1, 8, 1 << 20, 128, 128, 128, "bf16",
                               DECAY_GAMMA, False, False, 1.0 / math.sqrt(128), 0.1,
                               gamma_exp="1-2^(-5-h)", seed=1005),
}
# The headline throughput workload.
HEADLINE = "gla_d128"

# Packed variable-length sequences (token-major [total][H][d]): the GLA workload's head
# shape over n_seqs sequences whose lengths are log-uniform in [lo, hi] (seeded).
VARLEN = {
    "varlen_gla_d128": dict(H=16, dk=128, dv=128, chunk=64, dtype="bf16", decay=DECAY_GATE,
                            n_seqs=24, lo=64, hi=16384, seed=1007),
}


# Gated delta rule (NEXT-3): the headline's shape; alpha = sigmoid(x)^(1/16) per token and
# head (the GLA gate recipe, one column), beta = sigmoid(y); x, y ~ N(0, 1).
GDN = {
    "gdn_d128": Workload("gdn_d128", 8, 16, 16384, 128, 128, 64, "bf16", DECAY_TOKEN, False,
                         False, 1.0 / math.sqrt(128), 0.0, seed=1008),
}


def generate_gdn(w: Workload) -> dict:
    """Inputs of a gated-delta workload (numpy, library layouts): q, k, v as ``generate``
    (streams 1-3), alpha [B,H,T] (stream 4), beta [B,H,T] (stream 9), init (stream 5) or
    None (no value column for a normaliser)."""
    d = generate(w.with_(normalize=False))
    d["alpha"] = d.pop("decay")
    beta = np.empty((w.B, w.H, w.T), dtype=np.float32)

    def fill(g, b, h):
        y = g.standard_normal(w.T, dtype=np.float64)
        beta[b, h] = (1.0 / (1.0 + np.exp(-y))).astype(np.float32)

    _per_head(w, 9, fill)
    d["beta"] = beta
    return d


def generate_gdn_torch(w: Workload, device="cuda") -> dict:
    """Device-side counterpart of generate_gdn (torch's seeded generator)."""
    import torch

    d = generate_torch(w.with_(normalize=False), device)
    d["alpha"] = d.pop("decay")
    gen = torch.Generator(device=device)
    gen.manual_seed(w.seed + 2)
    y = torch.randn((w.B, w.H, w.T), generator=gen, device=device, dtype=torch.float64)
    d["beta"] = torch.sigmoid(y).to(torch.float32)
    return d


def varlen_lengths(n_seqs: int, lo: int, hi: int, seed: int) -> np.ndarray:
    """Sequence lengths, log-uniform in [lo, hi], int64."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 8])))
    x = np.exp(g.uniform(np.log(lo), np.log(hi), n_seqs))
    return np.rint(x).astype(np.int64)


def varlen_workload(name: str):
    """(Workload over the concatenated tokens with B = 1, lengths) for a VARLEN entry."""
    d = VARLEN[name]
    lengths = varlen_lengths(d["n_seqs"], d["lo"], d["hi"], d["seed"])
    w = Workload(name, 1, d["H"], int(lengths.sum()), d["dk"], d["dv"], d["chunk"], d["dtype"],
                 d["decay"], False, False, 1.0 / math.sqrt(d["dk"]), 0.0, seed=d["seed"])
    return w, lengths


def gamma_for(w: Workload) -> Optional[np.ndarray]:
    if w.decay != DECAY_GAMMA:
        return None
    if w.gamma_exp == "1-2^(-5-h*8/H)":
        return _gammas_offset(w.H, 8.0 / w.H)
    return _gammas_offset(w.H, 1.0)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even); returns the uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _per_head(w: Workload, stream: int, fill):
    """Run fill(rng, b, h) for every (b, h) with an independent child generator."""
    ss = np.random.SeedSequence([w.seed, stream])
    children = ss.spawn(w.B * w.H)
    jobs = [(b, h, np.random.Generator(np.random.PCG64(children[b * w.H + h])))
            for b in range(w.B) for h in range(w.H)]
    if len(jobs) == 1:
        b, h, g = jobs[0]
        fill(g, b, h)
        return
    with _fut.ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(lambda j: fill(j[2], j[0], j[1]), jobs))


def _normal_tensor(w: Workload, stream: int, d: int, scale: float, as_bf16: bool) -> np.ndarray:
    out = np.empty((w.B, w.H, w.T, d), dtype=np.uint16 if as_bf16 else np.float32)

    def fill(g, b, h):
        x = g.standard_normal((w.T, d), dtype=np.float32)
        if scale != 1.0:
            x *= np.float32(scale)
        out[b, h] = f32_to_bf16_bits(x) if as_bf16 else x

    _per_head(w, stream, fill)
    return out


def _gate_tensor(w: Workload, stream: int, per_key: bool = True) -> np.ndarray:
    """alpha = sigmoid(x)^(1/16), x ~ N(0,1); evaluated in fp64, rounded once to fp32.
    Shape [B,H,T,dk] (per-key gate) or [B,H,T] (per-token scalar decay)."""
    tail = (w.dk,) if per_key else ()
    out = np.empty((w.B, w.H, w.T) + tail, dtype=np.float32)

    def fill(g, b, h):
        x = g.standard_normal((w.T,) + tail, dtype=np.float64)
        out[b, h] = np.power(1.0 / (1.0 + np.exp(-x)), 1.0 / 16.0).astype(np.float32)

    _per_head(w, stream, fill)
    return out


def generate(w: Workload) -> dict:
    """Draw the inputs of workload ``w``.

    Returns numpy arrays in the library's layouts: q, k [B,H,T,dk]; v [B,H,T,dv]
    (uint16 bf16 bits or float32); 'decay' = gamma [H] fp32, gate [B,H,T,dk] fp32,
    per-token decay [B,H,T] fp32 or None; 'init' = fp32 [B,H,dk,dv+n] or None (n = 1 with the normaliser).
    Draw order: q, k, v, then the gate or the initial state.
    """
    bf = w.dtype == "bf16"
    q = _normal_tensor(w, 1, w.dk, w.qk_scale, bf)
    k = _normal_tensor(w, 2, w.dk, w.qk_scale, bf)
    v = _normal_tensor(w, 3, w.dv, 1.0, bf)
    if w.decay in (DECAY_GATE, DECAY_TOKEN):
        decay = _gate_tensor(w, 4, per_key=w.decay == DECAY_GATE)
    else:
        decay = gamma_for(w)
    init = None
    if w.init_sigma > 0:
        ncol = w.dv + (1 if w.normalize else 0)
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([w.seed, 5])))
        init = g.standard_normal((w.B, w.H, w.dk, ncol), dtype=np.float32)
        init *= np.float32(w.init_sigma)
    return {"q": q, "k": k, "v": v, "decay": decay, "init": init}


def generate_grads(w: Workload, with_dfinal: bool = True) -> dict:
    """Upstream gradients for the backward pass: dout ~ N(0,1) in the workload's dtype
    [B,H,T,dv] and, if asked, dfinal ~ N(0,1) fp32 [B,H,dk,dv].  Streams 6 and 7 of the
    workload's seed, so they are independent of the forward inputs."""
    dout = _normal_tensor(w, 6, w.dv, 1.0, w.dtype == "bf16")
    dfinal = None
    if with_dfinal:
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([w.seed, 7])))
        dfinal = g.standard_normal((w.B, w.H, w.dk, w.dv), dtype=np.float32)
    return {"dout": dout, "dfinal": dfinal}


def generate_grads_torch(w: Workload, device="cuda", with_dfinal: bool = True) -> dict:
    """Device-side counterpart of generate_grads (torch's seeded generator, seed + 1)."""
    import torch

    gen = torch.Generator(device=device)
    gen.manual_seed(w.seed + 1)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    dout = torch.randn((w.B, w.H, w.T, w.dv), generator=gen, device=device,
                       dtype=torch.float32).to(dt)
    dfinal = None
    if with_dfinal:
        dfinal = torch.randn((w.B, w.H, w.dk, w.dv), generator=gen, device=device,
                             dtype=torch.float32)
    return {"dout": dout, "dfinal": dfinal}


def small(name: str, **kw) -> Workload:
    """A named workload shrunk to oracle-friendly sizes (keeps dtype, decay, phi, norm)."""
    return WORKLOADS[name].with_(**kw)


def as_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact widening of stored inputs (bf16 bits or fp32) to fp64."""
    if dtype == "bf16":
        return bf16_bits_to_f32(x).astype(np.float64)
    return np.asarray(x, dtype=np.float64)


def generate_torch(w: Workload, device="cuda"):
    """Draw the inputs of workload ``w`` directly on a device with torch's seeded generator
    (for full-size runs, where numpy would take minutes).  Same layouts as ``generate``;
    bf16 tensors are torch.bfloat16 (round-to-nearest-even from fp32).  Draw order: q, k,
    v, then the gate's x or the initial state."""
    import torch

    gen = torch.Generator(device=device)
    gen.manual_seed(w.seed)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32

    def normal(shape, scale):
        x = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
        if scale != 1.0:
            x.mul_(scale)
        return x.to(dt)

    q = normal((w.B, w.H, w.T, w.dk), w.qk_scale)
    k = normal((w.B, w.H, w.T, w.dk), w.qk_scale)
    v = normal((w.B, w.H, w.T, w.dv), 1.0)
    decay = None
    if w.decay in (DECAY_GATE, DECAY_TOKEN):
        tail = (w.dk,) if w.decay == DECAY_GATE else ()
        decay = torch.empty((w.B, w.H, w.T) + tail, device=device, dtype=torch.float32)
        for b in range(w.B):  # fp64 per batch row keeps the temporary small
            x = torch.randn((w.H, w.T) + tail, generator=gen, device=device, dtype=torch.float64)
            decay[b] = torch.sigmoid(x).pow(1.0 / 16.0).to(torch.float32)
    elif w.decay == DECAY_GAMMA:
        decay = torch.from_numpy(gamma_for(w)).to(device)
    init = None
    if w.init_sigma > 0:
        ncol = w.dv + (1 if w.normalize else 0)
        init = torch.randn((w.B, w.H, w.dk, ncol), generator=gen, device=device,
                           dtype=torch.float32) * w.init_sigma
    return {"q": q, "k": k, "v": v, "decay": decay, "init": init}


def to_numpy_input(t):
    """A torch input tensor as the oracle consumes it: fp32 array, or bf16 bit patterns."""
    import torch

    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def strong_gates(kind: str, B: int, H: int, T: int, dk: int, seed: int) -> dict:
    """Decay sets that leave the range of the fused kernel's factorisation (strong
    forgetting, as the textbook's gated delta rule and decay-masked attention allow):
      sigmoid   plain sigmoid(x) gates, x ~ N(0, 1) (no 1/16 power);
      uniform   decays uniform in [0.02, 0.5];
      isolated  sigmoid(x)^(1/16) with isolated entries of 1e-6 (6%) and 0 (1%).
    Shape [B, H, T, dk] for kind "gate", [B, H, T] for "token" (also the gated delta
    rule's alpha); fp32, drawn with numpy PCG64 from seed."""
    rng = np.random.default_rng(seed)
    shape = (B, H, T, dk) if kind == "gate" else (B, H, T)
    x = rng.standard_normal(shape)
    plain = 1.0 / (1.0 + np.exp(-x))
    uniform = rng.uniform(0.02, 0.5, shape)
    iso = plain ** (1.0 / 16.0)
    pick = rng.random(shape)
    iso = np.where(pick < 0.06, 1e-6, iso)
    iso = np.where(pick > 0.99, 0.0, iso)
    return {"sigmoid": plain.astype(np.float32), "uniform": uniform.astype(np.float32),
            "isolated": iso.astype(np.float32)}


# The layer's input side (NEXT-4): activations x [B, T, hidden] and projection weights
# W_q, W_k [hidden, H*dk], W_v [hidden, H*dv] (the GLA layer's shape: hidden 2048 = 16
# heads of 128), scaled so that q, k ~ N(0, 1/dk) and v ~ N(0, 1) like the other
# workloads; the gate token-major [B, T, H, dk], sigmoid(x)^(1/16).
PROJ = {
    "gla_proj_d128": dict(B=8, T=4096, hidden=2048, H=16, dk=128, dv=128, chunk=64,
                          dtype="bf16", decay=DECAY_GATE, phi_elu1=False, normalize=False,
                          seed=1010),
}


def generate_proj(spec: dict) -> dict:
    """numpy inputs of a projection workload: x [B,T,hidden], w_q, w_k [hidden,H*dk], w_v
    [hidden,H*dv] (bf16 bits or fp32), decay (gamma [H] / token-major gate or per-token
    decay, fp32) and init (fp32 [B,H,dk,dv(+1)] or None if spec has no init_sigma)."""
    B, T, D, H, dk, dv = (spec[k] for k in ("B", "T", "hidden", "H", "dk", "dv"))
    bf = spec["dtype"] == "bf16"
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([spec["seed"], 11])))

    def cast(a):
        a = a.astype(np.float32)
        return f32_to_bf16_bits(a) if bf else a

    out = {"x": cast(g.standard_normal((B, T, D))),
           "w_q": cast(g.standard_normal((D, H * dk)) / math.sqrt(D * dk)),
           "w_k": cast(g.standard_normal((D, H * dk)) / math.sqrt(D * dk)),
           "w_v": cast(g.standard_normal((D, H * dv)) / math.sqrt(D))}
    kind = spec["decay"]
    if kind == DECAY_GATE:
        out["decay"] = np.power(1.0 / (1.0 + np.exp(-g.standard_normal((B, T, H, dk)))),
                                1.0 / 16.0).astype(np.float32)
    elif kind == DECAY_TOKEN:
        out["decay"] = np.power(1.0 / (1.0 + np.exp(-g.standard_normal((B, T, H)))),
                                1.0 / 16.0).astype(np.float32)
    elif kind == DECAY_GAMMA:
        out["decay"] = _gammas_offset(H, 1.0)
    else:
        out["decay"] = None
    init = None
    if spec.get("init_sigma", 0.0) > 0:
        ncol = dv + (1 if spec.get("normalize") else 0)
        init = (g.standard_normal((B, H, dk, ncol)) * spec["init_sigma"]).astype(np.float32)
    out["init"] = init
    return out


def generate_proj_torch(spec: dict, device="cuda") -> dict:
    """Device-side counterpart of generate_proj (torch's seeded generator)."""
    import torch

    B, T, D, H, dk, dv = (spec[k] for k in ("B", "T", "hidden", "H", "dk", "dv"))
    gen = torch.Generator(device=device)
    gen.manual_seed(spec["seed"])
    dt = torch.bfloat16 if spec["dtype"] == "bf16" else torch.float32

    def normal(shape, scale):
        return (torch.randn(shape, generator=gen, device=device, dtype=torch.float32) * scale).to(dt)

    out = {"x": normal((B, T, D), 1.0), "w_q": normal((D, H * dk), (D * dk) ** -0.5),
           "w_k": normal((D, H * dk), (D * dk) ** -0.5), "w_v": normal((D, H * dv), D ** -0.5)}
    kind = spec["decay"]
    tail = {DECAY_GATE: (dk,), DECAY_TOKEN: ()}.get(kind)
    out["decay"] = None
    if tail is not None:
        x = torch.randn((B, T, H) + tail, generator=gen, device=device, dtype=torch.float64)
        out["decay"] = torch.sigmoid(x).pow(1.0 / 16.0).to(torch.float32)
    elif kind == DECAY_GAMMA:
        out["decay"] = torch.from_numpy(_gammas_offset(H, 1.0)).to(device)
    out["init"] = None
    return out
