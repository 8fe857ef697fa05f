"""GPU parity at byte offsets beyond 2^32: two heads of 2^24 + 1000 tokens (dk = dv = 128,
bf16), so that the second head of every tensor starts 4 GiB in.

The values are zero up to the last 1037 tokens, so the state stays exactly zero until then
(a write k v^T with v = 0 adds nothing, for any decay): every earlier output row must be
exactly zero, and the tail (outputs and final state) equals the oracle run on the tail alone
from a zero state.  q, k and the decays are random over the whole length.  Covers the
streaming and the segment schedules, the per-key gate, the constant decay and the gated
delta rule.
"""
import numpy as np
import pytest

import oracle
from parity_util import TOL, rel_err, to_host
from workloads import gamma_for, small, to_numpy_input

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import chunkwise_causal_linear_amd as fla  # noqa: E402

H, D = 2, 128
T = (1 << 24) + 1000
T0 = (1 << 24) - 37  # first token with nonzero values


def say(msg):
    print(msg, flush=True)


def inputs(kind, seed):
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    q = torch.empty((1, H, T, D), device="cuda", dtype=torch.bfloat16)
    k = torch.empty_like(q)
    v = torch.zeros_like(q)
    for h in range(H):
        q[0, h] = (torch.randn((T, D), generator=gen, device="cuda") * D ** -0.5).to(torch.bfloat16)
        k[0, h] = (torch.randn((T, D), generator=gen, device="cuda") * D ** -0.5).to(torch.bfloat16)
        v[0, h, T0:] = torch.randn((T - T0, D), generator=gen, device="cuda").to(torch.bfloat16)
    if kind == "gate":
        dec = torch.empty((1, H, T, D), device="cuda", dtype=torch.float32)
        for h in range(H):
            x = torch.randn((T, D), generator=gen, device="cuda")
            dec[0, h] = torch.sigmoid(x).pow_(1.0 / 16.0)
    else:
        dec = torch.from_numpy(gamma_for(small("decayed_d128", H=H))).to("cuda")
    return q, k, v, dec


@pytest.mark.parametrize("kind,nseg", [("gate", 1), ("gate", None), ("gamma", None)])
def test_beyond_4gib_offsets(kind, nseg):
    say(f"[large] {kind} n_segments={nseg}: B1 H{H} T{T} d{D}")
    q, k, v, dec = inputs(kind, 4242 + (nseg or 0))
    out, fin = fla.fwd(q, k, v, dec, decay_kind=kind, n_segments=nseg)
    torch.cuda.synchronize()
    say(f"[large] {kind} n_segments={nseg}: gpu done")
    head_zero = bool((out[:, :, :T0] == 0).all().item())
    tail = slice(T0, T)
    part = lambda t: to_numpy_input(t[:, :, tail])
    dtail = to_numpy_input(dec) if kind == "gamma" else part(dec)
    ro, rf = oracle.fwd(part(q), part(k), part(v), dtail, kind, None)
    eo, ef = rel_err(to_host(out[:, :, tail]), ro), rel_err(to_host(fin), rf)
    say(f"[large] {kind} n_segments={nseg}: rows before the values zero: {head_zero}; "
        f"tail out {eo:.2e} final {ef:.2e}")
    del q, k, v, dec, out, fin
    torch.cuda.empty_cache()
    assert head_zero
    assert eo <= TOL["bf16"] and ef <= TOL["bf16"]


def test_gated_delta_rule_beyond_4gib_offsets():
    """The gated delta rule at the same length: with v = 0 and a zero state the delta
    correction and the write both vanish, so the state stays zero until the values start."""
    say(f"[large] gated delta rule: B1 H{H} T{T} d{D}")
    q, k, v, _ = inputs("gamma", 777)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(778)
    alpha = torch.sigmoid(torch.randn((1, H, T), generator=gen, device="cuda")).pow_(1.0 / 16.0)
    beta = torch.sigmoid(torch.randn((1, H, T), generator=gen, device="cuda"))
    out, fin = fla.gdn_fwd(q, k, v, alpha, beta)
    torch.cuda.synchronize()
    say("[large] gated delta rule: gpu done")
    head_zero = bool((out[:, :, :T0] == 0).all().item())
    tail = slice(T0, T)
    part = lambda t: to_numpy_input(t[:, :, tail])
    ro, rf = oracle.gdn_fwd(part(q), part(k), part(v), part(alpha), part(beta), None)
    eo, ef = rel_err(to_host(out[:, :, tail]), ro), rel_err(to_host(fin), rf)
    say(f"[large] gated delta rule: rows before the values zero: {head_zero}; "
        f"tail out {eo:.2e} final {ef:.2e}")
    del q, k, v, alpha, beta, out, fin
    torch.cuda.empty_cache()
    assert head_zero
    assert eo <= TOL["bf16"] and ef <= TOL["bf16"]
