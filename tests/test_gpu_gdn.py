"""GPU parity of the gated delta rule forward (fla_gdn_fwd through the C ABI) against the
fp64 token-by-token oracle.

Bar (per tensor, over all batches/heads/tokens/columns): max|o - o_ref| / max|o_ref|
<= 1e-5 for fp32 inputs and <= 1e-2 for bf16 inputs, for outputs and final states.
"""
import numpy as np
import pytest

import oracle
from parity_util import TOL, rel_err, to_device, to_host
from workloads import (GDN, Workload, f32_to_bf16_bits, generate_gdn, generate_gdn_torch,
                       to_numpy_input)

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import chunkwise_causal_linear_amd as fla  # noqa: E402


def say(msg):
    print(msg, flush=True)


def case(dtype, dk, dv, T, *, B=2, H=2, init=True, seed=0):
    w = Workload("gdn", B, H, T, dk, dv, 64, dtype, "token", False, False,
                 1.0 if dtype == "f32" else dk ** -0.5, 0.1 if init else 0.0, seed=seed)
    return w, generate_gdn(w)


def run_gpu(w, inp):
    bf = w.dtype == "bf16"
    out, fin = fla.gdn_fwd(to_device(inp["q"], bf16=bf), to_device(inp["k"], bf16=bf),
                           to_device(inp["v"], bf16=bf), to_device(inp["alpha"]),
                           to_device(inp["beta"]), init_state=to_device(inp["init"]))
    torch.cuda.synchronize()
    return to_host(out), to_host(fin)


def check(w, inp, tag):
    say(f"[gdn] {tag}: {w}")
    o, f = run_gpu(w, inp)
    ro, rf = oracle.gdn_fwd(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], inp["init"])
    eo, ef = rel_err(o, ro), rel_err(f, rf)
    say(f"[gdn] {tag}: out {eo:.2e} final {ef:.2e}")
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(f))
    assert eo <= TOL[w.dtype] and ef <= TOL[w.dtype], (tag, eo, ef)


SHAPES = [("bf16", 128, 128), ("bf16", 64, 64), ("bf16", 128, 256), ("bf16", 64, 192),
          ("f32", 64, 64), ("f32", 64, 128)]


@pytest.mark.parametrize("dtype,dk,dv", SHAPES)
@pytest.mark.parametrize("init", [False, True])
def test_gdn_shapes(dtype, dk, dv, init):
    i = SHAPES.index((dtype, dk, dv))
    w, inp = case(dtype, dk, dv, 2 * 64 + 33, init=init, seed=800 + 2 * i + init)
    check(w, inp, f"{dtype} dk={dk} dv={dv} init={init}")


@pytest.mark.parametrize("T", [1, 63, 64, 65, 300])
def test_gdn_lengths(T):
    w, inp = case("bf16", 128, 64, T, seed=820 + T)
    check(w, inp, f"T={T}")


def test_gdn_strong_writes_and_slow_decay():
    """beta near 1 and alpha near 1: the memory is overwritten hard and kept long, the
    regime where the pseudo-values U = U0 - W H cancel most."""
    w, inp = case("bf16", 128, 128, 400, seed=830)
    inp["beta"] = (0.9 + 0.1 * inp["beta"]).astype(np.float32)
    inp["alpha"] = (0.999 + 0.001 * inp["alpha"]).astype(np.float32)
    check(w, inp, "beta ~ 1, alpha ~ 1")


@pytest.mark.parametrize("memory", ["workload", "long"])
def test_gdn_long_sequence(memory):
    """65,536 tokens (four times the workload's length) on two heads: the workload's decays,
    and a long memory (alpha = 1 - 1e-4 (1 - u), beta ~ 0.5) where rounding errors of the
    carried state would have the whole sequence to add up."""
    w, inp = case("bf16", 128, 128, 1 << 16, B=1, H=2, init=False, seed=860 + len(memory))
    if memory == "long":
        inp["alpha"] = (1.0 - 1e-4 * (1.0 - inp["alpha"])).astype(np.float32)
        inp["beta"] = (0.5 * inp["beta"] + 0.25).astype(np.float32)
    check(w, inp, f"T=65536, {memory} memory")


def test_gdn_near_parallel_keys():
    """Keys of one chunk nearly parallel (k_t = u + 0.05 n_t) with beta = 1: every write
    almost cancels the previous one, the strictly lower A = beta_t g_t / g_j k^_t . k^_j is
    close to all ones, and U = T diag(beta)(V - diag(g) K^ H) comes from the largest
    cancellations the solve sees."""
    w, inp = case("bf16", 128, 128, 4 * 64 + 17, B=1, H=2, seed=870)
    rng = np.random.default_rng(871)
    u = rng.standard_normal((1, 2, 1, 128))
    inp["k"] = f32_to_bf16_bits((u + 0.05 * rng.standard_normal(inp["k"].shape)).astype(np.float32))
    inp["beta"] = np.ones_like(inp["beta"])
    check(w, inp, "near-parallel keys, beta = 1")


def test_gdn_exact_recall():
    """The pages' associative-memory property: one (key, value) pair written repeatedly with
    beta = alpha = 1 reads back as the value (not a multiple of it)."""
    rng = np.random.default_rng(840)
    B, H, T, d = 1, 1, 3, 64
    key = rng.standard_normal(d).astype(np.float32)
    val = rng.standard_normal(d).astype(np.float32)
    khat = (key / np.linalg.norm(key.astype(np.float64))).astype(np.float32)
    k = np.broadcast_to(key, (B, H, T, d)).copy()
    v = np.broadcast_to(val, (B, H, T, d)).copy()
    q = np.broadcast_to(khat, (B, H, T, d)).copy()
    one = np.ones((B, H, T), np.float32)
    out, _ = fla.gdn_fwd(*(to_device(x) for x in (q, k, v, one, one)))
    torch.cuda.synchronize()
    o = to_host(out)[0, 0]
    for t in range(T):
        assert rel_err(o[t], val) <= 1e-5, t


def test_gdn_empty_and_rejects():
    w, inp = case("f32", 64, 64, 0, seed=850)
    o, f = run_gpu(w, inp)
    assert o.shape == (2, 2, 0, 64)
    assert np.array_equal(f, inp["init"].astype(np.float64))
    q = torch.zeros((1, 1, 64, 128), device="cuda")
    al = torch.ones((1, 1, 64), device="cuda")
    with pytest.raises(fla.FlaError) as e:
        fla.gdn_fwd(q, q, q, al, al)                       # fp32 dk = 128: two stages exceed the LDS
    assert e.value.status == fla.FLA_ERR_UNSUPPORTED
    q32 = torch.zeros((1, 1, 64, 32), device="cuda", dtype=torch.bfloat16)
    with pytest.raises(fla.FlaError) as e:
        fla.gdn_fwd(q32, q32, q32, al, al)
    assert e.value.status == fla.FLA_ERR_UNSUPPORTED


def test_gdn_full_size_all_heads():
    """The full-size workload in the launch configuration bench.py times; the oracle checks
    every head, one batch row at a time."""
    w = GDN["gdn_d128"]
    say(f"[gdn-full] {w}")
    inp = generate_gdn_torch(w, "cuda")
    out, fin = fla.gdn_fwd(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"])
    torch.cuda.synchronize()
    d_o = m_o = d_f = m_f = 0.0
    for b in range(w.B):
        sl = (slice(b, b + 1),)
        ro, rf = oracle.gdn_fwd(*(to_numpy_input(inp[n][sl]) for n in ("q", "k", "v", "alpha", "beta")))
        o, f = to_host(out[sl]), to_host(fin[sl])
        d_o, m_o = max(d_o, float(np.max(np.abs(o - ro)))), max(m_o, float(np.max(np.abs(ro))))
        d_f, m_f = max(d_f, float(np.max(np.abs(f - rf)))), max(m_f, float(np.max(np.abs(rf))))
    eo, ef = d_o / m_o, d_f / m_f
    say(f"[gdn-full] all heads: out {eo:.2e} final {ef:.2e}")
    assert eo <= TOL["bf16"] and ef <= TOL["bf16"]
