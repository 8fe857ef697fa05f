"""GPU parity of the layer's input side (fla_linattn_fwd_proj: q, k, v projections with the
feature map fused into the projection kernel, then the forward pass) against the fp64
oracle's projection leg (oracle.fwd_proj: x W in fp64, then the recurrence).

Bar: max|o - o_ref| / max|o_ref| <= 1e-5 (fp32) and <= 1e-2 (bf16), outputs and final
states.  bf16 error budget: x and W are exact on both sides; the kernel rounds q, k, v to
bf16 once after fp32 accumulation (2^-9 relative), then the forward pass's own roundings.
"""
import numpy as np
import pytest

import oracle
from parity_util import TOL, rel_err, to_device, to_host
from workloads import PROJ, generate_proj, generate_proj_torch, to_numpy_input

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import chunkwise_causal_linear_amd as fla  # noqa: E402


def say(msg):
    print(msg, flush=True)


def spec(dtype, decay, B, T, hidden, H, dk, dv, *, phi=False, norm=False, init=0.0, seed=0):
    return dict(B=B, T=T, hidden=hidden, H=H, dk=dk, dv=dv, chunk=64, dtype=dtype, decay=decay,
                phi_elu1=phi, normalize=norm, init_sigma=init, seed=seed)


def run(sp, chunk=64):
    inp = generate_proj(sp)
    bf = sp["dtype"] == "bf16"
    dev = lambda a: to_device(a, bf16=bf)
    init = inp["init"]
    if init is not None and sp["normalize"]:
        init[..., sp["dv"]] = np.abs(init[..., sp["dv"]])
    out, fin = fla.fwd_proj(dev(inp["x"]), dev(inp["w_q"]), dev(inp["w_k"]), dev(inp["w_v"]),
                            sp["H"], to_device(inp["decay"]), decay_kind=sp["decay"],
                            init_state=to_device(init), chunk=chunk, phi_elu1=sp["phi_elu1"],
                            normalize=sp["normalize"])
    torch.cuda.synchronize()
    ro, rf = oracle.fwd_proj(inp["x"], inp["w_q"], inp["w_k"], inp["w_v"], sp["H"], inp["decay"],
                             sp["decay"], init, phi_elu1=sp["phi_elu1"], normalize=sp["normalize"])
    return to_host(out), to_host(fin), ro, rf


CASES = [(dt, dec, phi) for dt in ("bf16", "f32") for dec in ("none", "gamma", "gate", "token")
         for phi in (False, True)]


@pytest.mark.parametrize("dtype,decay,phi", CASES)
def test_projection_forward(dtype, decay, phi):
    i = CASES.index((dtype, decay, phi))
    sp = spec(dtype, decay, 2, 3 * 64 + 5, 128, 2, 64, 64, phi=phi, norm=phi, init=0.1,
              seed=1300 + i)
    say(f"[proj] {sp}")
    o, f, ro, rf = run(sp)
    eo, ef = rel_err(o, ro), rel_err(f, rf)
    say(f"[proj] {dtype} {decay} phi={phi}: out {eo:.2e} final {ef:.2e}")
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(f))
    assert eo <= TOL[dtype] and ef <= TOL[dtype], (eo, ef)


@pytest.mark.parametrize("B,T,hidden,H,dk,dv", [(1, 300, 96, 3, 16, 32), (3, 129, 64, 1, 128, 64),
                                                (1, 64, 256, 4, 64, 256), (2, 1, 32, 2, 32, 32)])
def test_projection_ragged_tiles(B, T, hidden, H, dk, dv):
    """Rows (B*T) and columns (H*d) that do not fill the 128 x 128 projection tiles, hidden
    sizes that are not multiples of the 64-element tile, a single token."""
    sp = spec("bf16", "gate", B, T, hidden, H, dk, dv, init=0.1, seed=1350 + hidden + T)
    say(f"[proj] ragged {sp}")
    o, f, ro, rf = run(sp)
    assert rel_err(o, ro) <= TOL["bf16"] and rel_err(f, rf) <= TOL["bf16"]


def test_projection_rejections():
    x = torch.zeros((1, 4, 48), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((48, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(fla.FlaError) as e:
        fla.fwd_proj(x, w, w, w, 1)                          # hidden not a multiple of 32
    assert e.value.status == fla.FLA_ERR_UNSUPPORTED
    x = torch.zeros((1, 4, 64), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((64, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(fla.FlaError) as e:
        fla.fwd_proj(x, w, w, w, 1, chunk=48)
    assert e.value.status == fla.FLA_ERR_UNSUPPORTED
    out, fin = fla.fwd_proj(x[:, :0].contiguous(), w, w, w, 1)   # T = 0: final = zeros
    torch.cuda.synchronize()
    assert torch.count_nonzero(fin).item() == 0


def test_projection_full_size_sampled_batch():
    """The projection workload (GLA layer shape: hidden 2048, 16 heads of 128) in the launch
    configuration the benchmark times; the oracle checks batch row 0 (all heads, all
    tokens)."""
    sp = PROJ["gla_proj_d128"]
    say(f"[proj-full] {sp}")
    inp = generate_proj_torch(sp, "cuda")
    out, fin = fla.fwd_proj(inp["x"], inp["w_q"], inp["w_k"], inp["w_v"], sp["H"], inp["decay"],
                            decay_kind=sp["decay"])
    torch.cuda.synchronize()
    h = lambda t: to_numpy_input(t)
    ro, rf = oracle.fwd_proj(h(inp["x"][:1]), h(inp["w_q"]), h(inp["w_k"]), h(inp["w_v"]), sp["H"],
                             h(inp["decay"][:1]), sp["decay"])
    eo, ef = rel_err(to_host(out[:1]), ro), rel_err(to_host(fin[:1]), rf)
    say(f"[proj-full] batch row 0: out {eo:.2e} final {ef:.2e}")
    assert eo <= TOL["bf16"] and ef <= TOL["bf16"]
