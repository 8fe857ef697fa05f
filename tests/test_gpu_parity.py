"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Bar (per tensor, over all batches/heads/tokens/columns): max|o - o_ref| / max|o_ref|
<= 1e-5 for fp32 inputs and <= 1e-2 for bf16 inputs, for outputs and final states.
"""
import itertools
import os
import sys

import numpy as np
import pytest

import oracle
from parity_util import TOL, rel_err, to_device, to_host
from workloads import WORKLOADS, generate, generate_torch, to_numpy_input, Workload

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import chunkwise_causal_linear_amd as fla  # noqa: E402


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def small_case(dtype, decay, dk, dv, T, *, B=2, H=2, chunk=64, phi=False, norm=False,
               init=False, seed=0):
    w = Workload("case", B, H, T, dk, dv, chunk, dtype, decay, phi, norm,
                 1.0 if dtype == "f32" else dk ** -0.5, 0.1 if init else 0.0,
                 gamma_exp="1-2^(-5-h)", seed=seed)
    return w, generate(w)


def run_gpu(w, inp, *, n_segments=None, chunk=None, init=True):
    bf = w.dtype == "bf16"
    q = to_device(inp["q"], bf16=bf)
    k = to_device(inp["k"], bf16=bf)
    v = to_device(inp["v"], bf16=bf)
    dec = to_device(inp["decay"])
    ini = to_device(inp["init"]) if init else None
    out, fin = fla.fwd(q, k, v, dec, decay_kind=w.decay, init_state=ini,
                       chunk=chunk or w.chunk, phi_elu1=w.phi_elu1, normalize=w.normalize,
                       n_segments=n_segments)
    torch.cuda.synchronize()
    return to_host(out), to_host(fin)


def run_oracle(w, inp, init=True):
    return oracle.fwd(inp["q"], inp["k"], inp["v"], inp["decay"], w.decay,
                      inp["init"] if init else None, phi_elu1=w.phi_elu1,
                      normalize=w.normalize)


def check(w, inp, tag, **kw):
    say(f"[parity] {tag}: {w}")
    o, f = run_gpu(w, inp, **kw)
    ro, rf = run_oracle(w, inp)
    eo, ef = rel_err(o, ro), rel_err(f, rf)
    tol = TOL[w.dtype]
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(f)), tag
    assert eo <= tol, f"{tag}: out rel err {eo:.3e} > {tol}"
    assert ef <= tol, f"{tag}: final rel err {ef:.3e} > {tol}"
    return eo, ef


# ---------------------------------------------------------------------------------------
# flag combinations at one shape (several chunks and a ragged tail)
FLAG_COMBOS = list(itertools.product(["f32", "bf16"], ["none", "gamma", "gate", "token"],
                                     [False, True], [False, True]))


@pytest.mark.parametrize("dtype,decay,norm,init", FLAG_COMBOS)
def test_flag_combinations(dtype, decay, norm, init):
    w, inp = small_case(dtype, decay, 64, 64, 3 * 64 + 5, phi=norm or decay == "none",
                        norm=norm, init=init, seed=FLAG_COMBOS.index((dtype, decay, norm, init)))
    check(w, inp, f"flags {dtype} {decay} norm={norm} init={init}")


def test_identity_phi_normalised_positive_inputs():
    w, inp = small_case("f32", "gamma", 32, 32, 100, phi=False, norm=True, init=False, seed=5)
    inp["q"] = np.abs(inp["q"]) + np.float32(0.1)
    inp["k"] = np.abs(inp["k"]) + np.float32(0.1)
    check(w, inp, "identity phi + normaliser")


# ---------------------------------------------------------------------------------------
# shape sweep: dk, dv (incl. dk != dv), chunk, ragged lengths
DIMS = [16, 32, 64, 128, 256]
CHUNKS = [16, 32, 64, 128]


def _supported(dtype, dk, chunk, decay):
    """The library's LDS budget for one workgroup (160 KiB on gfx950): one stage of the
    row-major operand tiles Qt, Kt [C][dk+pad] and V [C][64+pad], the per-key chunk
    decay (gate) and the gamma power table."""
    es = 2 if dtype == "bf16" else 4
    pad = 16 // es
    stage = (2 * chunk * (dk + pad) + chunk * (64 + pad)) * es
    if decay == "gate":
        stage += dk * 4
    pw = ((chunk + 4) // 4) * 16 if decay == "gamma" else 0
    return stage + pw <= 163840


SWEEP = []
for i, (dtype, dk, dv, chunk) in enumerate(itertools.product(["bf16", "f32"], DIMS, DIMS, CHUNKS)):
    decay = ["none", "gamma", "gate"][i % 3]
    if not _supported(dtype, dk, chunk, decay):
        continue
    Ts = [1, chunk - 1, chunk, chunk + 1, 3 * chunk + 5]
    SWEEP.append((dtype, dk, dv, chunk, Ts[i % len(Ts)], decay, i % 4 == 1, i % 2 == 0))


def test_sweep_covers_every_supported_dim_and_chunk():
    for dtype in ("bf16", "f32"):
        assert {c[1] for c in SWEEP if c[0] == dtype} == set(DIMS)
        assert {c[2] for c in SWEEP if c[0] == dtype} == set(DIMS)
        assert {c[3] for c in SWEEP if c[0] == dtype} == set(CHUNKS)


@pytest.mark.parametrize("dtype,dk,dv,chunk,T,decay,norm,init", SWEEP)
def test_shape_sweep(dtype, dk, dv, chunk, T, decay, norm, init):
    w, inp = small_case(dtype, decay, dk, dv, T, B=1, H=2, chunk=chunk, phi=norm, norm=norm,
                        init=init, seed=SWEEP.index((dtype, dk, dv, chunk, T, decay, norm, init)))
    check(w, inp, f"sweep {dtype} dk={dk} dv={dv} C={chunk} T={T} {decay} norm={norm}")


# Large tiles take the two-barrier schedule (one Qt tile, double-buffered Kt/V), small ones
# the shared-score schedule: every decay kind and the normaliser on representatives of each,
# with a ragged sequence end and value widths of half a slice (some consumer waves own no
# valid column) and of two slices.
SCHEDULE_SHAPES = [("bf16", 128, 128), ("bf16", 256, 64), ("f32", 128, 64), ("bf16", 64, 128),
                   ("bf16", 128, 64), ("f32", 32, 64)]
SCHEDULE_CASES = [(dt, dk, c, dec, norm) for (dt, dk, c) in SCHEDULE_SHAPES
                  for dec in ("none", "gamma", "gate", "token") for norm in (False, True)]


@pytest.mark.parametrize("dtype,dk,chunk,decay,norm", SCHEDULE_CASES)
def test_schedules(dtype, dk, chunk, decay, norm):
    i = SCHEDULE_CASES.index((dtype, dk, chunk, decay, norm))
    w, inp = small_case(dtype, decay, dk, 32 if i % 2 == 0 else 128, 2 * chunk + 7, B=1, H=2,
                        chunk=chunk, phi=norm, norm=norm, init=True, seed=500 + i)
    check(w, inp, f"schedule {dtype} dk={dk} C={chunk} {decay} norm={norm}")


def test_unsupported_chunk_raises():
    q = torch.zeros((1, 1, 128, 128), dtype=torch.float32, device="cuda")
    v = torch.zeros((1, 1, 128, 64), dtype=torch.float32, device="cuda")
    for chunk in (48, 2048, 8):
        with pytest.raises(fla.FlaError) as e:
            fla.fwd(q, q, v, chunk=chunk)
        assert e.value.status == fla.FLA_ERR_UNSUPPORTED


def test_chunk_128_of_slow_tiles_runs_as_64():
    """Chunk 128 with the per-key gate or dk = 256, fp32 chunk 128 at dk >= 128, and the
    constant decay at dk = 128 in bf16, runs as 64-token sub-chunks: bitwise the chunk-64
    result, and against the oracle (the fp32 cases' 128-token tiles would not fit the LDS)."""
    for dtype, decay, dk in (("bf16", "gate", 128), ("f32", "none", 256), ("bf16", "gamma", 256),
                             ("f32", "gamma", 128), ("f32", "token", 128), ("bf16", "gamma", 128)):
        w, inp = small_case(dtype, decay, dk, 64, 3 * 128 + 9, B=1, H=2, chunk=128, init=True,
                            seed=dk + len(decay))
        check(w, inp, f"chunk 128 as 64: {dtype} {decay} dk={dk}")
        o, f = run_gpu(w, inp)
        o64, f64 = run_gpu(w, inp, chunk=64)
        assert np.array_equal(o, o64) and np.array_equal(f, f64)


# ---------------------------------------------------------------------------------------
# schedules: segment path against the oracle and against the streaming path
@pytest.mark.parametrize("decay", ["none", "gamma", "gate", "token"])
@pytest.mark.parametrize("nseg", [2, 3, 7])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_segment_schedule(decay, nseg, dtype):
    w, inp = small_case(dtype, decay, 64, 128, 16 * 32 + 9, B=1, H=2, chunk=32,
                        phi=True, norm=(decay in ("gate", "token")), init=True,
                        seed=100 + nseg)
    check(w, inp, f"segments={nseg} {dtype} {decay}", n_segments=nseg)
    o1, f1 = run_gpu(w, inp, n_segments=1)
    o2, f2 = run_gpu(w, inp, n_segments=nseg)
    assert rel_err(o2, o1) <= TOL[dtype] and rel_err(f2, f1) <= TOL[dtype]


def test_empty_sequence_copies_init():
    w, inp = small_case("bf16", "gamma", 64, 64, 0, init=True, seed=7)
    o, f = run_gpu(w, inp)
    assert o.shape == (2, 2, 0, 64)
    assert np.array_equal(f, inp["init"].astype(np.float64))
    o, f = run_gpu(w, inp, init=False)
    assert np.all(f == 0)


@pytest.mark.parametrize("decay", ["gate", "token"])
def test_empty_sequence_with_empty_per_token_decay(decay):
    w, inp = small_case("bf16", decay, 64, 64, 0, init=True, seed=17)
    o, f = run_gpu(w, inp)
    assert o.shape == (2, 2, 0, 64)
    assert np.array_equal(f, inp["init"].astype(np.float64))


def test_single_token():
    w, inp = small_case("f32", "gate", 32, 16, 1, phi=True, norm=True, init=True, seed=8)
    check(w, inp, "T=1")


def test_deterministic_repeat():
    w, inp = small_case("bf16", "gate", 128, 128, 700, chunk=64, init=True, seed=9)
    o1, f1 = run_gpu(w, inp)
    o2, f2 = run_gpu(w, inp)
    assert np.array_equal(o1, o2) and np.array_equal(f1, f2)


@pytest.mark.parametrize("nseg", [1, 4])
def test_in_place_resume(nseg):
    """init_state aliasing final_state, with the z column and two value slices."""
    w, inp = small_case("f32", "gamma", 32, 128, 300, B=1, H=2, chunk=32, phi=True, norm=True,
                        init=True, seed=10 + nseg)
    q, k, v = (to_device(inp[n]) for n in ("q", "k", "v"))
    dec = to_device(inp["decay"])
    state = to_device(inp["init"]).clone()
    out, fin = fla.fwd(q, k, v, dec, init_state=state, final_state=state, chunk=32,
                       phi_elu1=True, normalize=True, n_segments=nseg)
    torch.cuda.synchronize()
    ro, rf = run_oracle(w, inp)
    assert rel_err(to_host(out), ro) <= 1e-5
    assert rel_err(to_host(state), rf) <= 1e-5


def test_split_resume_matches_one_pass():
    w, inp = small_case("bf16", "gate", 64, 64, 500, B=1, H=2, chunk=64, init=True, seed=11)
    bf = True
    q, k, v = (to_device(inp[n], bf16=bf) for n in ("q", "k", "v"))
    dec = to_device(inp["decay"])
    ini = to_device(inp["init"])
    T1 = 173
    o1, f1 = fla.fwd(q[:, :, :T1].contiguous(), k[:, :, :T1].contiguous(),
                     v[:, :, :T1].contiguous(), dec[:, :, :T1].contiguous(), init_state=ini)
    o2, f2 = fla.fwd(q[:, :, T1:].contiguous(), k[:, :, T1:].contiguous(),
                     v[:, :, T1:].contiguous(), dec[:, :, T1:].contiguous(), init_state=f1)
    torch.cuda.synchronize()
    ro, rf = run_oracle(w, inp)
    o = np.concatenate([to_host(o1), to_host(o2)], axis=2)
    assert rel_err(o, ro) <= 1e-2 and rel_err(to_host(f2), rf) <= 1e-2


@pytest.mark.parametrize("dtype,decay,norm", [("f32", "gate", True), ("bf16", "gamma", False),
                                              ("f32", "none", True), ("bf16", "gate", False),
                                              ("f32", "token", True), ("bf16", "token", False)])
def test_step_chain_matches_oracle(dtype, decay, norm):
    w, inp = small_case(dtype, decay, 64, 32, 20, B=2, H=3, phi=norm, norm=norm, init=True,
                        seed=12)
    bf = dtype == "bf16"
    q, k, v = (to_device(inp[n], bf16=bf) for n in ("q", "k", "v"))
    dec = to_device(inp["decay"])
    state = to_device(inp["init"]).clone()
    outs = []
    for t in range(w.T):
        d = None if dec is None else (dec if decay == "gamma" else dec[:, :, t].contiguous())
        # token: [B,H] per step; gate: [B,H,dk]
        outs.append(fla.step(q[:, :, t].contiguous(), k[:, :, t].contiguous(),
                             v[:, :, t].contiguous(), state, d, decay_kind=decay,
                             phi_elu1=norm, normalize=norm))
    torch.cuda.synchronize()
    o = np.stack([to_host(x) for x in outs], axis=2)
    ro, rf = run_oracle(w, inp)
    assert rel_err(o, ro) <= TOL[dtype]
    assert rel_err(to_host(state), rf) <= TOL[dtype]


@pytest.mark.parametrize("dtype,dk,chunk", [("bf16", 128, 64), ("f32", 64, 32), ("bf16", 32, 16)])
def test_token_decay_equals_broadcast_gate(dtype, dk, chunk):
    """A per-token scalar decay is the per-key gate with every key column equal: both
    library paths against each other, and against the oracle."""
    w, inp = small_case(dtype, "token", dk, 64, 3 * chunk + 11, B=2, H=2, chunk=chunk,
                        init=True, seed=40 + dk)
    check(w, inp, f"token {dtype} dk={dk} C={chunk}")
    ot, ft = run_gpu(w, inp)
    wg = w.with_(decay="gate")
    ig = dict(inp, decay=np.ascontiguousarray(
        np.broadcast_to(inp["decay"][..., None], inp["decay"].shape + (dk,))))
    og, fg = run_gpu(wg, ig)
    assert rel_err(ot, og) <= TOL[dtype] and rel_err(ft, fg) <= TOL[dtype]


def test_single_hip_runtime_in_process():
    maps = open("/proc/self/maps").read()
    libs = {line.split()[-1] for line in maps.splitlines() if "libamdhip64" in line}
    assert len(libs) == 1, libs


@pytest.mark.parametrize("dtype,decay,chunk", [("bf16", "gate", 256), ("bf16", "gamma", 512),
                                               ("f32", "token", 256), ("f32", "none", 512),
                                               ("bf16", "gate", 1024)])
def test_chunk_above_128(dtype, decay, chunk):
    """chunk_size = 512 as the FLA posts advise (and 256, 1024): accepted, evaluated as
    64-token sub-chunks; against the oracle, and bitwise equal to the call with the tile
    size it runs."""
    norm = decay == "none"
    w, inp = small_case(dtype, decay, 64, 64, 2 * chunk + 77, B=1, H=2, chunk=chunk, phi=norm,
                        norm=norm, init=True, seed=chunk + len(decay))
    check(w, inp, f"chunk {chunk} {dtype} {decay}")
    o, f = run_gpu(w, inp)
    o64, f64 = run_gpu(w, inp, chunk=64)
    assert np.array_equal(o, o64) and np.array_equal(f, f64)
