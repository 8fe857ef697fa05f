"""GPU: the measurement probes behind include/fla_probe.h move the bytes they claim to move.

The streaming probes are checked against their definitions (copy: dst = src; five reads
per write: output vector j = XOR of input vectors j, j + m, ..., j + 4m) and the forward
pass's access-pattern probe against a numpy restatement of its lane mapping (each output
vector = the value vector XOR the XOR of the q, k and gate vectors read by the same lane),
including a ragged last chunk whose rows past T are neither read nor written.
"""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import chunkwise_causal_linear_amd as fla  # noqa: E402


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def test_copy_and_mix5_probes():
    say("probe: copy and mix5, 1.5 MiB")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(7)
    nbytes = 96 * 16 * 1024
    src = torch.randint(-2**31, 2**31 - 1, (nbytes // 4,), generator=gen, device="cuda",
                        dtype=torch.int32)
    dst = torch.zeros(nbytes // 4, dtype=torch.int32, device="cuda")
    fla.probe_stream(src, dst, nbytes, fla.PROBE_COPY)
    torch.cuda.synchronize()
    assert torch.equal(dst, src)
    dst.zero_()
    fla.probe_stream(src, dst, nbytes, fla.PROBE_MIX5)
    torch.cuda.synchronize()
    m = nbytes // 6 // 16                      # output vectors
    s = src.cpu().numpy().view(np.uint32).reshape(-1, 4)
    want = s[0:m] ^ s[m:2 * m] ^ s[2 * m:3 * m] ^ s[3 * m:4 * m] ^ s[4 * m:5 * m]
    got = dst.cpu().numpy().view(np.uint32).reshape(-1, 4)
    assert np.array_equal(got[:m], want)
    assert not got[m:].any()


def pattern_reference(q, k, g, v, T):
    """numpy restatement of fla_probe_chunk_pattern's output (uint32 words)."""
    B, H, _, dk = q.shape
    dv = v.shape[-1]
    qw = q.view(torch.int16).cpu().numpy().view(np.uint16)
    kw = k.view(torch.int16).cpu().numpy().view(np.uint16)
    vw = v.view(torch.int16).cpu().numpy().view(np.uint16)
    gw = g.cpu().numpy().view(np.uint32)
    out = np.zeros((B, H, T, dv), dtype=np.uint16)
    for b in range(B):
        for h in range(H):
            for t0 in range(0, T, 64):
                L = min(64, T - t0)

                def vecs(a, words):   # rows t0.. of one head, zero-padded to 64 rows
                    x = np.zeros((64,) + a.shape[3:], dtype=a.dtype)
                    x[:L] = a[b, h, t0:t0 + L]
                    return x.reshape(-1).view(np.uint32).reshape(words, 256, 4)

                x = (np.bitwise_xor.reduce(vecs(qw, 4), axis=0)
                     ^ np.bitwise_xor.reduce(vecs(kw, 4), axis=0)
                     ^ np.bitwise_xor.reduce(vecs(gw, 8), axis=0))        # [lane][4]
                for vs in range(dv // 64):
                    sl = np.zeros((64, 64), dtype=np.uint16)
                    sl[:L] = vw[b, h, t0:t0 + L, 64 * vs:64 * vs + 64]
                    sv = sl.reshape(-1).view(np.uint32).reshape(512, 4)   # vector j = row j/8
                    o = sv ^ x[np.arange(512) % 256]
                    out[b, h, t0:t0 + L, 64 * vs:64 * vs + 64] = \
                        o.reshape(-1).view(np.uint16).reshape(64, 64)[:L]
    return out


@pytest.mark.parametrize("B,H,T,dv", [(1, 3, 200, 128), (2, 2, 64, 64), (1, 9, 130, 256)])
def test_chunk_pattern_probe(B, H, T, dv):
    say(f"probe: chunk pattern B={B} H={H} T={T} dv={dv}")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(11 + T)
    q = torch.randn((B, H, T, 128), generator=gen, device="cuda").to(torch.bfloat16)
    k = torch.randn((B, H, T, 128), generator=gen, device="cuda").to(torch.bfloat16)
    g = torch.rand((B, H, T, 128), generator=gen, device="cuda")
    v = torch.randn((B, H, T, dv), generator=gen, device="cuda").to(torch.bfloat16)
    out = torch.zeros_like(v)
    fla.probe_chunk_pattern(q, k, g, v, out)
    torch.cuda.synchronize()
    got = out.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, pattern_reference(q, k, g, v, T))
