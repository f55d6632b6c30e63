"""The decode and encode calls captured into HIP graphs (torch.cuda.CUDAGraph on
the capturing stream): they allocate nothing, clear nothing with memset and
never synchronise, so a captured call replays the same kernels.  Each graph is
replayed several times with the program's own eager work and synchronisations
in between, and every replay is compared with the eager result bit for bit
(the kernels are deterministic); a replay after the inputs change in place
must follow the new inputs."""
import sys

import numpy as np
import pytest
import torch

import synth
import compressed_attention_fwht_amd as kvq

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()


def cuda(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _capture(fn):
    side = torch.cuda.Stream()                           # default priority
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()                                             # warm-up off the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("key,over", [
    (2, dict(tokens=3000, window=128)),                  # LUT built in the chunk blocks
    (2, dict(batch=3, tokens=7000, window=128, n_stages=3)),  # LUT staged from its own pass
    (4, dict(tokens=40000, window=256)),                 # rotated-code kernels, four stages
])
def test_decode_graph_replays_match_eager(key, over):
    say(f"decode graph workload {key} {over}")
    w = synth.workload(key, **over)
    inp = synth.make_inputs(w)
    rng = np.random.default_rng(key)
    B, Hkv, Tc, S, G = w.batch, w.n_kv_heads, w.code_tokens, w.n_stages, w.n_groups
    kc = cuda(rng.integers(0, 256, size=(B, Hkv, Tc, S, G), dtype=np.uint8))
    vc = cuda(rng.integers(0, 256, size=(B, Hkv, Tc, S, G), dtype=np.uint8))
    kcb, vcb = cuda(inp["cb"][0]), cuda(inp["cb"][1])
    kw, vw = cuda(inp["k_win"]), cuda(inp["v_win"])
    q = cuda(inp["q"])
    D, Hq, W, C = w.head_dim, w.n_q_heads, w.window, w.n_codewords
    ws = torch.empty(kvq.attend_workspace_size(B, Hq, Hkv, D, Tc, W, S, G, C), dtype=torch.uint8,
                     device="cuda")
    out = torch.empty((B, Hq, D), dtype=torch.float32, device="cuda")
    g = _capture(lambda: kvq.attend_decode(q, kc, vc, kcb, vcb, kw, vw, out=out, workspace=ws))
    eager = kvq.attend_decode(q, kc, vc, kcb, vcb, kw, vw)
    for i in range(4):
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), i
        other = kvq.attend_decode(q * 0.5, kc, vc, kcb, vcb, kw, vw)   # eager work between
        torch.cuda.synchronize()
        assert not torch.equal(other, eager)
    q.copy_(torch.flip(q, dims=[1]))                      # new inputs, same buffers
    g.replay()
    torch.cuda.synchronize()
    assert torch.equal(out, kvq.attend_decode(q, kc, vc, kcb, vcb, kw, vw))


def test_encode_graph_replays_match_eager():
    say("encode graph, codebooks packed before the capture")
    w = synth.workload(3, batch=1, tokens=3000, window=0)
    inp = synth.make_inputs(w)
    x = torch.from_numpy(inp["x"].view(np.int16)).view(torch.bfloat16).cuda()
    cb = cuda(inp["cb"])
    ws = torch.empty(kvq.encode_workspace_size(128, 16, 2, 256, 2), dtype=torch.uint8,
                     device="cuda")
    eager = kvq.encode(x, cb, workspace=ws)              # also packs the codebooks
    codes = torch.empty_like(eager)
    g = _capture(lambda: kvq.encode(x, cb, codes=codes, workspace=ws, packed=True))
    for i in range(4):
        codes.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(codes, eager), i
        kvq.decode_reconstruct(eager, cb, unrotate=True)  # eager work between replays
        torch.cuda.synchronize()
    x.copy_(torch.flip(x, dims=[2]))
    g.replay()
    torch.cuda.synchronize()
    assert torch.equal(codes, kvq.encode(x, cb, workspace=ws, packed=True))
