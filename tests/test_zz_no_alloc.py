"""kvq_attend_decode_noalloc (decode attention in the library's own per-GPU
device array) against kvq_attend_decode with a workspace of its own: the same
kernels and plan, so the outputs must agree bit for bit, and both meet the
oracle's attention bar (2e-3 max-abs, 1e-3 relative L2).  Calls run back to
back on the one array, each smaller than the one before, so a call that read
what an earlier one left behind would show."""
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
import compressed_attention_fwht_amd as kvq

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def cuda(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _case(key, over):
    w = synth.workload(key, **over)
    inp = synth.make_inputs(w)
    Tc = w.code_tokens
    shp = (w.batch, w.n_kv_heads, Tc, w.n_stages, w.n_groups)
    codes = [oracle.rvq_encode(inp["x_f32"][b][:, :Tc].reshape(-1, w.head_dim),
                               inp["cb"][b]).reshape(shp) for b in range(2)]
    args = (cuda(inp["q"]), cuda(codes[0]), cuda(codes[1]), cuda(inp["cb"][0]),
            cuda(inp["cb"][1]), cuda(inp["k_win"]), cuda(inp["v_win"]))
    ref = oracle.attend(inp["q"], codes[0], codes[1], inp["cb"][0], inp["cb"][1], inp["k_win"],
                        inp["v_win"])
    sz = kvq.attend_workspace_size(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, Tc, w.window,
                                   w.n_stages, w.n_groups, w.n_codewords)
    return args, ref, sz


def test_noalloc_matches_workspace_call_on_shrinking_calls():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    torch.cuda.set_device(0)
    # four-stage long-context cache, then a smaller two-stage GQA-7 batch,
    # then a one-stage cache with a D-64 head
    cases = [(4, dict(tokens=5000, window=256)), (3, dict(batch=2, tokens=2100, window=64)),
             (1, dict(tokens=1500))]
    prev = None
    for key, over in cases:
        say(f"decode no-alloc workload {key} {over}")
        args, ref, sz = _case(key, over)
        assert sz <= kvq.NOALLOC_SCRATCH_BYTES
        if prev is not None:
            assert sz < prev
        prev = sz
        want = kvq.attend_decode(*args).cpu().numpy()
        out = torch.empty(args[0].shape, dtype=torch.float32, device="cuda")
        torch.cuda.synchronize()
        before = torch.cuda.memory_allocated()
        for rep in range(2):
            out.fill_(float("nan"))
            kvq.attend_decode_noalloc(*args, out=out)
            torch.cuda.synchronize()
            assert torch.cuda.memory_allocated() == before
            got = out.cpu().numpy()
            assert np.array_equal(got, want), (key, rep)
        res = oracle.check_attn(got, ref)
        say("   ", res)
        assert res["ok"], res


def test_noalloc_refuses_oversized_workspace():
    torch.cuda.set_device(0)
    B, Hq, Hkv, Tc, W = 64, 28, 4, 8128, 64
    assert kvq.attend_workspace_size(B, Hq, Hkv, 128, Tc, W, 2, 16, 256) \
        > kvq.NOALLOC_SCRATCH_BYTES
    # the call is refused before it launches anything
    q = torch.zeros(B, Hq, 128, device="cuda")
    kc = torch.zeros(B, Hkv, Tc, 2, 16, dtype=torch.uint8, device="cuda")
    cb = torch.zeros(2, 16, 256, 8, device="cuda")
    win = torch.zeros(B, Hkv, W, 128, dtype=torch.float16, device="cuda")
    out = torch.zeros(B, Hq, 128, device="cuda")
    with pytest.raises(kvq.KvqError):
        kvq.attend_decode_noalloc(q, kc, kc, cb, cb, win, win, out=out)
