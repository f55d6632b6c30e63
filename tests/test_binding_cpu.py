"""The Python binding checks every tensor against the sizes it hands to the C
ABI (which sees only pointers) before any call: a wrong dtype raises
TypeError, a wrong shape, a non-contiguous tensor or a host tensor raises
ValueError, and nothing reaches the library.  CPU only: every call below is
refused by the binding itself (the last check of each case is that the
tensors are not on a GPU)."""
import pytest
import torch

import compressed_attention_fwht_amd as kvq

B, Hq, Hkv, D, T, W, S, G, C = 2, 8, 2, 128, 40, 16, 2, 16, 256


def _attn(**over):
    a = dict(q=torch.zeros(B, Hq, D), k_codes=torch.zeros(B, Hkv, T, S, G, dtype=torch.uint8),
             v_codes=torch.zeros(B, Hkv, T, S, G, dtype=torch.uint8),
             k_cb=torch.zeros(S, G, C, D // G), v_cb=torch.zeros(S, G, C, D // G),
             k_win=torch.zeros(B, Hkv, W, D, dtype=torch.float16),
             v_win=torch.zeros(B, Hkv, W, D, dtype=torch.float16))
    a.update(over)
    return a


def _call(fn, a, **kw):
    return fn(a["q"], a["k_codes"], a["v_codes"], a["k_cb"], a["v_cb"], a["k_win"], a["v_win"],
              **kw)


@pytest.mark.parametrize("fn", [kvq.attend_decode, kvq.attend_decode_noalloc])
def test_attend_rejects_mismatched_tensors(fn):
    out = torch.zeros(B, Hq, D)
    kw = {"out": out}
    bad_type = [dict(q=torch.zeros(B, Hq, D, dtype=torch.bfloat16)),
                dict(k_codes=torch.zeros(B, Hkv, T, S, G, dtype=torch.int8)),
                dict(v_cb=torch.zeros(S, G, C, D // G, dtype=torch.float64)),
                dict(k_win=torch.zeros(B, Hkv, W, D))]
    for over in bad_type:
        with pytest.raises(TypeError):
            _call(fn, _attn(**over), **kw)
    bad_value = [dict(q=torch.zeros(B, Hq, D, 1)),
                 dict(v_codes=torch.zeros(B, Hkv, T - 1, S, G, dtype=torch.uint8)),
                 dict(v_codes=torch.zeros(B, Hkv, T, S, G + 1, dtype=torch.uint8)),
                 dict(k_codes=torch.zeros(B + 1, Hkv, T, S, G, dtype=torch.uint8)),
                 dict(k_cb=torch.zeros(S, G, C, 4)),
                 dict(v_cb=torch.zeros(S, G, C - 1, D // G)),
                 dict(v_win=torch.zeros(B, Hkv, W + 1, D, dtype=torch.float16)),
                 dict(k_win=torch.zeros(B, Hkv + 1, W, D, dtype=torch.float16)),
                 dict(v_win=None),
                 dict(q=torch.zeros(B, D, Hq).transpose(1, 2))]
    for over in bad_value:
        with pytest.raises(ValueError):
            _call(fn, _attn(**over), **kw)
    with pytest.raises(ValueError):
        _call(fn, _attn(), out=torch.zeros(B, Hq - 1, D))
    with pytest.raises(TypeError):
        _call(fn, _attn(), out=torch.zeros(B, Hq, D, dtype=torch.float16))
    with pytest.raises(ValueError, match="GPU tensor"):      # right sizes, host memory
        _call(fn, _attn(), **kw)


def test_attend_decode_workspace_must_be_bytes():
    with pytest.raises(TypeError):
        kvq.attend_decode(*_attn().values(), workspace=torch.zeros(16, dtype=torch.float32))
    with pytest.raises(ValueError):
        kvq.attend_decode(*_attn().values(), workspace=torch.zeros(4, 4, dtype=torch.uint8))


def test_encode_and_reconstruct_reject_mismatched_tensors():
    x = torch.zeros(2, 3, 50, D, dtype=torch.bfloat16)
    cb = torch.zeros(2, S, G, C, D // G)
    with pytest.raises(TypeError):
        kvq.encode(x.to(torch.int16), cb)
    with pytest.raises(TypeError):
        kvq.encode(x, cb.double())
    with pytest.raises(ValueError):
        kvq.encode(x, torch.zeros(1, S, G, C, D // G))                # one book, two inputs
    with pytest.raises(ValueError):
        kvq.encode(x, torch.zeros(2, S, 12, C, 10))                    # 12 x 10 != 128
    with pytest.raises(ValueError):
        kvq.encode(x, cb, n_rows=40, codes=torch.zeros(2, 3, 50, S, G, dtype=torch.uint8))
    with pytest.raises(TypeError):
        kvq.encode(x, cb, codes=torch.zeros(2, 3, 50, S, G, dtype=torch.int32))
    with pytest.raises(ValueError, match="GPU tensor"):
        kvq.encode(x, cb)
    codes = torch.zeros(2, 70, S, G, dtype=torch.uint8)
    with pytest.raises(ValueError):
        kvq.decode_reconstruct(codes, torch.zeros(2, S + 1, G, C, D // G))
    with pytest.raises(ValueError):
        kvq.decode_reconstruct(codes[:1], cb)
    with pytest.raises(ValueError):
        kvq.decode_reconstruct(codes, cb, out=torch.zeros(2, 69, D))
    with pytest.raises(TypeError):
        kvq.decode_reconstruct(codes, cb, out=torch.zeros(2, 70, D, dtype=torch.float16))
    with pytest.raises(ValueError, match="GPU tensor"):
        kvq.decode_reconstruct(codes, cb)


def test_rotate_and_scalar_calls_reject_mismatched_tensors():
    x = torch.zeros(10, D)
    with pytest.raises(ValueError):
        kvq.rotate(x, out=torch.zeros(10, D + 1))
    with pytest.raises(TypeError):
        kvq.rotate(x, out=torch.zeros(10, D, dtype=torch.bfloat16))
    with pytest.raises(TypeError):
        kvq.rotate(x.long())
    xs = torch.zeros(2, 1, 30, D)
    lv = torch.zeros(2, 2, 4)
    with pytest.raises(ValueError):
        kvq.scalar_encode(xs, torch.zeros(2, 2, 8), 2)                 # 8 levels for 2 bits
    with pytest.raises(ValueError):
        kvq.scalar_encode(xs, lv, 2, codes=torch.zeros(2, 1, 30, 2, 16, dtype=torch.uint8))
    with pytest.raises(ValueError):
        kvq.scalar_encode(xs, lv, 5)
    codes = torch.zeros(2, 30, 2, D * 2 // 8, dtype=torch.uint8)
    with pytest.raises(ValueError):
        kvq.scalar_decode_reconstruct(codes, torch.zeros(1, 2, 4), 2)
    with pytest.raises(ValueError):
        kvq.scalar_decode_reconstruct(codes, lv, 2, out=torch.zeros(2, 30, D // 2))
    with pytest.raises(ValueError):
        kvq.scalar_product_codebook(torch.zeros(2, 4), 2, D, out=torch.zeros(2, 32, 256, 2))
    with pytest.raises(ValueError, match="GPU tensor"):
        kvq.scalar_product_codebook(torch.zeros(2, 4), 2, D)


def test_streaming_calibration_and_fit_reject_mismatched_tensors():
    kw = torch.zeros(B, Hkv, W, D, dtype=torch.float16)
    new = torch.zeros(B, Hkv, D, dtype=torch.float16)
    with pytest.raises(ValueError):
        kvq.window_append(new[:1], new, kw, kw, 3)
    with pytest.raises(TypeError):
        kvq.window_append(new.float(), new, kw, kw, 3)
    kc = torch.zeros(B, Hkv, T, S, G, dtype=torch.uint8)
    cb = torch.zeros(S, G, C, D // G)
    with pytest.raises(ValueError):
        kvq.window_flush(kw, kw, W, 4, kc, kc[:, :, :-1].contiguous(), 0, cb, cb)
    with pytest.raises(ValueError):
        kvq.window_flush(kw, kw, W, 4, kc, kc, 0, cb, torch.zeros(S, G, C, 4))
    with pytest.raises(ValueError, match="GPU tensor"):
        kvq.window_flush(kw, kw, W, 4, kc, kc, 0, cb, cb)
    x = torch.zeros(1, 4, 30, D)
    with pytest.raises(ValueError):
        kvq.smooth_calibrate(x, 2, out=torch.zeros(1, 1, D))
    with pytest.raises(ValueError):
        kvq.smooth_calibrate(x[0])
    with pytest.raises(ValueError):
        kvq.codebook_fit(torch.zeros(100, D), torch.zeros(S, G, C, 4), 2)
    with pytest.raises(TypeError):
        kvq.codebook_fit(torch.zeros(100, D), cb, 2, workspace=torch.zeros(8))
