"""Unit tests of the tolerance checker with constructed near ties.  CPU only."""
import numpy as np

import oracle
from oracle import check_codes, check_recon, check_attn, rvq_encode


def _two_point_book(eps):
    # codewords at distance^2 1 and 1+eps from the origin-centred input
    cb = np.zeros((1, 1, 3, 2))
    cb[0, 0, 0] = [1.0, 0.0]
    cb[0, 0, 1] = [0.0, np.sqrt(1.0 + eps)]
    cb[0, 0, 2] = [5.0, 5.0]
    return cb


def test_exact_match_counts():
    rng = np.random.default_rng(0)
    cb = rng.standard_normal((2, 4, 256, 8))
    x = rng.standard_normal((100, 32))
    codes = rvq_encode(x, cb)
    res = check_codes(x, cb, codes)
    assert res == {**res, "total": 800, "exact": 800, "near_tie": 0, "hard": 0}


def test_near_tie_is_accepted_and_far_choice_is_hard():
    x = np.zeros((1, 2))
    cb = _two_point_book(5e-5)          # second-best within 1e-4 relative
    res = check_codes(x, cb, np.array([[[1]]], dtype=np.uint8), rotate=False)
    assert res["near_tie"] == 1 and res["hard"] == 0
    cb = _two_point_book(5e-4)          # outside the tolerance
    res = check_codes(x, cb, np.array([[[1]]], dtype=np.uint8), rotate=False)
    assert res["hard"] == 1 and res["hard_examples"][0][3:] == (1, 0)
    res = check_codes(x, cb, np.array([[[2]]], dtype=np.uint8), rotate=False)
    assert res["hard"] == 1


def test_teacher_forcing_follows_the_candidate():
    """After an accepted near tie at stage 0, stage 1 is checked from the
    candidate's residual, where the candidate's stage-1 code is exact."""
    cb = np.zeros((2, 1, 2, 2))
    cb[0, 0, 0] = [1.0, 0.0]
    cb[0, 0, 1] = [0.0, 1.0 + 1e-6]
    cb[1, 0, 0] = [-1.0, 0.0]            # best follow-up to choice 0
    cb[1, 0, 1] = [0.0, -1.0]            # best follow-up to choice 1
    x = np.zeros((1, 2))
    res = check_codes(x, cb, np.array([[[1], [1]]], dtype=np.uint8), rotate=False)
    assert res["near_tie"] == 1 and res["exact"] == 1 and res["hard"] == 0
    res = check_codes(x, cb, np.array([[[1], [0]]], dtype=np.uint8), rotate=False)
    assert res["hard"] == 1


def test_recon_and_attn_rules():
    ref = np.linspace(-3, 3, 50)
    assert check_recon(ref + 9e-7, ref)["ok"]
    assert not check_recon(ref + 2e-6, ref)["ok"]
    ref = np.ones((2, 3, 64))
    assert check_attn(ref + 1e-4, ref)["ok"]
    assert not check_attn(ref + 3e-3, ref)["ok"]          # max-abs rule
    small = np.full((2, 3, 64), 1e-3)
    r = check_attn(small * 1.5, small)                    # relative L2 rule
    assert r["max_abs"] < 2e-3 and not r["ok"]


def test_scalar_checker_rules():
    """Exact indices pass; an index on the wrong side of a threshold by a hair
    (squared distances within 1e-4 relative) is a near tie; one 1e-4 of the
    spacing away is hard; a far one is hard; stage 2 follows the candidate's
    stage 1."""
    lv1 = np.array([-1.5, -0.5, 0.5, 1.5])
    lv2 = np.array([-0.3, -0.1, 0.1, 0.3])
    y = np.array([[0.2, -0.9, 1.0 + 1e-7, 1.4] * 4])            # rms ~ 1
    z1 = oracle.scalar_nearest(y, lv1)
    z2 = oracle.scalar_nearest(y - lv1[z1], lv2)
    res = oracle.check_scalar_codes(y, lv1, lv2, z1, z2)
    assert res["exact"] == res["total"] == 32 and res["hard"] == 0
    zt = z1.copy()
    zt[0, 2] = 2                                                 # 1.0 + 1e-7: threshold by a hair
    z2t = oracle.scalar_nearest(y - lv1[zt], lv2)                # stage 2 on the candidate's residual
    res = oracle.check_scalar_codes(y, lv1, lv2, zt, z2t)
    assert res["near_tie"] == 1 and res["hard"] == 0
    yh = y.copy()
    yh[0, 2] = 1.0 + 1e-4                                        # (d_c / d_1) - 1 ~ 4e-4: hard
    z1h = oracle.scalar_nearest(yh, lv1)
    zh = z1h.copy()
    zh[0, 2] = 2
    z2h = oracle.scalar_nearest(yh - lv1[zh], lv2)
    res = oracle.check_scalar_codes(yh, lv1, lv2, zh, z2h)
    assert res["hard"] == 1 and res["near_tie"] == 0
    zf = z1.copy()
    zf[0, 0] = 0                                                 # 0.2 coded as -1.5: hard
    res = oracle.check_scalar_codes(y, lv1, lv2, zf, z2)
    assert res["hard"] >= 1
