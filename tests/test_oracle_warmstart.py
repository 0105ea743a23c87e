"""Pins for oracle/warmstart.py (the int4-g32 page's warm-start magnitude fit).

* the candidate set and its 8-bit parameter codes (family, b_rel, beta), with
  b_rel against numpy's own logspace;
* every inverse inverts its transform: beta = 1 and tanh to rounding, beta < 1
  against the page's fixed-point iteration run to a standstill, within the
  bound the result's own residual gives;
* the f-space grid: levels ascending from 0, the top level back at gmax, and
  every weight's q the nearest grid point;
* a scalar brute force (math.pow / tanh / atanh, Python sums) of every
  candidate's squared error on a few groups: the oracle's sums agree and its
  choice is a minimum;
* Lloyd never raises a group's error above its warm start (page section 1.3,
  step 3), and on Student-t groups the page's ordering of section 1.4 holds:
  warm start < parametric alone < cold (quantile) start;
* all-zero and single-value groups.
"""

import math

import numpy as np
import pytest

import synthetic
from oracle import bits, lut16, warmstart

CANDS = warmstart.candidates()


def _groups(n, seed, nu=5):
    w = synthetic.student_t_bf16((n, 32), nu, 0.02, seed)
    return np.abs(bits.bf16_to_f64(w))


def test_candidate_codes():
    assert len(CANDS) == warmstart.N_CAND == 112
    codes = [c[0] for c in CANDS]
    assert codes == sorted(codes) and len(set(codes)) == 112
    for code, family, b_rel, beta in CANDS:
        assert family == code >> 7
        bi = (code >> 3) & 15
        if family == 0:
            assert b_rel == warmstart.B_REL_RAT[bi] and beta == warmstart.BETAS[code & 7]
        else:
            assert b_rel == warmstart.B_REL_TANH[bi] and code & 7 == 0
    assert np.allclose(warmstart.B_REL_RAT, np.logspace(-3, 2, 15), rtol=1e-15, atol=0)


def _iterate_to_standstill(fd, b, beta):
    """The page's iteration w <- fd*b + fd*w**beta from the beta = 1 solution,
    run until a value repeats (at most 100000 steps)."""
    w = (fd * b) / (1.0 - fd)
    seen = set()
    for _ in range(100000):
        if w in seen:
            break
        seen.add(w)
        w = fd * b + fd * w ** beta
    return w


@pytest.mark.parametrize("family,beta", [(0, 1.0), (0, 0.5), (0, 0.75), (0, 0.95), (1, None)])
def test_inverse_inverts_the_transform(family, beta):
    a = _groups(64, 11)
    gmax = a.max(axis=-1)
    for b_rel in (warmstart.B_REL_TANH if family else warmstart.B_REL_RAT):
        b = b_rel * gmax
        fmax = warmstart.forward(gmax[:, None], b, family, beta)[:, 0]
        fd = np.linspace(0, 1, 9)[None, :] * fmax[:, None]
        w = warmstart.inverse(fd, b, family, beta, gmax)
        if family == 1 or beta == 1.0:
            back = warmstart.forward(w, b, family, beta)
            assert np.allclose(back, fd, rtol=1e-12, atol=0), b_rel
            continue
        # beta < 1: the fixed point of w <- fd*b + fd*w**beta.  With r the
        # residual of that equation at the result and s the map's slope
        # fd * beta * w**(beta - 1) at the smaller of the result and a root
        # found here by the page's own iteration run to a standstill (the map
        # is concave, so s bounds the secant slope), the mean value theorem
        # gives |w - w*| <= r / (1 - s) when s < 1.
        for r in range(0, 64, 7):
            for j in range(1, 9):
                ws = _iterate_to_standstill(fd[r, j], b[r], beta)
                wr = w[r, j]
                res = abs(fd[r, j] * b[r] + fd[r, j] * wr ** beta - wr)
                sl = fd[r, j] * beta * min(wr, ws) ** (beta - 1)
                assert sl < 1, (b_rel, r, j)
                # + rounding: g is evaluated to a few ulps of w
                slack = 8 * 2.0 ** -52 * ws / (1 - sl)
                assert abs(wr - ws) <= res / (1 - sl) + slack, (b_rel, r, j)
                assert abs(wr - ws) <= 1e-13 * ws, (b_rel, r, j)


def test_grid_levels_and_nearest_q():
    a = _groups(128, 12)
    gmax = a.max(axis=-1)
    for code, family, b_rel, beta in CANDS[::5] + CANDS[-7:]:
        lev, q, _ = warmstart.candidate_levels(a, family, b_rel, beta)
        assert np.all(lev[:, 0] == 0) and np.all(np.diff(lev, axis=-1) > 0), code
        # the top level goes back to gmax: exactly up to rounding for the closed
        # forms, within the fixed point's reach otherwise
        assert np.allclose(lev[:, 7], gmax, rtol=1e-9, atol=0), code
        b = b_rel * gmax
        f = warmstart.forward(a, b, family, beta)
        fmax = warmstart.forward(gmax[:, None], b, family, beta)
        t = f / fmax * 7.0
        assert np.all(np.abs(t - q) <= 0.5), code


def _brute_sse(a, family, b_rel, beta):
    """Scalar statement of one candidate's squared error for one group."""
    gmax = max(a)
    b = b_rel * gmax
    if family == 1:
        f = lambda w: math.tanh(w / b)
        inv = lambda fd: b * math.atanh(fd)
    else:
        f = lambda w: w / (b + (w if beta == 1.0 else math.pow(w, beta)))

        def inv(fd):
            if beta == 1.0:
                return (fd * b) / (1.0 - fd)
            return _iterate_to_standstill(fd, b, beta) if fd > 0 else 0.0
    fmax = f(gmax)
    levels = [inv((q / 7.0) * fmax) for q in range(8)]
    sse = 0.0
    for w in a:
        q = min(7, max(0, round(f(w) / fmax * 7.0)))   # Python round: half to even
        sse += (w - levels[q]) ** 2
    return sse


def test_candidate_errors_vs_scalar_bruteforce():
    a = _groups(6, 13)
    lev, code, sses = warmstart.warm_start(a)
    for gi in range(a.shape[0]):
        brute = np.array([_brute_sse(list(a[gi]), fam, br, be) for _, fam, br, be in CANDS])
        assert np.allclose(sses[gi], brute, rtol=1e-12, atol=0), gi
        best = int(np.searchsorted([c[0] for c in CANDS], code[gi]))
        assert brute[best] <= brute.min() * (1 + 1e-12), gi


def test_lloyd_never_worse_than_the_warm_start_and_page_ordering():
    a = _groups(2048, 14)
    lev, code, sses = warmstart.warm_start(a)
    c = lut16.lloyd(a, lev, lut16.LLOYD_ITERS)
    s_near = warmstart.group_sse(a, lev)
    s_warm = warmstart.group_sse(a, c)
    s_param = sses.min(axis=-1)       # the chosen candidate's own (f-space) error
    # nearest-level assignment can only lower the candidate's error, and each
    # Lloyd round lowers it further
    assert np.all(s_near <= s_param * (1 + 1e-12))
    assert np.all(s_warm <= s_near * (1 + 1e-12))
    # section 1.4: warm < parametric < cold start, as relative weight errors
    c_cold = lut16.lloyd(a, lut16.quantile_init(a, 8), lut16.LLOYD_ITERS)
    s_cold = warmstart.group_sse(a, c_cold)
    tot = (a ** 2).sum()
    e_warm, e_param, e_cold = (np.sqrt(s.sum() / tot) for s in (s_warm, s_param, s_cold))
    assert e_warm < e_param < e_cold, (e_warm, e_param, e_cold)


def test_fit_output_and_degenerate_groups():
    w = synthetic.student_t_bf16((3, 128), 5, 0.02, 15)
    w[0, :32] = 0                                   # all zero
    w[1, 32:64] = 0
    w[1, 40] = 0x3C00                               # one nonzero value (2**-7)
    w[2, 64:96] = bits.rne_bf16(np.full(32, -0.25))  # one magnitude
    M, code = warmstart.fit(w)
    assert M.shape == (3, 4, 8) and code.shape == (3, 4) and M.dtype == np.uint16
    assert np.all(M[0, 0] == 0) and code[0, 0] == 0
    # every Lloyd level is a mean of members or a start level: finite, >= 0
    Mv = bits.f16_to_f64(M)
    assert np.all(np.isfinite(Mv)) and np.all(Mv >= 0)
    # a group's largest magnitude is always a level's member: the level
    # nearest to it is within the level spacing; for the one-value groups it
    # is that value exactly
    assert bits.f16_to_f64(M[1, 1]).max() == 2.0 ** -7
    assert 0.25 in bits.f16_to_f64(M[2, 2])
