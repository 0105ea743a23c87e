"""Warm-start fit of the SIGNMAG8 magnitudes: a parametric transform chosen
per group gives the 8 starting levels, Lloyd rounds refine them.

Oracle (test infrastructure).  int4-g32 page:

* section 1.2: two transform families over the group's magnitudes -- the
  bounded rational ``f(w) = c*w / (b + |w|**beta)`` with ``b = b_rel * gmax``,
  ``b_rel`` in logspace(-3, 2, 15) and beta in {0.50, 0.55, 0.65, 0.75, 0.85,
  0.95, 1.00} (105 candidates), and ``f(w) = tanh(w / b)`` with b_rel in
  {0.25, 0.4, 0.6, 0.85, 1.2, 1.8, 3.0} (7 candidates); inverses: beta = 1
  ``w = fd*b / (1 - fd)``, beta < 1 the fixed point of ``w <- fd*b + fd*w**beta``,
  tanh ``w = b * atanh(fd)``;
* section 1.3 steps 1-3 and section 5.1: for each candidate, 8 uniform levels
  in f-space (``q = round(f / fmax * 7)`` clamped to 0..7), rebuilt by the
  inverse at ``q/7 * fmax``; the candidate with the smallest mean squared
  error over the group wins; its 8 rebuilt levels start 25 Lloyd rounds;
* section 2: the per-group parameter code is 8 bits -- family (1), b_rel
  index (4), beta index (3).

Readings (listed in the design notes):

* ``c`` cancels in ``f / fmax`` and is left out; ``fmax = f(gmax)``;
* the candidates are tried in increasing parameter code, ``code = family << 7
  | b_idx << 3 | beta_idx`` (tanh: beta_idx 0), and the lowest code wins a tie
  of the squared-error sums;
* ``round`` is round-half-to-even; ``b_rel = 10 ** ((5 i - 42) / 14)``;
* beta < 1: the inverse is the fixed point itself (the root of
  ``w = fd*b + fd*w**beta``) to fp64 precision, not a fixed number of steps
  towards it: near the root the page's iteration contracts only by
  ``beta * w**beta / (b + w**beta)`` per step (up to 0.95), so 100 steps can
  leave a top level 2% short of gmax;
* every step in fp64 in the order written on the page: ``f / fmax * 7`` is
  ``(f / fmax) * 7``, a level is ``(q / 7) * fmax``, the error sum runs over
  the group's weights in element order;
* Lloyd as in the cold-start fit (nearest level, lowest on a tie; member sums
  in element order; an empty level keeps its value), then RNE to fp16;
* a group of all zeros gets 8 zero levels and code 0.

The libm functions used here (pow, tanh, atanh) and the GPU's own may differ
in the last bits, so the GPU is compared with this within the tolerance its
tests state.  The fitted levels themselves are "parity unpinned" (a heuristic
start and a local optimum); the steps are pinned by procedure and by the
mathematics in ``tests/test_oracle_warmstart.py``.
"""

import numpy as np

from .bits import bf16_to_f64, rne_fp16
from .lut16 import lloyd, LLOYD_ITERS

GROUP = 32
N_MAG = 8
BETAS = (0.50, 0.55, 0.65, 0.75, 0.85, 0.95, 1.00)
B_REL_RAT = tuple(10.0 ** ((5 * i - 42) / 14) for i in range(15))
B_REL_TANH = (0.25, 0.4, 0.6, 0.85, 1.2, 1.8, 3.0)
# halvings of [0, 2 gmax]: the smallest nonzero level is above gmax * 2**-130
# for every candidate, so 200 reach adjacent fp64 values
BISECT_STEPS = 200
N_CAND = len(BETAS) * len(B_REL_RAT) + len(B_REL_TANH)   # 112


def candidates():
    """[(code, family, b_rel, beta)] in increasing code (family 0: rational,
    1: tanh; beta None for tanh)."""
    out = []
    for bi, br in enumerate(B_REL_RAT):
        for ki, beta in enumerate(BETAS):
            out.append(((bi << 3) | ki, 0, br, beta))
    for bi, br in enumerate(B_REL_TANH):
        out.append((128 | (bi << 3), 1, br, None))
    return out


def forward(a, b, family, beta, apow=None):
    """f(a) for magnitudes a [G, n] and b [G] (apow: a**beta if known)."""
    if family == 1:
        return np.tanh(a / b[:, None])
    if beta == 1.0:
        return a / (b[:, None] + a)
    if apow is None:
        apow = np.power(a, beta)
    return a / (b[:, None] + apow)


def _residual(w, fd, bb, beta):
    """g(w) = w - (fd*b + fd*w**beta): negative at 0 (for fd > 0), convex, one
    root on w > 0, the fixed point of the page's iteration."""
    return w - (fd * bb + fd * np.power(w, beta))


def inverse(fd, b, family, beta, gmax):
    """w with f(w) = fd, for fd [G, n] in [0, fmax] and b, gmax [G].

    beta < 1: the root of ``w = fd*b + fd*w**beta`` to fp64 precision, by
    bisection on [0, 2*gmax] (f increases and fd <= f(gmax), so the root is at
    most gmax), ending on the fp64 endpoint with the smaller |g| (the lower
    one on a tie).  fd = 0 gives 0."""
    bb = b[:, None]
    if family == 1:
        return bb * np.arctanh(fd)
    w1 = (fd * bb) / (1.0 - fd)
    if beta == 1.0:
        return w1
    lo = np.zeros_like(fd)
    hi = np.broadcast_to(2.0 * gmax[:, None], fd.shape).copy()
    for _ in range(BISECT_STEPS):
        mid = 0.5 * (lo + hi)
        neg = _residual(mid, fd, bb, beta) <= 0.0
        lo = np.where(neg, mid, lo)
        hi = np.where(neg, hi, mid)
    glo = np.abs(_residual(lo, fd, bb, beta))
    ghi = np.abs(_residual(hi, fd, bb, beta))
    return np.where(ghi < glo, hi, lo)


def candidate_levels(a, family, b_rel, beta):
    """For magnitudes a [G, 32] (gmax > 0): (levels [G, 8], q [G, 32], sse [G])
    of one candidate."""
    gmax = np.max(a, axis=-1)
    b = b_rel * gmax
    apow = None if (family == 1 or beta == 1.0) else np.power(a, beta)
    f = forward(a, b, family, beta, apow)
    fmax = forward(gmax[:, None], b, family, beta,
                   None if apow is None else np.power(gmax[:, None], beta))[:, 0]
    q = np.clip(np.rint((f / fmax[:, None]) * 7.0), 0, 7).astype(np.int64)
    fd = (np.arange(8) / 7.0)[None, :] * fmax[:, None]
    lev = inverse(fd, b, family, beta, gmax)
    wr = np.take_along_axis(lev, q, axis=-1)
    sse = np.zeros(a.shape[0])
    for i in range(a.shape[-1]):            # element order
        d = a[:, i] - wr[:, i]
        sse = sse + d * d
    return lev, q, sse


def warm_start(a):
    """Best candidate per group of magnitudes a [G, 32]: (levels [G, 8] fp64,
    code [G] uint8, sse of every candidate [G, 112]).  All-zero groups:
    zero levels, code 0."""
    a = np.asarray(a, dtype=np.float64)
    g = a.shape[0]
    gmax = np.max(a, axis=-1)
    live = gmax > 0
    al = a[live] if not live.all() else a
    levs, sses, codes = [], [], []
    for code, family, b_rel, beta in candidates():
        lev, _, sse = candidate_levels(al, family, b_rel, beta)
        levs.append(lev)
        sses.append(sse)
        codes.append(code)
    sses = np.stack(sses, axis=-1)                    # [G', 112]
    best = np.argmin(sses, axis=-1)                   # first minimum = lowest code
    lev_all = np.stack(levs, axis=1)                  # [G', 112, 8]
    out_lev = np.zeros((g, N_MAG))
    out_code = np.zeros(g, dtype=np.uint8)
    out_sse = np.zeros((g, N_CAND))
    out_lev[live] = lev_all[np.arange(al.shape[0]), best]
    out_code[live] = np.asarray(codes, dtype=np.uint8)[best]
    out_sse[live] = sses
    return out_lev, out_code, out_sse


def fit(w_bits, iters=LLOYD_ITERS):
    """Warm-start fit.  w [N, K] bf16 bits -> (fp16 bits [N, K/32, 8], parameter
    code uint8 [N, K/32])."""
    w_bits = np.asarray(w_bits)
    n, k = w_bits.shape
    g = k // GROUP
    a = np.abs(bf16_to_f64(w_bits)).reshape(n * g, GROUP)
    lev, code, _ = warm_start(a)
    c = lloyd(a, lev, iters)
    return rne_fp16(c).reshape(n, g, N_MAG), code.reshape(n, g)


def group_sse(a, levels):
    """Squared error of magnitudes a [G, 32] against their nearest level
    (lowest on a tie), summed in element order."""
    a = np.asarray(a, dtype=np.float64)
    levels = np.asarray(levels, dtype=np.float64)
    j = np.argmin(np.abs(a[:, :, None] - levels[:, None, :]), axis=-1)
    wr = np.take_along_axis(levels, j, axis=-1)
    sse = np.zeros(a.shape[0])
    for i in range(a.shape[-1]):
        d = a[:, i] - wr[:, i]
        sse = sse + d * d
    return sse
