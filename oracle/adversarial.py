"""Searches for inputs that sit on the quantizer's rounding decisions.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

A bit-exact comparison proves nothing about a rounding rule unless some
input actually exercises it: on ordinary data, several competing readings of
the quantizer produce identical bytes.  These helpers construct inputs on
which those readings give different int8 values, so that a GPU matching the
oracle there has followed the reading this oracle takes (the DaisyChain-Train
page "Verification — why you can trust the numbers", section "Layer 1: exact
init gates", asks for such discriminating inputs):

* :func:`plant_ties` -- entries x with RN(x * inv) = k + 0.5 exactly, for
  scales that are not powers of two (half-up rounding vs ties-to-even vs
  half-away-from-zero disagree there);
* :func:`plant_fma_splits` -- entries with |x * inv| next to 0.5, where the
  two-rounding quantizer and a fused multiply-add one give different int8
  (the page's section "Hardware ground truth (RDNA2 ISA audit)" claims the
  two always agree; they do not at these points).

They modify a copy of X in place of non-maximal entries only, so the
line's absmax, scale and reciprocal stay what they were.
"""
import numpy as np

from . import ieee32 as I
from . import ref

F32 = np.float32


def _line_view(X, axis):
    """Lines along which scales are taken: rows (axis='rows') or columns."""
    return X if axis == "rows" else X.T


def _search(x0, inv, pred, span=16):
    """First x in {x0 +- j ulps, j <= span} (nearest first) with pred(x)."""
    cand = [x0]
    up = x0
    dn = x0
    for _ in range(span):
        up = np.nextafter(up, F32(np.inf), dtype=F32)
        dn = np.nextafter(dn, F32(-np.inf), dtype=F32)
        cand += [up, dn]
    for c in cand:
        if pred(F32(c)):
            return F32(c)
    return None


def plant_ties(X, axis, rng, frac=0.02, ks=None):
    """Copy of X with a fraction of entries moved onto exact ties.

    For each chosen entry of a line with scale s and inv = RN(1/s), pick k
    (uniform in -127..126 unless ``ks`` is given) and search x near
    RN((k + 0.5) * s) with RN(x * inv) == k + 0.5 and |x| < the line's
    absmax.  Returns (X', number of ties planted).
    """
    X = np.array(X, dtype=F32, copy=True)
    L = _line_view(X, axis)
    a = ref.absmax_rows(L)
    s, inv = ref.scales_from_absmax(a)
    planted = 0
    for li in range(L.shape[0]):
        if a[li] == 0:
            continue
        amax_pos = int(np.argmax(np.abs(L[li])))
        picks = np.flatnonzero(rng.random(L.shape[1]) < frac)
        for p in picks:
            if p == amax_pos:
                continue
            k = int(rng.choice(ks)) if ks is not None else int(rng.integers(-127, 127))
            target = F32(k + 0.5)
            x0 = F32(F32(target) * s[li])
            hit = _search(x0, inv[li],
                          lambda x: F32(x * inv[li]) == target and abs(x) < a[li])
            if hit is not None:
                L[li, p] = hit
                planted += 1
    return X, planted


def _fma_quantize_bits(x, inv):
    """floor(fma(x, inv, 0.5)) with one rounding (the contracted kernel)."""
    u = I.fma(int(F32(x).view(np.uint32)), int(F32(inv).view(np.uint32)),
              int(F32(0.5).view(np.uint32)))
    return I.floor_int(u)


def plant_fma_splits(X, axis, rng, per_line=2):
    """Copy of X with entries where the two-rounding quantizer and the fused
    one disagree: x * inv just below +0.5 (two roundings give 1, fused 0)
    or just below -0.5 (two roundings give 0, fused -1).

    Returns (X', number planted).
    """
    X = np.array(X, dtype=F32, copy=True)
    L = _line_view(X, axis)
    a = ref.absmax_rows(L)
    s, inv = ref.scales_from_absmax(a)
    planted = 0
    for li in range(L.shape[0]):
        if a[li] == 0 or L.shape[1] < 2:
            continue
        amax_pos = int(np.argmax(np.abs(L[li])))
        for _ in range(per_line):
            p = int(rng.integers(0, L.shape[1]))
            if p == amax_pos:
                continue
            sign = 1 if rng.random() < 0.5 else -1
            x0 = F32(F32(0.5 * sign) * s[li])

            def splits(x, li=li):
                if not abs(x) < a[li]:
                    return False
                two = int(np.floor(F32(F32(x * inv[li]) + F32(0.5))))
                return two != _fma_quantize_bits(x, inv[li])

            hit = _search(x0, inv[li], splits, span=24)
            if hit is not None:
                L[li, p] = hit
                planted += 1
    return X, planted
