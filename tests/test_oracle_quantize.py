"""Pins of the oracle's absmax / scale / quantize steps (oracle/ref.py).

Page: DaisyChain-Train "Verification — why you can trust the numbers",
section "The verified INT8 units", step 1 (per-row / per-column scale
max(|row|)/127 floored at 1e-8, values to int8) and section "Hardware ground
truth (RDNA2 ISA audit)" (the quantizer x*inv + 0.5, floored).

Each pin compares the numpy oracle with something other than itself:
exact-rational evaluation (oracle/ieee32.py, integer arithmetic only),
closed forms on power-of-two scales, the error bound of the presk page's
"Integer weights" rule (|w - q*s| <= s/2 up to float rounding), and
discriminating sets on which a plausible wrong reading gives other bytes.
"""
from fractions import Fraction

import numpy as np
import pytest

from oracle import adversarial, ieee32 as I, ref

F32 = np.float32
U32 = np.uint32


def _b(x):
    return int(F32(x).view(U32))


def test_scale_special_cases():
    a = np.array([127.0, 0.0, -0.0, 127.0 * 2**-5, 127.0 * 2**7, 1.27e-6, 1e30], dtype=F32)
    s, inv = ref.scales_from_absmax(np.abs(a))
    assert s[0] == 1.0 and inv[0] == 1.0
    assert s[1].view(U32) == 0x322BCC77 and s[2].view(U32) == 0x322BCC77   # floor RN(1e-8)
    assert s[3] == 2.0**-5 and inv[3] == 2.0**5
    assert s[4] == 2.0**7 and inv[4] == 2.0**-7
    # 1.27e-6 / 127 ~ 1e-8: the max() picks whichever is larger, exactly
    q = I.div(_b(1.27e-6), _b(127.0))
    assert s[5].view(U32) == max(q, 0x322BCC77, key=lambda v: I.decode(v))
    assert np.isfinite(s[6]) and np.isfinite(inv[6])


def test_scale_and_reciprocal_match_exact_rational():
    rng = np.random.default_rng(21)
    a = np.abs(rng.standard_t(2, 20_000)).astype(F32)
    a[:2000] = np.abs(rng.standard_normal(2000) * 1e-7).astype(F32)   # near the floor
    s, inv = ref.scales_from_absmax(a)
    floor_b = 0x322BCC77
    for av, sv, iv in zip(a.view(U32).tolist(), s.view(U32).tolist(), inv.view(U32).tolist()):
        d = I.div(av, _b(127.0))
        want_s = d if I.decode(d) > I.decode(floor_b) else floor_b
        assert sv == want_s
        assert iv == I.div(_b(1.0), want_s)


def _exact_quantize(xb, invb):
    t = I.mul(xb, invb)
    u = I.add(t, _b(0.5))
    return I.floor_int(u)


def test_quantize_matches_exact_rational():
    rng = np.random.default_rng(22)
    X = rng.standard_t(2, (40, 500)).astype(F32)
    X[rng.random(X.shape) < 0.02] = F32(-0.0)
    X, _ = adversarial.plant_ties(X, "rows", rng, frac=0.05)
    X, _ = adversarial.plant_fma_splits(X, "rows", rng, per_line=4)
    Q, s = ref.quantize_rows(X)
    _, inv = ref.scales_from_absmax(ref.absmax_rows(X))
    for i in range(X.shape[0]):
        ib = int(inv[i].view(U32))
        for xb, q in zip(X[i].view(U32).tolist(), Q[i].tolist()):
            assert q == _exact_quantize(xb, ib)


def test_quantize_closed_forms_on_power_of_two_scales():
    """Line max 127*2^e gives s = 2^e and inv = 2^-e exactly; then
    x = k*2^e quantizes to k and x = (k+0.5)*2^e to k+1 (half rounds up)."""
    for e in (-20, -3, 0, 5, 30):
        unit = 2.0**e
        ks = np.arange(-127, 127)
        row_int = np.concatenate([[127.0], ks]) * unit
        row_tie = np.concatenate([[127.0], ks + 0.5]) * unit
        X = np.stack([row_int, row_tie]).astype(F32)
        Q, s = ref.quantize_rows(X)
        assert s[0] == unit and s[1] == unit
        assert Q[0, 0] == 127 and Q[1, 0] == 127
        assert np.array_equal(Q[0, 1:], ks)
        assert np.array_equal(Q[1, 1:], ks + 1)        # k + 0.5 -> k + 1, incl. -0.5 -> 0
    Q, _ = ref.quantize_rows(np.array([[127.0, -0.5, 0.5, -1.5, 1.5, -126.5]], dtype=F32))
    assert Q.tolist() == [[127, 0, 1, -1, 2, -126]]


def test_quantize_error_bound_and_range():
    """|x - q*s| <= s/2 (plus float rounding of x*inv), |q| <= 127 and the
    largest-magnitude entry of each line quantizes to +-127 unless floored."""
    rng = np.random.default_rng(23)
    X = rng.standard_t(2, (200, 300)).astype(F32)
    X[0] = 0
    X[1, :] = F32(-0.0)
    X[2, :] = F32(1e-12)
    Q, s = ref.quantize_rows(X)
    assert np.all(np.abs(Q.astype(int)) <= 127)
    err = np.abs(X.astype(np.float64) - Q.astype(np.float64) * s[:, None].astype(np.float64))
    assert np.all(err <= s[:, None].astype(np.float64) * 0.5 * (1 + 2.0**-20))
    a = np.max(np.abs(X), axis=1)
    live = a / 127 > 1e-8
    amax = np.argmax(np.abs(X), axis=1)
    qa = Q[np.arange(X.shape[0]), amax].astype(int)
    xa = X[np.arange(X.shape[0]), amax]
    assert np.all(np.abs(qa[live]) == 127)
    assert np.all(np.sign(qa[live]) == np.sign(xa[live]))
    assert np.all(Q[0] == 0) and np.all(Q[1] == 0) and np.all(Q[2] == 0)


def test_quantize_cols_is_rows_of_transpose():
    rng = np.random.default_rng(24)
    X = rng.standard_normal((37, 53)).astype(F32)
    Qt, s = ref.quantize_cols(X)
    assert Qt.shape == (53, 37)
    for j in range(53):
        col = X[:, j]
        sj = max(F32(np.max(np.abs(col))) / F32(127), F32(1e-8))
        assert s[j] == sj
        assert np.array_equal(Qt[j], np.floor(F32(col * (F32(1) / F32(sj))) + F32(0.5)).astype(np.int8))


# ---------------------------------------------------------------------------
# discriminating sets ("gate the gate"): a wrong reading must change bytes
# ---------------------------------------------------------------------------
def _quantize_with(X, inv_of, step):
    a = ref.absmax_rows(X)
    s = np.maximum(a / F32(127), F32(1e-8)).astype(F32)
    inv = inv_of(s, a)
    return step(X, inv[:, None])


def _two_round(X, inv):
    return np.floor(((X * inv).astype(F32) + F32(0.5)).astype(F32)).astype(np.int8)


def test_fused_quantize_is_caught():
    """fma(x, inv, 0.5) then floor differs from the two-rounding quantizer
    at |x*inv| next to 0.5 (k = 0 and k = -1), contrary to the page's claim."""
    rng = np.random.default_rng(25)
    X = rng.standard_normal((30, 64)).astype(F32)
    X, n = adversarial.plant_fma_splits(X, "rows", rng, per_line=3)
    assert n >= 30
    Q, _ = ref.quantize_rows(X)
    _, inv = ref.scales_from_absmax(ref.absmax_rows(X))
    diff_pos = diff_neg = 0
    for i in range(X.shape[0]):
        ib = int(inv[i].view(U32))
        for xb, q in zip(X[i].view(U32).tolist(), Q[i].tolist()):
            fused = I.floor_int(I.fma(xb, ib, _b(0.5)))
            if fused != q:
                assert (q, fused) in ((1, 0), (0, -1))
                diff_pos += q == 1
                diff_neg += q == 0
    assert diff_pos > 0 and diff_neg > 0


def test_ties_to_even_and_half_away_are_caught():
    rng = np.random.default_rng(26)
    X = rng.standard_normal((40, 128)).astype(F32)
    X, n = adversarial.plant_ties(X, "rows", rng, frac=0.1, ks=list(range(-127, 127)))
    assert n > 100
    Q, _ = ref.quantize_rows(X)
    _, inv = ref.scales_from_absmax(ref.absmax_rows(X))
    t = (X * inv[:, None]).astype(F32)
    rne = np.rint(t).astype(np.int8)                         # ties to even
    away = (np.sign(t) * np.floor(np.abs(t) + F32(0.5))).astype(np.int8)
    assert np.any(rne != Q) and np.any(away != Q)
    ties = (t - np.floor(t)) == F32(0.5)
    assert np.all(Q[ties] == (np.floor(t[ties]) + 1))           # half rounds up


def test_reciprocal_reading_is_caught():
    """inv = RN(1/s) vs the alternative RN(127/a) and a one-ulp-off reciprocal
    (what an approximate hardware reciprocal may give) change some int8."""
    rng = np.random.default_rng(27)
    X = rng.standard_normal((400, 256)).astype(F32)
    X, _ = adversarial.plant_ties(X, "rows", rng, frac=0.05)
    Q, _ = ref.quantize_rows(X)
    alt = _quantize_with(X, lambda s, a: np.where(a > 0, F32(127) / np.maximum(a, F32(1e-30)),
                                                  F32(1) / s).astype(F32), _two_round)
    ulp = _quantize_with(X, lambda s, a: np.nextafter(F32(1) / s, F32(np.inf)).astype(F32),
                         _two_round)
    assert np.any(alt != Q)
    assert np.any(ulp != Q)


def test_missing_floor_is_caught():
    X = np.zeros((2, 8), dtype=F32)
    X[1, :] = F32(1e-12)
    Q, s = ref.quantize_rows(X)
    assert s[0].view(U32) == 0x322BCC77
    with np.errstate(all="ignore"):
        s_nofloor = (np.max(np.abs(X), axis=1) / F32(127)).astype(F32)
        inv = F32(1) / s_nofloor
        q_bad = np.floor((X * inv[:, None]).astype(F32) + F32(0.5))
    assert not np.array_equal(np.nan_to_num(q_bad, nan=99), Q.astype(np.float64))
