"""Workload definitions and seeded f32 input generators.

Every generator draws from numpy's PCG64 seeded by
SeedSequence([BASE_SEED, workload, index, ...]) so that the GPU path and the
oracle see the same bytes.  Normal variates are drawn directly in float32.
"N(0, sigma)" means standard deviation sigma (0.02 is GPT-2's weight-init
standard deviation).

Workloads (GPT-2 small: d=768, MLP 3072, vocab 50304, batch 8 x seq 1024,
so M = 8192 token rows):

  w1  single GEMM, M=N=K=256, A and B ~ N(0,1), no ReLU
  w2  MLP up-projection 8192x768 @ 768x3072 (ReLU), then the down-projection
      8192x3072 @ 3072x768 on the up-projection's output
  w3  LM head forward 8192x768 @ 768x50304, and its weight gradient
      768x8192 @ 8192x50304 (upstream gradient ~ N(0,1e-4))
  w4  200 ragged/adversarial GEMMs (see ``adversarial_case``)
  w5  the 147 GEMMs of one GPT-2-small training step (see ``step_gemms``)
"""
import hashlib
from dataclasses import dataclass

import numpy as np

BASE_SEED = 20261202
TOKENS = 8192            # batch 8 x sequence 1024
D_MODEL = 768
D_MLP = 3072
VOCAB = 50304
N_LAYERS = 12
STD_ACT = 1.0
STD_WEIGHT = 0.02
STD_GRAD = 1e-4


def rng_for(*key) -> np.random.Generator:
    """PCG64 generator for a key path (workload, index, tensor, ...)."""
    return np.random.Generator(
        np.random.PCG64(np.random.SeedSequence([BASE_SEED, *[int(k) for k in key]])))


def normal(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def sha256(arr: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(arr).tobytes()).hexdigest()


# --------------------------------------------------------------------------
# w1 .. w3: plain Gaussian workloads
# --------------------------------------------------------------------------
def w1_inputs():
    r = rng_for(1, 0)
    return normal(r, (256, 256), STD_ACT), normal(r, (256, 256), STD_ACT)


def w2_inputs():
    """(X 8192x768 ~N(0,1), W_up 768x3072 ~N(0,.02), W_down 3072x768 ~N(0,.02))."""
    return (normal(rng_for(2, 0), (TOKENS, D_MODEL), STD_ACT),
            normal(rng_for(2, 1), (D_MODEL, D_MLP), STD_WEIGHT),
            normal(rng_for(2, 2), (D_MLP, D_MODEL), STD_WEIGHT))


def w3_fwd_inputs():
    """(X 8192x768 ~N(0,1), W_head 768x50304 ~N(0,.02))."""
    return (normal(rng_for(3, 0), (TOKENS, D_MODEL), STD_ACT),
            normal(rng_for(3, 1), (D_MODEL, VOCAB), STD_WEIGHT))


def w3_wgrad_inputs():
    """(X 8192x768 ~N(0,1), dY 8192x50304 ~N(0,1e-4)); the GEMM is X^T @ dY."""
    return (normal(rng_for(3, 0), (TOKENS, D_MODEL), STD_ACT),
            normal(rng_for(3, 2), (TOKENS, VOCAB), STD_GRAD))


# --------------------------------------------------------------------------
# w4: ragged and adversarial sweep
# --------------------------------------------------------------------------
W4_CASES = 200


def _ragged_dim(rng) -> int:
    while True:
        d = int(rng.integers(1, 1001))
        if d % 16:
            return d


def _binade_edges(rng, x: np.ndarray, frac: float) -> None:
    """Replace a fraction of non-zero entries by +-2^e or +-pred(2^e), where
    2^e <= |x| < 2^(e+1), so that no magnitude grows."""
    flat = x.reshape(-1)
    nz = np.flatnonzero(flat != 0)
    if nz.size == 0:
        return
    pick = nz[rng.random(nz.size) < frac]
    if pick.size == 0:
        return
    v = flat[pick]
    _, ex = np.frexp(v)                                  # |v| = m * 2^ex, m in [0.5, 1)
    p2 = np.ldexp(np.float32(1.0), ex - 1).astype(np.float32)
    below = np.nextafter(p2, np.float32(0)).astype(np.float32)
    use_pred = rng.random(pick.size) < 0.5
    mag = np.where(use_pred, below, p2).astype(np.float32)
    flat[pick] = np.where(v < 0, -mag, mag).astype(np.float32)


def _tie_lines(rng, x: np.ndarray, axis: int, frac_lines: float, frac_ties: float) -> None:
    """Rebuild some lines (rows if axis=1 reduces over columns, i.e. a row of
    A; columns for B) so that their absmax is exactly 127 * 2^e, and fill
    them with values (k + 0.5) * 2^e (exact ties) and k * 2^e plus random
    fractions, |k + f| < 127.  Only construction: nothing is divided,
    rounded or quantized here."""
    lines = x.shape[0] if axis == 1 else x.shape[1]
    length = x.shape[1] if axis == 1 else x.shape[0]
    for li in np.flatnonzero(rng.random(lines) < frac_lines):
        e = int(rng.integers(-12, 9))
        unit = np.float32(2.0 ** e)
        k = rng.integers(-127, 127, size=length)          # -127 .. 126
        f = rng.integers(0, 256, size=length) / 256.0     # 8-bit fractions: exact
        tie = rng.random(length) < max(frac_ties, 0.3)
        val = np.where(tie, k + 0.5, k + f)
        val = np.clip(val, -126.5, 126.5)
        line = (val * float(unit)).astype(np.float32)
        p0 = int(rng.integers(0, length))
        line[p0] = np.float32(127.0) * unit * (1 if rng.random() < 0.5 else -1)
        if axis == 1:
            x[li, :] = line
        else:
            x[:, li] = line


@dataclass
class AdversarialCase:
    index: int
    A: np.ndarray      # M x K f32
    B: np.ndarray      # K x N f32
    relu: bool

    @property
    def shape(self):
        return self.A.shape[0], self.B.shape[1], self.A.shape[1]


def adversarial_case(c: int) -> AdversarialCase:
    """Case c of w4.

    M, N, K uniform in [1, 1000], resampled while a multiple of 16; values
    Student-t with 2 degrees of freedom; 5% of the rows of A and of the
    columns of B all zero; 2% of non-zero entries moved to binade edges;
    ~10% of rows of A / columns of B rebuilt with a power-of-two scale and
    exact k + 0.5 ties (k from -127 to 126, so k = -1 and k = 0 included);
    1% of entries -0.0; ReLU on for odd c.  Ties for scales that are not
    powers of two are planted by the tests with the oracle's help.
    """
    r = rng_for(4, c)
    M, N, K = _ragged_dim(r), _ragged_dim(r), _ragged_dim(r)
    A = r.standard_t(2, size=(M, K)).astype(np.float32)
    B = r.standard_t(2, size=(K, N)).astype(np.float32)
    _binade_edges(r, A, 0.02)
    _binade_edges(r, B, 0.02)
    _tie_lines(r, A, axis=1, frac_lines=0.10, frac_ties=0.02)
    _tie_lines(r, B, axis=0, frac_lines=0.10, frac_ties=0.02)
    A[r.random(M) < 0.05, :] = 0.0
    B[:, r.random(N) < 0.05] = 0.0
    A[r.random((M, K)) < 0.01] = np.float32(-0.0)
    B[r.random((K, N)) < 0.01] = np.float32(-0.0)
    return AdversarialCase(c, A, B, relu=bool(c & 1))


# --------------------------------------------------------------------------
# w5: the GEMMs of one GPT-2-small training step
# --------------------------------------------------------------------------
@dataclass(frozen=True)
class StepGemm:
    index: int          # position in the step (0..146)
    linear: str         # e.g. "L3.fc", "head"
    kind: str           # "fwd" | "dgrad" | "wgrad"
    d_in: int
    d_out: int

    @property
    def mnk(self):
        if self.kind == "fwd":
            return TOKENS, self.d_out, self.d_in
        if self.kind == "dgrad":
            return TOKENS, self.d_in, self.d_out
        return self.d_in, self.d_out, TOKENS

    @property
    def operands(self):
        """How each operand is quantized, as (A's source, A's mode, B's source,
        B's mode); mode 'rows' = per-row scales, 'cols' = per-column scales."""
        if self.kind == "fwd":
            return ("X", "rows", "W", "cols")       # X @ W
        if self.kind == "dgrad":
            return ("dY", "rows", "W", "rows")      # dY @ W^T
        return ("X", "cols", "dY", "cols")          # X^T @ dY


LINEARS = (("qkv", D_MODEL, 3 * D_MODEL), ("attn_out", D_MODEL, D_MODEL),
           ("fc", D_MODEL, D_MLP), ("proj", D_MLP, D_MODEL))


def step_gemms():
    """The 147 GEMMs in step order: 12 layers x 4 forward, LM-head forward,
    LM-head dgrad and wgrad, then layers 11..0 with linears proj, fc,
    attn_out, qkv, each dgrad then wgrad."""
    out = []
    for layer in range(N_LAYERS):
        for name, di, do in LINEARS:
            out.append(StepGemm(len(out), f"L{layer}.{name}", "fwd", di, do))
    out.append(StepGemm(len(out), "head", "fwd", D_MODEL, VOCAB))
    out.append(StepGemm(len(out), "head", "dgrad", D_MODEL, VOCAB))
    out.append(StepGemm(len(out), "head", "wgrad", D_MODEL, VOCAB))
    for layer in reversed(range(N_LAYERS)):
        for name, di, do in reversed(LINEARS):
            out.append(StepGemm(len(out), f"L{layer}.{name}", "dgrad", di, do))
            out.append(StepGemm(len(out), f"L{layer}.{name}", "wgrad", di, do))
    assert len(out) == 147
    return out


def _linear_id(linear: str) -> int:
    if linear == "head":
        return 1000
    layer, name = linear[1:].split(".")
    return int(layer) * 10 + [n for n, _, _ in LINEARS].index(name)


def step_tensor(linear: str, which: str, d_in: int, d_out: int) -> np.ndarray:
    """One of the f32 tensors of a linear: 'X' (8192 x d_in, N(0,1)),
    'W' (d_in x d_out, N(0,.02)) or 'dY' (8192 x d_out, N(0,1e-4))."""
    lid = _linear_id(linear)
    if which == "X":
        return normal(rng_for(5, lid, 0), (TOKENS, d_in), STD_ACT)
    if which == "W":
        return normal(rng_for(5, lid, 1), (d_in, d_out), STD_WEIGHT)
    if which == "dY":
        return normal(rng_for(5, lid, 2), (TOKENS, d_out), STD_GRAD)
    raise ValueError(which)


def step_ops() -> float:
    """Total int8 operations (2MNK) of the 147 step GEMMs."""
    return float(sum(2.0 * m * n * k for m, n, k in (g.mnk for g in step_gemms())))
