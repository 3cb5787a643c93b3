"""The kernel probe's inputs and its expected hash.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The DaisyChain-Train page "Verification — why you can trust the numbers",
section "Layer 3: the kernel probe", has every device run the same seeded
int8 GEMM through its live kernel and publish the output hash.  The page does
not say how the seeded inputs are drawn; this reading (the library's
``i8g_probe_hash`` documents the same one) uses SplitMix64 as a counter-based
generator:

    output k of the generator seeded with s  =  mix(s + (k+1) * GAMMA)
    mix(z): z ^= z >> 30; z *= C1; z ^= z >> 27; z *= C2; z ^= z >> 31
    GAMMA = 0x9E3779B97F4A7C15, C1 = 0xBF58476D1CE4E5B9, C2 = 0x94D049BB133111EB

(Steele, Lea and Flood, "Fast splittable pseudorandom number generators",
OOPSLA 2014; the constants are those of Vigna's public-domain splitmix64.c).
A (M x K) takes outputs 0 .. MK-1 in row-major order and B (K x N) the next
KN outputs, also row-major; output z becomes the binary32 value
((z >> 40) - 2^23) / 2^21, an exact value in [-4, 4).  The probe is then the
method (``ref.blockscaled_gemm``, no ReLU) and the output hash
(``hashref.output_hash``).
"""
import numpy as np

from . import hashref, ref

MASK64 = (1 << 64) - 1
GAMMA = 0x9E3779B97F4A7C15
C1 = 0xBF58476D1CE4E5B9
C2 = 0x94D049BB133111EB


def splitmix64_py(seed: int, count: int, first: int = 0):
    """Outputs first .. first+count-1 of SplitMix64(seed), pure Python."""
    out = []
    for k in range(first, first + count):
        z = (seed + (k + 1) * GAMMA) & MASK64
        z = ((z ^ (z >> 30)) * C1) & MASK64
        z = ((z ^ (z >> 27)) * C2) & MASK64
        out.append(z ^ (z >> 31))
    return out


def splitmix64_np(seed: int, count: int, first: int = 0):
    """The same outputs as a numpy uint64 array (arithmetic mod 2^64)."""
    k = np.arange(first + 1, first + count + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = np.uint64(seed & MASK64) + k * np.uint64(GAMMA)
        z = (z ^ (z >> np.uint64(30))) * np.uint64(C1)
        z = (z ^ (z >> np.uint64(27))) * np.uint64(C2)
        return z ^ (z >> np.uint64(31))


def probe_values(z):
    """Generator outputs -> float32 inputs: ((z >> 40) - 2^23) / 2^21."""
    top = (np.asarray(z, dtype=np.uint64) >> np.uint64(40)).astype(np.int64) - (1 << 23)
    return (top.astype(np.float64) / 2.0 ** 21).astype(np.float32)   # exact


def probe_inputs(seed: int, M: int, N: int, K: int):
    A = probe_values(splitmix64_np(seed, M * K, 0)).reshape(M, K)
    B = probe_values(splitmix64_np(seed, K * N, M * K)).reshape(K, N)
    return A, B


def probe_hash(seed: int, M: int, N: int, K: int) -> int:
    """The probe's output hash H."""
    A, B = probe_inputs(seed, M, N, K)
    C = ref.blockscaled_gemm(A, B, relu=False)[0]
    return hashref.output_hash(C)
