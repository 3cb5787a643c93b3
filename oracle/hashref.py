"""Output hash of an f32 matrix: the definition, in numpy and in pure Python.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The DaisyChain-Train page "Verification — why you can trust the numbers"
compares replicas by hashing raw output bytes (its opening paragraph) and
has every device publish a probe hash of a seeded GEMM ("Layer 3: the kernel
probe").  The page names no hash function, so this library defines one.  The
choice is made so that a GPU can reduce it exactly in any order (modular
integer sums, no float), cheaply (one 32x32->64 multiply-add per element),
while every single-bit change and every swap of two unequal elements changes
the value:

    bits(i, j) = the 32-bit pattern of out[i, j]        (-0 and +0 differ)
    mix31(x)   = a bijection of [0, 2^31): xorshift / odd-multiply rounds
    r(i)       = 2 * mix31(i mod 2^31) + 1              odd, 32 bits, distinct
    c(j)       = fmix64((j + 0x9E3779B97F4A7C15) mod 2^64) OR 1   odd, 64 bits
    S          = sum_{i<M, j<N}  c(j) * r(i) * bits(i, j)       mod 2^64
    H          = fmix64(S XOR fmix64(M * 2^32 + N))

fmix64 is the public-domain 64-bit finalizer of MurmurHash3 (Austin Appleby):
three xorshift-33 steps around two multiplications by odd constants.

Why these properties hold: a flip of bit b of one element changes S by
+-2^b * r(i) * c(j), odd times 2^b with b < 32, never 0 mod 2^64.  Swapping
unequal x, y within column j between rows i1 != i2 changes S by
c(j) * (r(i1) - r(i2)) * (x - y); both differences are non-zero and below
2^32, so their 2-adic valuations sum to < 64 and the change is non-zero.
Within a row the change is r(i) * (c(j1) - c(j2)) * (x - y), non-zero unless
c(j1) - c(j2) is divisible by 2^33 or more (probability ~2^-32 per pair for
the pseudo-random column keys).

This is a checksum against honest faults (wrong kernels, drivers, modes), not
a cryptographic hash; the page's "What this does NOT protect against" section
likewise leaves malicious peers out of scope.
"""
import numpy as np

MASK64 = (1 << 64) - 1
MASK31 = (1 << 31) - 1
FMIX_C1 = 0xFF51AFD7ED558CCD
FMIX_C2 = 0xC4CEB9FE1A85EC53
COL_OFFSET = 0x9E3779B97F4A7C15
MIX31_M1 = 0x3B9C5A1D
MIX31_M2 = 0x2F6E8B35


# --------------------------------------------------------------------------
# pure Python (every step an arbitrary-precision integer op, then masked)
# --------------------------------------------------------------------------
def fmix64(k: int) -> int:
    k &= MASK64
    k ^= k >> 33
    k = (k * FMIX_C1) & MASK64
    k ^= k >> 33
    k = (k * FMIX_C2) & MASK64
    k ^= k >> 33
    return k


def mix31(x: int) -> int:
    x &= MASK31
    x ^= x >> 16
    x = (x * MIX31_M1) & MASK31
    x ^= x >> 13
    x = (x * MIX31_M2) & MASK31
    x ^= x >> 16
    return x


def row_key(i: int) -> int:
    return (mix31(i) << 1) | 1


def col_key(j: int) -> int:
    return fmix64((j + COL_OFFSET) & MASK64) | 1


def shape_key(m: int, n: int) -> int:
    return fmix64(((m << 32) | n) & MASK64)


def finalize(s: int, m: int, n: int) -> int:
    return fmix64((s & MASK64) ^ shape_key(m, n))


def output_hash_py(bits_rows, m: int, n: int) -> int:
    """Hash from a list of rows of 32-bit patterns, pure Python loops."""
    s = 0
    for i in range(m):
        ri = row_key(i)
        row = bits_rows[i]
        for j in range(n):
            s = (s + col_key(j) * ri * (row[j] & 0xFFFFFFFF)) & MASK64
    return finalize(s, m, n)


# --------------------------------------------------------------------------
# numpy (uint64 arithmetic wraps modulo 2^64)
# --------------------------------------------------------------------------
def _fmix64_np(k):
    k = k.astype(np.uint64, copy=True)
    k ^= k >> np.uint64(33)
    k *= np.uint64(FMIX_C1)
    k ^= k >> np.uint64(33)
    k *= np.uint64(FMIX_C2)
    k ^= k >> np.uint64(33)
    return k


def _mix31_np(x):
    m31 = np.uint64(MASK31)
    x = x.astype(np.uint64) & m31
    x ^= x >> np.uint64(16)
    x = (x * np.uint64(MIX31_M1)) & m31
    x ^= x >> np.uint64(13)
    x = (x * np.uint64(MIX31_M2)) & m31
    x ^= x >> np.uint64(16)
    return x


def row_keys_np(row0: int, count: int):
    i = np.arange(row0, row0 + count, dtype=np.uint64)
    return (_mix31_np(i) << np.uint64(1)) | np.uint64(1)


def col_keys_np(n: int):
    j = np.arange(n, dtype=np.uint64) + np.uint64(COL_OFFSET)
    return _fmix64_np(j) | np.uint64(1)


def partial_sum(block, row0: int = 0) -> int:
    """S restricted to the rows ``row0 .. row0+len(block)`` of the output.

    ``block`` is a float32 (rows, N) array.  S is a sum modulo 2^64, so the
    partial sums of any split of the rows add up (mod 2^64) to S.
    """
    block = np.ascontiguousarray(block, dtype=np.float32)
    rows, n = block.shape
    if rows == 0 or n == 0:
        return 0
    bits = block.view(np.uint32).astype(np.uint64)
    r = row_keys_np(row0, rows)
    t = (bits * r[:, None]).sum(axis=0, dtype=np.uint64)   # per column, mod 2^64
    c = col_keys_np(n)
    return int((t * c).sum(dtype=np.uint64))


def output_hash(C, row_chunk: int = 4096) -> int:
    """H of a float32 matrix (numpy), processed in row chunks to bound memory."""
    C = np.asarray(C)
    assert C.dtype == np.float32 and C.ndim == 2
    m, n = C.shape
    s = 0
    for r0 in range(0, m, row_chunk):
        s = (s + partial_sum(C[r0:r0 + row_chunk], r0)) & MASK64
    return finalize(s, m, n)


def step_hash(hashes) -> int:
    """Fold per-GEMM hashes H_0..H_{G-1}, in order, into one step hash.

    T_0 = fmix64(G); T_{g+1} = fmix64(T_g XOR H_g XOR (g + 1)).
    """
    hashes = list(hashes)
    t = fmix64(len(hashes))
    for g, h in enumerate(hashes):
        t = fmix64(t ^ (h & MASK64) ^ (g + 1))
    return t
