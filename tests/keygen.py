"""Test-side key material and decryption checks, built only from oracle calls.

A switching key from s_from to s over Q u P with dnum digits of alpha primes is,
for each digit j, the pair ( -a_j s + e_j + P T_j s_from, a_j ) in the NTT domain,
where T_j is 1 modulo the primes of digit j and 0 modulo the other primes of Q
(and P T_j vanishes modulo the primes of P).  A rotation key has s_from =
sigma_g(s); a relinearisation key has s_from = s^2.
"""
import numpy as np

import oracle as orc
from negacyclic_ntt_amd import inputs


def to_limbs(v_signed, primes) -> np.ndarray:
    return np.array([[int(x) % q for x in v_signed] for q in primes], dtype=np.uint64)


def pmul(a, b, primes) -> np.ndarray:
    """Negacyclic products per limb through the oracle's transform (a, b: [L, n])."""
    fa = orc.batch_ntt(a, primes)
    fb = orc.batch_ntt(b, primes)
    return orc.batch_ntt(orc.batch_pointwise(fa, fb, primes), primes, inverse=True)


def padd(a, b, primes) -> np.ndarray:
    q = np.array(primes, dtype=object)[:, None]
    return ((a.astype(object) + b.astype(object)) % q).astype(np.uint64)


def psub(a, b, primes) -> np.ndarray:
    q = np.array(primes, dtype=object)[:, None]
    return ((a.astype(object) - b.astype(object)) % q).astype(np.uint64)


def product(values) -> int:
    out = 1
    for v in values:
        out *= int(v)
    return out


def switching_key(s_from, s, qp, nq: int, dnum: int, seed: int, err_bound: int = 8) -> np.ndarray:
    """s_from, s: [nq + np, n] limbs.  Returns [dnum, 2, nq + np, n] (NTT domain)."""
    L, n = s.shape
    alpha = nq // dnum
    Pm = product(qp[nq:])
    ksk = np.zeros((dnum, 2, L, n), dtype=np.uint64)
    for j in range(dnum):
        a_j = inputs.uniform_residues((L, n), list(qp), seed + 2 * j)
        e_j = to_limbs(inputs.small_signed(n, err_bound, seed + 2 * j + 1), qp)
        b = psub(e_j, pmul(a_j, s, qp), qp)
        for l in range(j * alpha, (j + 1) * alpha):
            q = qp[l]
            b[l] = ((b[l].astype(object) + s_from[l].astype(object) * (Pm % q)) % q).astype(np.uint64)
        ksk[j, 0] = orc.batch_ntt(b, qp)
        ksk[j, 1] = orc.batch_ntt(a_j, qp)
    return ksk


def centered_crt_max(diff, primes, stride: int = 1) -> int:
    """max |v| over columns (every `stride`-th) of the centered CRT value of diff [L, n]."""
    M = product(primes)
    worst = 0
    for i in range(0, diff.shape[1], stride):
        v = orc.crt_int([int(diff[l][i]) for l in range(len(primes))], list(primes))
        if v > M // 2:
            v -= M
        worst = max(worst, abs(v))
    return worst


def centered_values(x, primes) -> list:
    """Centered CRT values of every column of x [L, n]."""
    M = product(primes)
    out = []
    for i in range(x.shape[1]):
        v = orc.crt_int([int(x[l][i]) for l in range(len(primes))], list(primes))
        out.append(v - M if v > M // 2 else v)
    return out
