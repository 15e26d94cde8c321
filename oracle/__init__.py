"""ctypes wrapper around the plain-C oracle (``oracle/ntt_oracle.c``).

TEST INFRASTRUCTURE: a slow, obviously correct CPU reference for the GPU
library.  Only the test-suite, the smoke check and the benchmark's CPU-baseline
leg may import it.  Arrays are numpy ``uint64`` (C-contiguous); residues are
canonical.  Semantics of every function are documented in ``ntt_oracle.h``.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_lib = None
_U64P = ctypes.POINTER(ctypes.c_uint64)


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        L = ctypes.CDLL(_build.LIB)
        u64, u32, i32 = ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int
        sig = {
            "orc_is_prime": (i32, [u64]),
            "orc_find_primes": (u32, [u32, u64, u32, _U64P]),
            "orc_find_psi": (u64, [u64, u64]),
            "orc_pow_mod": (u64, [u64, u64, u64]),
            "orc_inv_mod": (u64, [u64, u64]),
            "orc_ntt_definition": (None, [_U64P, _U64P, u64, u64, u64]),
            "orc_intt_definition": (None, [_U64P, _U64P, u64, u64, u64]),
            "orc_ntt_forward": (None, [_U64P, u64, u64, u64]),
            "orc_ntt_inverse": (None, [_U64P, u64, u64, u64]),
            "orc_negacyclic_schoolbook": (None, [_U64P, _U64P, _U64P, u64, u64]),
            "orc_automorph_coeff": (None, [_U64P, _U64P, u64, u64, u64]),
            "orc_automorph_ntt": (None, [_U64P, _U64P, u64, u64]),
            "orc_batch_ntt": (i32, [_U64P, u64, u32, u64, _U64P, i32, i32]),
            "orc_batch_pointwise": (None, [_U64P, _U64P, _U64P, u64, u32, u64, _U64P]),
            "orc_batch_tensor": (None, [_U64P, _U64P, _U64P, u64, u32, u64, _U64P]),
            "orc_batch_automorph": (None, [_U64P, _U64P, u64, i32, u64, u32, u64, _U64P]),
            "orc_basis_extend": (None, [_U64P, u32, _U64P, _U64P, u32, _U64P, u64]),
            "orc_moddown": (None, [_U64P, _U64P, _U64P, u32, u32, u64]),
            "orc_keyswitch": (i32, [_U64P, _U64P, _U64P, u64, u64, u64, _U64P, u32, u32, u32, i32]),
            "orc_crt_words": (i32, [_U64P, _U64P, u32, _U64P, u32]),
            "orc_relinearize": (i32, [_U64P, _U64P, _U64P, u64, u64, _U64P, u32, u32, u32, i32]),
            "orc_rescale": (i32, [_U64P, _U64P, i32, u64, u32, u64, _U64P]),
            "orc_modraise": (i32, [_U64P, _U64P, u64, u32, u32, u64, _U64P]),
            "orc_keyswitch_hoisted": (i32, [_U64P, _U64P, _U64P, _U64P, u32, u64, u64, _U64P, u32, u32, u32, i32]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _p(a: np.ndarray):
    assert a.dtype == np.uint64 and a.flags["C_CONTIGUOUS"], (a.dtype, a.flags)
    return a.ctypes.data_as(_U64P)


def _u64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.uint64))


def default_threads() -> int:
    return max(1, len(os.sched_getaffinity(0)))


# ---- number theory --------------------------------------------------------

def is_prime(n: int) -> bool:
    return bool(lib().orc_is_prime(n))


def find_primes(bits: int, two_n: int, count: int) -> list:
    out = np.zeros(max(count, 1), dtype=np.uint64)
    got = lib().orc_find_primes(bits, two_n, count, _p(out))
    if got != count:
        raise ValueError(f"only {got} of {count} primes below 2^{bits} with q = 1 mod {two_n}")
    return [int(x) for x in out[:count]]


def find_psi(q: int, n: int) -> int:
    return int(lib().orc_find_psi(q, n))


def pow_mod(b: int, e: int, q: int) -> int:
    return int(lib().orc_pow_mod(b, e, q))


# ---- single-limb ----------------------------------------------------------

def ntt_definition(a, q: int, psi: int) -> np.ndarray:
    a = _u64(a)
    out = np.zeros_like(a)
    lib().orc_ntt_definition(_p(a), _p(out), a.size, q, psi)
    return out


def intt_definition(a, q: int, psi: int) -> np.ndarray:
    a = _u64(a)
    out = np.zeros_like(a)
    lib().orc_intt_definition(_p(a), _p(out), a.size, q, psi)
    return out


def ntt_forward(a, q: int, psi: int) -> np.ndarray:
    a = _u64(a).copy()
    lib().orc_ntt_forward(_p(a), a.size, q, psi)
    return a


def ntt_inverse(a, q: int, psi: int) -> np.ndarray:
    a = _u64(a).copy()
    lib().orc_ntt_inverse(_p(a), a.size, q, psi)
    return a


def schoolbook(a, b, q: int) -> np.ndarray:
    a, b = _u64(a), _u64(b)
    out = np.zeros_like(a)
    lib().orc_negacyclic_schoolbook(_p(a), _p(b), _p(out), a.size, q)
    return out


def automorph_coeff(a, g: int, q: int) -> np.ndarray:
    a = _u64(a)
    out = np.zeros_like(a)
    lib().orc_automorph_coeff(_p(a), _p(out), a.size, q, g)
    return out


def automorph_ntt(a, g: int) -> np.ndarray:
    a = _u64(a)
    out = np.zeros_like(a)
    lib().orc_automorph_ntt(_p(a), _p(out), a.size, g)
    return out


# ---- batched [..., limbs, n] ------------------------------------------------

def _shape_bln(x: np.ndarray, primes):
    n = x.shape[-1]
    limbs = x.shape[-2]
    assert limbs == len(primes), (x.shape, len(primes))
    batch = x.size // (limbs * n) if x.size else 0
    return batch, limbs, n


def batch_ntt(x, primes, inverse: bool = False, threads: int = 0) -> np.ndarray:
    x = _u64(x).copy()
    pr = _u64(primes)
    batch, limbs, n = _shape_bln(x, primes)
    rc = lib().orc_batch_ntt(_p(x), batch, limbs, n, _p(pr), 1 if inverse else 0, threads or default_threads())
    if rc:
        raise ValueError("a prime has no primitive 2n-th root")
    return x


def batch_pointwise(a, b, primes) -> np.ndarray:
    a, b = _u64(a), _u64(b)
    assert a.shape == b.shape
    out = np.zeros_like(a)
    batch, limbs, n = _shape_bln(a, primes)
    lib().orc_batch_pointwise(_p(out), _p(a), _p(b), batch, limbs, n, _p(_u64(primes)))
    return out


def batch_tensor(a, b, primes) -> np.ndarray:
    """a, b: [..., 2, limbs, n] -> [..., 3, limbs, n]."""
    a, b = _u64(a), _u64(b)
    assert a.shape == b.shape and a.shape[-3] == 2
    n, limbs = a.shape[-1], a.shape[-2]
    batch = a.size // (2 * limbs * n) if a.size else 0
    out = np.zeros(a.shape[:-3] + (3, limbs, n), dtype=np.uint64)
    lib().orc_batch_tensor(_p(out), _p(a), _p(b), batch, limbs, n, _p(_u64(primes)))
    return out


def ct_tensor_coeff(a, b, primes, threads: int = 0) -> np.ndarray:
    """Ciphertext product in the coefficient domain (the ciphertext "mul" of the
    kestrel-llm overview's CKKS layer, section 3): a, b [..., 2, limbs, n] ->
    [..., 3, limbs, n] with the negacyclic products d0 = a0 b0, d1 = a0 b1 + a1 b0,
    d2 = a1 b1 mod q.  The oracle's forward NTT, slot products and inverse NTT in
    the order the definition gives (convolution theorem), each step pinned."""
    a, b = _u64(a), _u64(b)
    assert a.shape == b.shape and a.shape[-3] == 2
    fa = batch_ntt(a, primes, threads=threads)
    fb = batch_ntt(b, primes, threads=threads)
    return batch_ntt(batch_tensor(fa, fb, primes), primes, inverse=True, threads=threads)


def batch_automorph(x, g: int, domain: int, primes) -> np.ndarray:
    x = _u64(x)
    out = np.zeros_like(x)
    batch, limbs, n = _shape_bln(x, primes)
    lib().orc_batch_automorph(_p(out), _p(x), g, domain, batch, limbs, n, _p(_u64(primes)))
    return out


# ---- key-switch pieces ------------------------------------------------------

def basis_extend(x, src, dst) -> np.ndarray:
    x = _u64(x)
    k, n = x.shape
    assert k == len(src)
    out = np.zeros((len(dst), n), dtype=np.uint64)
    lib().orc_basis_extend(_p(x), k, _p(_u64(src)), _p(out), len(dst), _p(_u64(dst)), n)
    return out


def moddown(acc, qp, nq: int) -> np.ndarray:
    acc = _u64(acc)
    k, n = acc.shape
    np_ = k - nq
    assert k == len(qp)
    out = np.zeros((nq, n), dtype=np.uint64)
    lib().orc_moddown(_p(acc), _p(out), _p(_u64(qp)), nq, np_, n)
    return out


def keyswitch(ct, ksk, g: int, qp, nq: int, dnum: int, threads: int = 0) -> np.ndarray:
    """ct: [batch, 2, nq, n] (or [2, nq, n]); ksk: [dnum, 2, nq+np, n]."""
    ct, ksk = _u64(ct), _u64(ksk)
    n = ct.shape[-1]
    assert ct.shape[-2] == nq and ct.shape[-3] == 2
    batch = ct.size // (2 * nq * n)
    np_ = len(qp) - nq
    assert ksk.shape == (dnum, 2, nq + np_, n), ksk.shape
    out = np.zeros_like(ct)
    rc = lib().orc_keyswitch(_p(out), _p(ct), _p(ksk), g, batch, n, _p(_u64(qp)), nq, np_, dnum,
                             threads or default_threads())
    if rc:
        raise ValueError("bad key-switch arguments")
    return out


def keyswitch_hoisted(ct, ksk, gs, qp, nq: int, dnum: int, threads: int = 0) -> np.ndarray:
    """ct: [batch, 2, nq, n]; ksk: [R, dnum, 2, nq+np, n]; gs: R elements -> [R, batch, 2, nq, n]."""
    ct, ksk = _u64(ct), _u64(ksk)
    n = ct.shape[-1]
    assert ct.ndim == 4 and ct.shape[1:3] == (2, nq)
    batch = ct.shape[0]
    R = len(gs)
    np_ = len(qp) - nq
    assert ksk.shape == (R, dnum, 2, nq + np_, n), ksk.shape
    out = np.zeros((R, batch, 2, nq, n), dtype=np.uint64)
    rc = lib().orc_keyswitch_hoisted(_p(out), _p(ct), _p(ksk), _p(_u64(gs)), R, batch, n, _p(_u64(qp)), nq, np_,
                                     dnum, threads or default_threads())
    if rc:
        raise ValueError("bad hoisted key-switch arguments")
    return out


def crt_int(residues, moduli) -> int:
    """Exact CRT value (Python int) of residues modulo distinct primes."""
    x, m = _u64(residues), _u64(moduli)
    words = len(moduli) + 2
    out = np.zeros(words, dtype=np.uint64)
    got = lib().orc_crt_words(_p(x), _p(m), len(moduli), _p(out), words)
    if got < 0:
        raise ValueError("CRT value does not fit")
    return sum(int(w) << (64 * i) for i, w in enumerate(out))


def relinearize(d, rlk, qp, nq: int, dnum: int, threads: int = 0) -> np.ndarray:
    """d: [batch, 3, nq, n] (or [3, nq, n]); rlk: [dnum, 2, nq+np, n] -> [..., 2, nq, n]."""
    d, rlk = _u64(d), _u64(rlk)
    n = d.shape[-1]
    assert d.shape[-2] == nq and d.shape[-3] == 3
    batch = d.size // (3 * nq * n)
    np_ = len(qp) - nq
    assert rlk.shape == (dnum, 2, nq + np_, n), rlk.shape
    out = np.zeros(d.shape[:-3] + (2, nq, n), dtype=np.uint64)
    rc = lib().orc_relinearize(_p(out), _p(d), _p(rlk), batch, n, _p(_u64(qp)), nq, np_, dnum,
                               threads or default_threads())
    if rc:
        raise ValueError("bad relinearisation arguments")
    return out


def rescale(x, primes, mode: int) -> np.ndarray:
    """x: [..., limbs, n] -> [..., limbs - 1, n]; mode 0 truncating, 1 nearest."""
    x = _u64(x)
    n, limbs = x.shape[-1], x.shape[-2]
    assert limbs == len(primes) and limbs >= 2
    batch = x.size // (limbs * n)
    out = np.zeros(x.shape[:-2] + (limbs - 1, n), dtype=np.uint64)
    rc = lib().orc_rescale(_p(out), _p(x), mode, batch, limbs, n, _p(_u64(primes)))
    if rc:
        raise ValueError("bad rescale arguments")
    return out


def modraise(x, primes_to, from_limbs: int) -> np.ndarray:
    """x: [..., from_limbs, n] over primes_to[:from_limbs] -> [..., len(primes_to), n]."""
    x = _u64(x)
    n = x.shape[-1]
    assert x.shape[-2] == from_limbs
    to = len(primes_to)
    batch = x.size // (from_limbs * n)
    out = np.zeros(x.shape[:-2] + (to, n), dtype=np.uint64)
    rc = lib().orc_modraise(_p(out), _p(x), batch, from_limbs, to, n, _p(_u64(primes_to)))
    if rc:
        raise ValueError("bad modraise arguments")
    return out
