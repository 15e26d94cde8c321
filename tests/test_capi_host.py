"""C-ABI checks that need no GPU: the library loads and exports every declared
symbol, the host-side prime search and plan tables agree with the oracle and with
closed forms, and argument validation rejects bad input before any launch."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle as orc
from negacyclic_ntt_amd import binding as B
from negacyclic_ntt_amd import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    text = open(os.path.join(ROOT, "include", "negacyclic_ntt.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert "ntt_forward" in names and "keyswitch" in names and len(names) >= 17
    L = B.lib()
    for name in names:
        assert hasattr(L, name), name


def test_status_strings():
    L = B.lib()
    for s in (0, -1, -2, -3, -4, -5):
        assert L.ntt_status_string(s).decode() != "unknown status"
    assert L.ntt_status_string(7).decode() == "unknown status"


@pytest.mark.parametrize("w", workloads.ALL, ids=lambda w: w.name)
def test_find_primes_matches_oracle(w):
    assert B.find_primes(w.bits, w.n, w.prime_count) == orc.find_primes(w.bits, 2 * w.n, w.prime_count)


def test_find_primes_edges():
    assert B.find_primes(62, 1 << 16, 2) == orc.find_primes(62, 1 << 17, 2)
    assert B.find_primes(4, 2, 2) == [13, 5]  # below 16, 1 mod 4
    with pytest.raises(B.NttError):
        B.find_primes(2, 4, 1)
    with pytest.raises(B.NttError):
        B.find_primes(5, 8, 5)  # too few exist
    with pytest.raises(B.NttError):
        B.find_primes(30, 3, 1)  # n not a power of two


def brv(x, bits):
    return int(format(x, f"0{bits}b")[::-1], 2) if bits else 0


@pytest.mark.parametrize("n,bits", [(16, 30), (2048, 30), (1024, 60), (4096, 62), (2, 20)])
def test_host_plan_tables(n, bits):
    primes = orc.find_primes(bits, 2 * n, 3)
    plan = B.Plan(n, primes, device=-1)
    logn = n.bit_length() - 1
    for l, q in enumerate(primes):
        t = plan.tables(l)
        psi = t["psi"]
        assert psi == orc.find_psi(q, n)
        ipsi = pow(psi, -1, q)
        ks = range(n) if n <= 64 else list(range(32)) + list(range(n - 32, n))
        for k in ks:
            w, iw = pow(psi, brv(k, logn), q), pow(ipsi, brv(k, logn), q)
            assert int(t["fwd"][k]) == w and int(t["inv"][k]) == iw
            assert int(t["fwd_shoup"][k]) == (w << 64) // q and int(t["inv_shoup"][k]) == (iw << 64) // q
    plan.destroy()


def test_explicit_psi_is_used():
    n, q = 8, orc.find_primes(30, 16, 1)[0]
    other = pow(orc.find_psi(q, n), 3, q)  # another primitive 2n-th root (odd power)
    assert pow(other, n, q) == q - 1 and other != orc.find_psi(q, n)
    plan = B.Plan(n, [q], device=-1, psi=[other])
    assert plan.tables(0)["psi"] == other
    assert int(plan.tables(0)["fwd"][1]) == pow(other, n // 2, q)  # brv(1) = n/2


def _create(n, primes, psi=None, device=-1):
    h = ctypes.c_void_p()
    arr = np.asarray(primes, dtype=np.uint64)
    pp = arr.ctypes.data_as(ctypes.POINTER(ctypes.c_uint64))
    psi_p = None
    if psi is not None:
        parr = np.asarray(psi, dtype=np.uint64)
        psi_p = parr.ctypes.data_as(ctypes.POINTER(ctypes.c_uint64))
    rc = B.lib().ntt_plan_create(ctypes.byref(h), n, pp, len(primes), psi_p, device)
    if rc == 0:
        B.lib().ntt_plan_destroy(h)
    return rc


def test_plan_validation():
    q = orc.find_primes(30, 4096, 2)
    assert _create(2048, q) == B.NTT_OK
    assert _create(2047, q) == B.NTT_EINVAL               # not a power of two
    assert _create(1 << 17, q) == B.NTT_EINVAL            # too large
    assert _create(1, q) == B.NTT_EINVAL
    assert _create(2048, [q[0], q[0]]) == B.NTT_EINVAL    # duplicate
    composite = next(c for c in range(4097, 1 << 20, 4096) if not orc.is_prime(c))
    assert _create(2048, [composite]) == B.NTT_EINVAL     # 1 mod 2n but composite
    assert _create(2048, [q[0] + 2]) == B.NTT_EINVAL      # not 1 mod 2n
    big = orc.find_primes(63, 4096, 1)[0]
    assert big >= 1 << 62 and _create(2048, [big]) == B.NTT_EINVAL  # beyond the lazy range
    assert _create(2048, []) == B.NTT_EINVAL
    assert _create(2048, q, psi=[3, 3]) == B.NTT_EINVAL   # not a root
    assert _create(2048, q, device=-2) == B.NTT_EINVAL
    assert B.lib().ntt_plan_create(None, 2048, None, 0, None, -1) == B.NTT_EINVAL


def test_compute_calls_reject_host_plans_and_bad_args():
    q = orc.find_primes(30, 4096, 2)
    plan = B.Plan(2048, q, device=-1)
    L = B.lib()
    fake = ctypes.c_void_p(0x1000)
    assert L.ntt_forward(plan.handle, fake, 1, 0, 2, None) == B.NTT_EDEVICE
    assert L.ntt_inverse(plan.handle, fake, 1, 0, 2, None) == B.NTT_EDEVICE
    assert L.poly_mul_ntt(plan.handle, fake, fake, fake, 1, 0, 2, None) == B.NTT_EDEVICE
    assert L.automorph(plan.handle, fake, fake, 5, 0, 1, 0, 2, None) == B.NTT_EDEVICE
    assert L.ntt_forward(None, fake, 1, 0, 2, None) == B.NTT_EINVAL
    # keyswitch plans need a device plan
    h = ctypes.c_void_p()
    assert L.keyswitch_plan_create(ctypes.byref(h), plan.handle, 1, 1, 1) == B.NTT_EDEVICE
    assert L.keyswitch_plan_create(ctypes.byref(h), None, 1, 1, 1) == B.NTT_EINVAL
    assert L.keyswitch_plan_create(None, plan.handle, 1, 1, 1) == B.NTT_EINVAL
    # rescale: host plan, then argument errors that need no device
    assert L.rescale(plan.handle, fake, fake, 0, 1, 0, 2, None) == B.NTT_EDEVICE
    assert L.rescale(None, fake, fake, 0, 1, 0, 2, None) == B.NTT_EINVAL
    # modraise plans need a device plan
    assert L.modraise_plan_create(ctypes.byref(h), plan.handle, 1, 2) == B.NTT_EDEVICE
    assert L.modraise_plan_create(ctypes.byref(h), None, 1, 2) == B.NTT_EINVAL
    assert L.modraise_plan_create(None, plan.handle, 1, 2) == B.NTT_EINVAL
    # every entry point taking a key-switch / modraise plan rejects a null plan
    g = (ctypes.c_uint64 * 1)(5)
    sz = ctypes.c_size_t()
    assert L.keyswitch(None, fake, fake, fake, 5, 1, fake, 1 << 30, None) == B.NTT_EINVAL
    assert L.relinearize(None, fake, fake, fake, 1, fake, 1 << 30, None) == B.NTT_EINVAL
    assert L.keyswitch_hoisted(None, fake, fake, fake, g, 1, 1, fake, 1 << 30, None) == B.NTT_EINVAL
    assert L.keyswitch_workspace_size(None, 1, ctypes.byref(sz)) == B.NTT_EINVAL
    assert L.keyswitch_hoisted_workspace_size(None, 1, 1, ctypes.byref(sz)) == B.NTT_EINVAL
    assert L.modraise(None, fake, fake, 1, None) == B.NTT_EINVAL
    L.keyswitch_plan_destroy(None)  # null is a no-op
    L.modraise_plan_destroy(None)


def test_plan_info():
    q = orc.find_primes(30, 4096, 3)
    plan = B.Plan(2048, q, device=-1)
    n, np_, dev = ctypes.c_uint32(), ctypes.c_uint32(), ctypes.c_int()
    assert B.lib().ntt_plan_info(plan.handle, ctypes.byref(n), ctypes.byref(np_), ctypes.byref(dev)) == 0
    assert (n.value, np_.value, dev.value) == (2048, 3, -1)
    v = ctypes.c_uint64()
    assert B.lib().ntt_plan_prime(plan.handle, 2, ctypes.byref(v)) == 0 and v.value == q[2]
    assert B.lib().ntt_plan_prime(plan.handle, 3, ctypes.byref(v)) == B.NTT_EINVAL


def test_launch_cap_setter():
    L = B.lib()
    assert L.ntt_set_max_launch_threads(1) == B.NTT_EINVAL
    assert L.ntt_set_max_launch_threads(255) == B.NTT_EINVAL
    assert L.ntt_set_max_launch_threads(256) == B.NTT_OK
    assert L.ntt_set_max_launch_threads(1 << 40) == B.NTT_OK  # clamped to the hardware cap
    assert L.ntt_set_max_launch_threads(0) == B.NTT_OK
