"""GPU: keyswitch_noalloc (static device workspace) against keyswitch (caller
workspace), bit for bit, through the C ABI: two calls in a row, the second on a
smaller input (a smaller ring, two ciphertexts), then a call beyond the static
workspace, which must be refused with nothing launched."""
import ctypes

import numpy as np
import pytest

import oracle as orc
from negacyclic_ntt_amd import workloads
from tests.helpers import announce, assert_bits_equal, dev, host, primes, require_gpu, residues

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    require_gpu()
    from negacyclic_ntt_amd import binding
    return binding


def _call_noalloc(B, ks, out, ct, ksk, g, batch):
    V = ctypes.c_void_p
    return B.lib().keyswitch_noalloc(ks.handle, V(out.data_ptr()), V(ct.data_ptr()), V(ksk.data_ptr()), g, batch,
                                     None)


def test_noalloc_matches_keyswitch_twice_then_refuses_oversize(B):
    import torch
    w = workloads.KEYSWITCH
    cases = []
    # call 1: the full key-switch workload (n = 2^16, Q 24 + P 8, dnum 3, one ciphertext)
    qp = list(primes(60, 1 << 17, 32))
    cases.append((w.n, qp, 24, 8, 3, 1, 5, w.seed_a, w.seed_b))
    # call 2: a smaller input (n = 2^13, Q 12 + P 4, dnum 3, two ciphertexts)
    cases.append((1 << 13, qp[:16], 12, 4, 3, 2, 25, 7301, 7302))
    plans = []
    for i, (n, ps, nq, npr, dnum, batch, g, s_ct, s_k) in enumerate(cases):
        plan = B.Plan(n, ps, 0)
        ks = B.KeySwitchPlan(plan, nq, npr, dnum)
        plans.append((plan, ks))
        ct = dev(residues((batch, 2, nq, n), ps[:nq], s_ct))
        ksk = dev(residues((dnum, 2, nq + npr, n), ps[: nq + npr], s_k))
        want = torch.zeros_like(ct)
        B.keyswitch(ks, want, ct, ksk, g)
        got = torch.full_like(ct, -1)
        announce("keyswitch_noalloc call", i, n, nq, npr, dnum, batch, g)
        assert _call_noalloc(B, ks, got, ct, ksk, g, batch) == B.NTT_OK
        torch.cuda.synchronize()
        assert_bits_equal(host(got), host(want), f"keyswitch_noalloc call {i} vs keyswitch")
        if i == 1:  # the small case is also checked against the oracle
            want_o = orc.keyswitch(host(ct), host(ksk), g, ps[: nq + npr], nq, dnum)
            assert_bits_equal(host(got), want_o, "keyswitch_noalloc small case vs oracle")
    # two ciphertexts of the full workload need 160 MiB: refused before any launch
    plan, ks = plans[0]
    ct2 = torch.zeros((2, 2, 24, w.n), dtype=torch.int64, device="cuda:0")
    out2 = torch.full_like(ct2, 7)
    ksk = torch.zeros((3, 2, 32, w.n), dtype=torch.int64, device="cuda:0")
    torch.cuda.synchronize()
    announce("keyswitch_noalloc oversize refusal")
    assert _call_noalloc(B, ks, out2, ct2, ksk, 5, 2) == B.NTT_EUNSUPPORTED
    torch.cuda.synchronize()
    assert bool((out2 == 7).all())
    # argument errors are those of keyswitch
    assert _call_noalloc(B, ks, out2[:1], ct2[:1], ksk, 4, 1) == B.NTT_EINVAL  # even Galois element
