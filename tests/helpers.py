"""Shared helpers for the GPU parity tests."""
import functools
import sys

import numpy as np
import pytest

import oracle as orc
from negacyclic_ntt_amd import inputs


def require_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


@functools.lru_cache(maxsize=None)
def primes(bits: int, two_n: int, count: int) -> tuple:
    return tuple(orc.find_primes(bits, two_n, count))


def announce(*what):
    """Print (and flush) what a GPU step is about to run, so a crash names its case."""
    print("[gpu-case]", *what, flush=True)
    sys.stdout.flush()


def dev(arr: np.ndarray):
    from negacyclic_ntt_amd import binding as B
    return B.to_device(arr, "cuda:0")


def host(t) -> np.ndarray:
    from negacyclic_ntt_amd import binding as B
    import torch
    torch.cuda.synchronize()
    return B.to_host(t)


def assert_bits_equal(got: np.ndarray, want: np.ndarray, what: str):
    assert got.shape == want.shape, (what, got.shape, want.shape)
    if not np.array_equal(got, want):
        bad = np.argwhere(got != want)
        idx = tuple(bad[0])
        raise AssertionError(f"{what}: {len(bad)} mismatches, first at {idx}: got {got[idx]} want {want[idx]}")


def residues(shape, prime_list, seed):
    return inputs.uniform_residues(shape, list(prime_list), seed)
