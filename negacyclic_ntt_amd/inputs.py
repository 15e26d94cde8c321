"""Seeded synthetic inputs shared by the GPU tests, the benchmark and the oracle
tests.

This module holds no arithmetic of the transform, the products or the
key-switch: it only turns a seed into reproducible residues.

Generator: SplitMix64 (Steele, Lea, Flood, "Fast splittable pseudorandom number
generators", OOPSLA 2014).  The k-th output (k = 0, 1, ...) of a stream with
seed s is mix(s + (k + 1) * 0x9E3779B97F4A7C15 mod 2^64), where mix is the
published xor-shift/multiply finaliser.  Because the state is a counter, the
stream is evaluated vectorised.

Uniform residues in [0, q): take x = next() >> (64 - bitlen(q)) and reject
while x >= q.  A tensor [..., limbs, n] is filled in row-major order from one
stream; the n entries of row r use the prime of limb r % limbs.
"""
import numpy as np

GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)


def splitmix64(seed: int, start: int, count: int) -> np.ndarray:
    """Outputs start .. start+count-1 of the SplitMix64 stream `seed`."""
    with np.errstate(over="ignore"):
        k = np.arange(start + 1, start + count + 1, dtype=np.uint64)
        z = np.uint64(seed & 0xFFFFFFFFFFFFFFFF) + k * GAMMA
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
        return z ^ (z >> np.uint64(31))


class Stream:
    """A SplitMix64 stream with a position, for sequential rejection sampling."""

    def __init__(self, seed: int):
        self.seed = int(seed)
        self.pos = 0

    def next_block(self, count: int) -> np.ndarray:
        out = splitmix64(self.seed, self.pos, count)
        self.pos += count
        return out

    def uniform_row(self, q: int, n: int) -> np.ndarray:
        """n draws uniform in [0, q) by rejection (consumes exactly the draws used)."""
        q = int(q)
        shift = np.uint64(64 - q.bit_length())
        out = np.empty(n, dtype=np.uint64)
        filled = 0
        while filled < n:
            need = n - filled
            block = splitmix64(self.seed, self.pos, need + need // 64 + 16) >> shift
            ok = np.nonzero(block < np.uint64(q))[0]
            take = min(need, ok.size)
            if take:
                out[filled:filled + take] = block[ok[:take]]
                filled += take
                self.pos += int(ok[take - 1]) + 1
            else:
                self.pos += block.size
        return out


def uniform_residues(shape, primes, seed: int) -> np.ndarray:
    """uint64 tensor of `shape` ([..., limbs, n]) with row r uniform mod primes[r % limbs]."""
    shape = tuple(int(s) for s in shape)
    limbs, n = shape[-2], shape[-1]
    assert limbs == len(primes), (shape, len(primes))
    rows = int(np.prod(shape[:-1])) if len(shape) > 1 else 1
    out = np.empty((rows, n), dtype=np.uint64)
    st = Stream(seed)
    for r in range(rows):
        out[r] = st.uniform_row(primes[r % limbs], n)
    return out.reshape(shape)


def small_signed(count: int, bound: int, seed: int) -> np.ndarray:
    """int64 values in [-bound, bound] (bound small), e.g. ternary secrets (bound 1)."""
    span = 2 * int(bound) + 1
    st = Stream(seed)
    out = np.empty(count, dtype=np.int64)
    filled = 0
    lim = (1 << 64) - ((1 << 64) % span)  # unbiased: reject the top partial interval
    while filled < count:
        block = st.next_block(count - filled + 16)
        ok = block[block < np.uint64(lim)] if lim < (1 << 64) else block
        take = min(count - filled, ok.size)
        out[filled:filled + take] = (ok[:take] % np.uint64(span)).astype(np.int64) - int(bound)
        filled += take
    return out
