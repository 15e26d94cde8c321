"""The five synthetic workloads this library is checked and measured on.

Shapes follow the [*batch, limb, coefficient] layout of FHElium "Eager, Compile,
and native execution" (section "Shared implementation and native path").  The
n = 2048 / 112-prime shape of the inner chain is the one the kestrel-llm
data-flow overview (lpnh.cn, sections 5 and 7) reports: 4 token positions x 2
ciphertext components, 112 primes, n = 2048, 8-byte residues (about 3.5 MB per
ciphertext).  The others are throughput shapes.

Prime rule (all workloads): the first `count` primes below 2^bits that are
1 mod 2n, in descending order.  For the key-switch, Q is the first 24 and P the
next 8 of the same list.  This module holds no arithmetic; primes come from
whichever side needs them (the library's own prime search, or the oracle's).
"""
from dataclasses import dataclass, field


@dataclass(frozen=True)
class Workload:
    name: str
    n: int
    bits: int
    limbs: int                 # Q limbs
    shape_a: tuple             # operand A, [..., limbs, n]
    seed_a: int
    seed_b: int = 0            # second operand (0 = none)
    special: int = 0           # P limbs (key-switch)
    dnum: int = 0              # key-switch digits
    galois: tuple = field(default_factory=tuple)

    @property
    def prime_count(self) -> int:
        return self.limbs + self.special


def galois_powers(n: int) -> tuple:
    """g = 5^(2^m) mod 2n for m = 0 .. log2(n)-1 (the k = 1, 2, 4, ... rotations)."""
    out, g = [], 5 % (2 * n)
    for _ in range(n.bit_length() - 1):
        out.append(g)
        g = g * g % (2 * n)
    return tuple(out)


POLYMUL = Workload("polymul_n2048_q4x30", n=2048, bits=30, limbs=4, shape_a=(4, 2048), seed_a=101, seed_b=102)
CHAIN = Workload("chain_n2048_q112x30_b4x2", n=2048, bits=30, limbs=112, shape_a=(4, 2, 112, 2048),
                 seed_a=201, seed_b=202)
BATCH = Workload("batch_n16384_q16x60_b64x2", n=16384, bits=60, limbs=16, shape_a=(64, 2, 16, 16384),
                 seed_a=301, seed_b=302)
RING = Workload("ring_n65536_q24x60_b8x2", n=65536, bits=60, limbs=24, shape_a=(8, 2, 24, 65536), seed_a=401,
                galois=galois_powers(65536))
KEYSWITCH = Workload("keyswitch_n65536_q24_p8_d3", n=65536, bits=60, limbs=24, shape_a=(1, 2, 24, 65536),
                     seed_a=501, seed_b=502, special=8, dnum=3, galois=(5,))

ALL = (POLYMUL, CHAIN, BATCH, RING, KEYSWITCH)
