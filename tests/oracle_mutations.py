"""Mutation check of the oracle's pins (CPU only, test infrastructure).

Plants one plausible mistake at a time -- a dropped term, a wrong sign, index or
operand, a skipped step -- in a copy of oracle/ntt_oracle.c, rebuilds the copy and
runs tests/test_oracle_pins.py against it.  Every mutant must make some pin fail.

    python tests/oracle_mutations.py            # all mutants (about 4 minutes)
    python tests/oracle_mutations.py 3 12       # by index
"""
import os
import shutil
import subprocess
import sys
import tempfile
import time

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
MUTANTS = [
 ("psi: largest root instead of smallest", "if (p < best) best = p;", "if (p > best) best = p;"),
 ("definition: even exponents", "uint64_t ek = 2 * bitrev(k, m) + 1, acc = 0;", "uint64_t ek = 2 * bitrev(k, m), acc = 0;"),
 ("forward butterfly: + instead of -", "a[j + t] = subm(u, v, q);", "a[j + t] = addm(u, v, q);"),
 ("forward: twiddle index off by one", "s = tab[m + i];", "s = tab[m + i - (i > 0)];"),
 ("inverse: no n^-1", "for (uint64_t j = 0; j < n; ++j) a[j] = mulm(a[j], n_inv, q);", "for (uint64_t j = 0; j < n; ++j) a[j] = a[j];"),
 ("inverse butterfly: v - u", "a[j + t] = mulm(subm(u, v, q), s, q);", "a[j + t] = mulm(subm(v, u, q), s, q);"),
 ("schoolbook: cyclic wrap", "acc[i + j - n] = subm(acc[i + j - n], p, q);", "acc[i + j - n] = addm(acc[i + j - n], p, q);"),
 ("automorph coeff: no sign", "out[e - n] = negm(in[i], q);", "out[e - n] = in[i];"),
 ("automorph ntt: no bit reversal", "out[k] = in[bitrev((e - 1) / 2, m)];", "out[k] = in[(e - 1) / 2];"),
 ("tensor: d1 uses a1 b1", "d1[i] = addm(mulm(a0[i], b1[i], q), mulm(a1[i], b0[i], q), q);", "d1[i] = addm(mulm(a0[i], b1[i], q), mulm(a1[i], b1[i], q), q);"),
 ("tensor: d2 = a1 b0", "d2[i] = mulm(a1[i], b1[i], q);", "d2[i] = mulm(a1[i], b0[i], q);"),
 ("pointwise: first prime for all limbs", "uint64_t off = (bi * limbs + l) * n, q = primes[l];\n      for (uint64_t e = 0; e < n; ++e) out[off + e] = mulm(", "uint64_t off = (bi * limbs + l) * n, q = primes[0];\n      for (uint64_t e = 0; e < n; ++e) out[off + e] = mulm("),
 ("moddown: r - acc", "uint64_t diff = subm(c->acc[(uint64_t)l * c->n + e], big_mod_u64(&r, q), q);", "uint64_t diff = subm(big_mod_u64(&r, q), c->acc[(uint64_t)l * c->n + e], q);"),
 ("moddown: no P^-1", "c->out[(uint64_t)l * c->n + e] = mulm(diff, c->p_inv[l], q);", "c->out[(uint64_t)l * c->n + e] = diff;"),
 ("keyswitch: un-rotated c0 added", "o[comp * plane + i] = comp == 0 ? addm(rot[i], md[i], qp[l]) : md[i];", "o[comp * plane + i] = comp == 0 ? addm(c[i], md[i], qp[l]) : md[i];"),
 ("keyswitch: key components swapped", "s = addm(s, mulm(ext[((uint64_t)j * nqp + t) * n + e], ksk[(((uint64_t)j * 2 + comp) * nqp + t) * n + e], q), q);", "s = addm(s, mulm(ext[((uint64_t)j * nqp + t) * n + e], ksk[(((uint64_t)j * 2 + 1 - comp) * nqp + t) * n + e], q), q);"),
 ("keyswitch: decomposes c0", "basis_extend_threads(rot + plane + (uint64_t)j * alpha * n, alpha,", "basis_extend_threads(rot + (uint64_t)j * alpha * n, alpha,"),
 ("keyswitch: digit primes shifted", "basis_extend_threads(rot + plane + (uint64_t)j * alpha * n, alpha, qp + (uint64_t)j * alpha,", "basis_extend_threads(rot + plane + (uint64_t)j * alpha * n, alpha, qp + (uint64_t)j * alpha + (j > 0),"),
 ("hoisted: c0 not rotated", "orc_automorph_coeff(c0 + (uint64_t)l * n, c0r + (uint64_t)l * n, n, qp[l], g);", "memcpy(c0r + (uint64_t)l * n, c0 + (uint64_t)l * n, n * 8);"),
 ("hoisted: digits permuted by g^-1 direction", "orc_automorph_ntt(ext + row * n, perm + row * n, n, g);", "orc_automorph_ntt(ext + row * n, perm + row * n, n, (2 * n - g) % (2 * n));"),
 ("relinearize: d1 added to component 0", "o[plane + i] = addm(o[plane + i], d1[i], qp[l]);", "o[i] = addm(o[i], d1[i], qp[l]);"),
 ("rescale: modes swapped", "big_set_u64(&half, mode ? ql / 2 : 0);", "big_set_u64(&half, mode ? 0 : ql / 2);"),
 ("rescale: half rounded up", "big_set_u64(&half, mode ? ql / 2 : 0);", "big_set_u64(&half, mode ? (ql + 1) / 2 : 0);"),
 ("modraise: source primes shifted", "orc_basis_extend(in + bi * from * n, from, primes, out + bi * to * n, to, primes, n);", "orc_basis_extend(in + bi * from * n, from, primes + 1, out + bi * to * n, to, primes, n);"),
 ("basis extend: first target prime for all", "c->out[(uint64_t)t * c->n + e] = big_mod_u64(&D, c->dst[t]);", "c->out[(uint64_t)t * c->n + e] = big_mod_u64(&D, c->dst[t > 0 ? t - 1 : 0]);"),
 ("crt: no final reduction", "while (big_cmp(X, &b->M) >= 0) big_sub(X, &b->M);", "if (big_cmp(X, &b->M) > 0) big_sub(X, &b->M);"),
 ("find_primes: skips the first", "if (orc_is_prime(c)) out[found++] = c;", "if (orc_is_prime(c) && c != (top / two_n) * two_n + 1) out[found++] = c;"),
 ("is_prime: one MR base", "for (int i = 0; i < 12; ++i) {\n    uint64_t x = orc_pow_mod(bases[i], d, n);", "for (int i = 0; i < 1; ++i) {\n    uint64_t x = orc_pow_mod(bases[i], d, n);"),
 ("batch ntt: wrong limb prime", "uint32_t l = (uint32_t)(u % c->limbs);", "uint32_t l = (uint32_t)((u + 1) % c->limbs);"),
 ("keyswitch: inner product misses last digit", "for (uint32_t j = 0; j < dnum; ++j)\n            s = addm(s, mulm(ext[", "for (uint32_t j = 0; j + 1 < dnum; ++j)\n            s = addm(s, mulm(ext["),
]


def run_mutant(idx: int) -> str:
    """'killed: <first failing pin>' or 'SURVIVED' for mutant idx."""
    name, old, new = MUTANTS[idx]
    src = open(os.path.join(ROOT, "oracle", "ntt_oracle.c")).read()
    if src.count(old) != 1:
        raise ValueError(f"mutant {idx} ({name}): pattern found {src.count(old)} times")
    with tempfile.TemporaryDirectory() as tmp:
        work = os.path.join(tmp, "repo")
        shutil.copytree(ROOT, work, ignore=shutil.ignore_patterns(
            ".git", "_work", "gpurun_out", "_build", "*.so", "__pycache__", "profiles"))
        open(os.path.join(work, "oracle", "ntt_oracle.c"), "w").write(src.replace(old, new))
        r = subprocess.run([sys.executable, "-m", "pytest", "tests/test_oracle_pins.py", "-x", "-q",
                            "-p", "no:cacheprovider"], cwd=work, capture_output=True, text=True, timeout=900)
    if r.returncode == 0:
        return "SURVIVED"
    failed = [l for l in r.stdout.splitlines() if l.startswith(("FAILED", "ERROR"))]
    return "killed: " + (failed[0] if failed else r.stdout.strip().splitlines()[-1])[:110]


def main(argv):
    picks = [int(a) for a in argv] or list(range(len(MUTANTS)))
    survivors = []
    for idx in picks:
        t = time.time()
        res = run_mutant(idx)
        print(f"{idx:2d} {MUTANTS[idx][0]:45s} {res} ({time.time() - t:.0f}s)", flush=True)
        if res == "SURVIVED":
            survivors.append(idx)
    print("survivors:", survivors)
    return 1 if survivors else 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
