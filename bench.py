#!/usr/bin/env python3
"""Throughput benchmark on one MI355X.

One step = one pass of every hot-path operation over one batch of the
large-ring workload (n = 2^16, 24 primes of 60 bits, 8 ciphertexts = 16
polynomials, tensor [8][2][24][65536], seeded uniform residues):
  1. forward NTT of A                                  (384 limb-NTTs)
  2. pointwise product  C = A_hat * B_hat              (NTT domain)
  3. ciphertext tensor product D = (A_hat, B_hat)      ([8][3][24][n])
  4. inverse NTT of C                                  (384 limb-INTTs)
  5. coefficient-domain automorphism E = sigma_g(B'), g = 5^(2^(s mod 16)) mod 2n, of
     the B operand of another input set (not written or read for a whole step)
  6. one rotation key-switch of a 1-ciphertext batch (Q = 24, P = 8, dnum = 3)
     with the same g (96 forward + 64 inverse limb transforms inside), over ten
     distinct ciphertexts and keys in turn
`value` is limb-NTTs per second over whole steps (forward and inverse
transforms, those inside the key-switch included).  Inputs are resident in HBM
before timing; the timed steps rotate over enough distinct buffers and keys
(> 2 GB) that the 256 MB Infinity Cache cannot hold them.

`roofline` is the forward NTT's algorithmic HBM rate against the 8 TB/s peak;
`alu_issue` gives the same call against the 32-bit multiply issue peak, with the
clock that peak assumes and the clock sampled during the timed steps.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
# Integer ALU peak: 256 CUs x 64 lanes x 2.4 GHz of full-rate 32-bit multiply issue
# (v_mul_lo_u32 / v_mul_hi_u32 / v_mad_u64_u32 all issue at full rate on gfx950).
MUL32_PEAK_TOPS = 256 * 64 * 2.4e9 / 1e12
# A lazy 64-bit Shoup butterfly needs at least 10 32x32-bit multiplies: 4 for the
# high half of y * w', 3 for the low half of y * w, 3 for the low half of Q * q.
MUL32_PER_BUTTERFLY = 10
CALIBRATION_COPY_BYTES = 256 << 20
PROFILES = os.path.join(ROOT, "profiles")


def code_text(source: str) -> str:
    """C/HIP source with comments removed and whitespace collapsed: two sources
    with the same code text compile to the same kernels."""
    import re
    source = re.sub(r"/\*.*?\*/", " ", source, flags=re.S)
    source = re.sub(r"//[^\n]*", " ", source)
    return " ".join(source.split())


def kernel_sources_digest(read=None):
    """sha256/16 over the code text of modarith.h + ntt_passes.h + ntt.hip (comments
    excluded, so a comment edit does not invalidate counters taken on the same kernels)."""
    import hashlib
    if read is None:
        def read(name):
            with open(os.path.join(ROOT, "negacyclic_ntt_amd", "csrc", name)) as fh:
                return fh.read()
    h = hashlib.sha256()
    for f in ("modarith.h", "ntt_passes.h", "ntt.hip"):
        h.update(code_text(read(f)).encode())
    return h.hexdigest()[:16]


def recorded_fields(name):
    """The `- key: value` fields of a committed counter summary under profiles/, if it
    was taken on the current kernel sources (its kernel_sources_sha256_16 matches the
    code text of modarith.h + ntt_passes.h + ntt.hip); else {}."""
    path = os.path.join(PROFILES, name)
    if not os.path.exists(path):
        return {}
    fields = {}
    for line in open(path):
        if line.startswith("- ") and ":" in line:
            k, v = line[2:].split(":", 1)
            fields[k.strip()] = v.strip().strip("`")
    if fields.get("kernel_sources_sha256_16") != kernel_sources_digest():
        return {}
    return fields


def recorded_traffic():
    """HBM bytes per forward-NTT call from the committed counter summary, if it was
    taken on the current kernel sources (else None)."""
    try:
        return int(recorded_fields("ntt_forward_n65536_q24x60_traffic.md")["hbm_bytes_per_call"])
    except (KeyError, ValueError):
        return None


def recorded_valu():
    """VALU instructions per butterfly and VALUBusy of the forward NTT's two passes from
    the committed counter summary (current kernel sources only; else None)."""
    f = recorded_fields("ntt_forward_n65536_q24x60_valu.md")
    try:
        return {"valu_insts_per_butterfly_col": float(f["valu_insts_per_butterfly_col"]),
                "valu_insts_per_butterfly_row": float(f["valu_insts_per_butterfly_row"]),
                "valu_busy_pct_col": float(f["valu_busy_pct_col"]),
                "valu_busy_pct_row": float(f["valu_busy_pct_row"])}
    except (KeyError, ValueError):
        return None


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--rotate", type=int, default=3, help="distinct input sets cycled through")
    ap.add_argument("--ks-rotate", type=int, default=10,
                    help="distinct key-switch ciphertexts and keys cycled through (100.7 MB per key)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-next-rows", action="store_true", help="skip relin / rescale / hoisted / modraise timings")
    ap.add_argument("--no-other-configs", action="store_true", help="skip the n = 2^14 and n = 2048 workloads")
    ap.add_argument("--next-reps", type=int, default=10)
    ap.add_argument("--sustained", type=int, default=0, metavar="K",
                    help="instead of the step: K forward transforms of the large-ring batch back to back, "
                         "each timed with HIP events (shows the clock falling under sustained load)")
    ap.add_argument("--cpu-sample-limbs", type=int, default=384,
                    help="limbs of the batch the oracle processes for the CPU baseline (384 = all 16 polys)")
    return ap.parse_args()


def oracle_step_sample(primes, n, nq, npr, dnum, rows, a_host, b_host, ct_host, ksk_host, g, threads, min_seconds,
                       max_passes):
    """Whole passes of the step's operations on `rows` polynomials plus one key-switch,
    repeated until at least min_seconds of CPU work.  Returns (limb transforms, seconds,
    passes)."""
    import numpy as np

    import oracle as orc
    L = nq
    a = np.ascontiguousarray(a_host.reshape(-1, L, n)[:rows])
    b = np.ascontiguousarray(b_host.reshape(-1, L, n)[:rows])
    qs = primes[:L]
    per_pass = 2 * rows * L + dnum * (nq + npr) + 2 * (nq + npr)
    passes = 0
    t0 = time.perf_counter()
    while passes < max_passes and (passes == 0 or time.perf_counter() - t0 < min_seconds):
        ah = orc.batch_ntt(a, qs, threads=threads)
        c = orc.batch_pointwise(ah, b, qs)
        if rows % 2 == 0:
            orc.batch_tensor(ah.reshape(-1, 2, L, n), b.reshape(-1, 2, L, n), qs)
        c = orc.batch_ntt(c, qs, inverse=True, threads=threads)
        orc.batch_automorph(c, g, 0, qs)
        orc.keyswitch(ct_host, ksk_host, g, primes[: nq + npr], nq, dnum, threads=threads)
        passes += 1
    return per_pass * passes, time.perf_counter() - t0, passes


def cpu_baseline(primes, n, nq, npr, dnum, sample_limbs, a_host, b_host, ct_host, ksk_host, g, min_seconds=10.0,
                 max_passes=40):
    """The plain-C oracle on a bounded sample of one step, timed on the host cores: all
    of them (the reported value), and one core on a smaller sample."""
    import oracle as orc
    threads = orc.default_threads()
    L = nq
    rows = max(2, min(a_host.size // (L * n), sample_limbs // L))  # whole polynomials of the batch
    work, dt, passes = oracle_step_sample(primes, n, nq, npr, dnum, rows, a_host, b_host, ct_host, ksk_host, g,
                                          threads, min_seconds, max_passes)
    rows1 = 2
    work1, dt1, passes1 = oracle_step_sample(primes, n, nq, npr, dnum, rows1, a_host, b_host, ct_host, ksk_host, g,
                                             1, min_seconds / 2, max_passes)
    return {
        "value": work / dt,
        "unit": "limb-NTT/s",
        "cores": threads,
        "kind": "oracle",
        "sample": (f"{passes} passes over {rows} of the 16 polynomials (forward NTT, pointwise, tensor, inverse "
                   f"NTT, automorphism) plus one key-switch: {work} limb transforms in {dt:.1f} s"),
        "single_core": {
            "value": work1 / dt1,
            "unit": "limb-NTT/s",
            "cores": 1,
            "sample": (f"{passes1} passes over {rows1} polynomials plus one key-switch, one thread: {work1} limb "
                       f"transforms in {dt1:.1f} s"),
        },
    }


def time_op(fn, reps):
    """Mean milliseconds of fn over `reps` calls, HIP events on the current stream."""
    import torch
    fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def next_rows(B, plan, ksp, ws, primes, W, KS, C, ct, ksk, galois, reps):
    """Timings of the operations that complete a ciphertext product and of the
    bootstrapping-side ones, on the same workloads (not part of `value`)."""
    import torch
    n, L, nq, npr, dnum = W.n, W.limbs, KS.limbs, KS.special, KS.dnum
    nqp = nq + npr
    out = {}
    polys = C.numel() // (L * n)
    r_out = torch.empty(C.shape[:-2] + (L - 1, n), dtype=torch.int64, device=C.device)
    for mode, name in ((0, "rescale_truncating"), (1, "rescale_nearest")):
        ms = time_op(lambda: B.rescale(plan, r_out, C, mode), reps)
        byts = polys * (2 * L - 1) * n * 8
        out[name] = {"us": round(ms * 1e3, 2), "alg_GBps": round(byts / (ms * 1e-3) / 1e9, 1),
                     "hbm_frac": round(byts / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                     "shape": f"{polys} polys x {L} -> {L - 1} limbs"}
    del r_out
    if ksp is not None:
        d = torch.empty((1, 3, nq, n), dtype=torch.int64, device=C.device)
        d[:, :2].copy_(ct)
        d[:, 2].copy_(ct[:, 1])
        rel = torch.empty_like(ct)
        ms_rel = time_op(lambda: B.relinearize(ksp, rel, d, ksk, ws), reps)
        ms_ks = time_op(lambda: B.keyswitch(ksp, rel, ct, ksk, galois[0], ws), reps)
        out["relinearize"] = {"us": round(ms_rel * 1e3, 2), "per_s": round(1e3 / ms_rel, 1),
                              "keyswitch_us_same_run": round(ms_ks * 1e3, 2)}
        del d, rel
        # the same rotation on 4 ciphertexts in one call: larger launches fill the GPU
        nb = 4
        ctb = ct.repeat(nb, 1, 1, 1).contiguous()
        outb = torch.empty_like(ctb)
        wsb = B.workspace(ksp, nb)
        ms_b = time_op(lambda: B.keyswitch(ksp, outb, ctb, ksk, galois[0], wsb), reps)
        out["keyswitch_batch4"] = {"us": round(ms_b * 1e3, 2), "us_per_ciphertext": round(ms_b * 1e3 / nb, 2),
                                   "keyswitch_per_s": round(nb * 1e3 / ms_b, 1)}
        del ctb, outb, wsb
        R = 8
        gs = [galois[i % len(galois)] for i in range(R)]
        keys = ksk.unsqueeze(0).expand(R, *ksk.shape).contiguous()
        hout = torch.empty((R,) + tuple(ct.shape), dtype=torch.int64, device=C.device)
        hws = B.hoisted_workspace(ksp, R, 1)
        ms_h = time_op(lambda: B.keyswitch_hoisted(ksp, hout, ct, keys, gs, hws), reps)

        def separate():
            for r in range(R):
                B.keyswitch(ksp, hout[r], ct, keys[r], gs[r], ws)
        ms_sep = time_op(separate, reps)
        out["hoisted_rotations"] = {"rotations": R, "us": round(ms_h * 1e3, 2),
                                    "us_per_rotation": round(ms_h * 1e3 / R, 2),
                                    "separate_keyswitches_us": round(ms_sep * 1e3, 2),
                                    "speedup": round(ms_sep / ms_h, 3)}
        del keys, hout, hws
    for frm in (1, 2):
        mr = B.ModRaisePlan(plan, frm, L)
        x = torch.remainder(C[:2, 0, :frm], 1 << 20).contiguous()  # one ciphertext, residues below every prime
        y = torch.empty((2, L, n), dtype=torch.int64, device=C.device)
        ms = time_op(lambda: B.modraise(mr, y, x), reps)
        byts = 2 * (frm + L) * n * 8
        out[f"modraise_{frm}_to_{L}"] = {"us": round(ms * 1e3, 2), "alg_GBps": round(byts / (ms * 1e-3) / 1e9, 1)}
        del x, y, mr
    return out


def time_cycle(fns, reps):
    """Mean milliseconds per call of fns[i % len(fns)] over `reps` calls (HIP events)."""
    import torch
    for f in fns[: min(len(fns), 3)]:
        f()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(reps):
        fns[i % len(fns)]()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def time_graph(fns, replays=5):
    """Mean milliseconds per call when all of fns run inside one captured HIP graph."""
    import torch
    for f in fns:
        f()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for f in fns:
            f()
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(replays):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    del g
    return e0.elapsed_time(e1) / (replays * len(fns))


def galois_rows(B, plan, sets, E, galois, reps):
    """The forward NTT with sigma_g folded into its loads (ntt_forward_galois, in place)
    for each of the 16 Galois elements of the large-ring workload, next to the plain
    forward NTT timed the same way, and the coefficient-domain automorphism of each g.
    Calls rotate over the input sets, so an input was last touched two calls (> 400 MB)
    earlier."""
    fwd = time_cycle([lambda a=a: B.ntt_forward(plan, a) for a, _ in sets], max(reps, 2 * len(sets)))
    gal, aut = {}, {}
    for g in galois:
        gal[str(g)] = round(1e3 * time_cycle([lambda a=a, g=g: B.ntt_forward_galois(plan, a, a, g) for a, _ in sets],
                                             max(reps, 2 * len(sets))), 2)
        aut[str(g)] = round(1e3 * time_cycle([lambda b=b, g=g: B.automorph(plan, E, b, g, 0) for _, b in sets],
                                             max(reps, 2 * len(sets))), 2)
    gm, am = sum(gal.values()) / len(gal), sum(aut.values()) / len(aut)
    elem = sets[0][0].numel()
    return {"ntt_forward_us": round(fwd * 1e3, 2), "ntt_forward_galois_us": gal,
            "ntt_forward_galois_mean_us": round(gm, 2), "galois_over_plain": round(gm / (fwd * 1e3), 4),
            "automorph_coeff_us": aut, "automorph_coeff_mean_us": round(am, 2),
            "automorph_coeff_alg_GBps": round(16 * elem / (am * 1e-6) / 1e9, 1)}


def other_configs(B, reps):
    """Per-call times on the three smaller workloads (their parity is tested; these
    numbers are context, not part of `value`).  Operands rotate through copies of
    about 1 GB in total so that the 256 MB Infinity Cache does not stand in for HBM.
    The n = 2048 calls are also timed inside one HIP graph of many calls: their
    launch latency exceeds their memory time."""
    import torch
    from negacyclic_ntt_amd import inputs, workloads
    out = {}
    r3 = lambda x: round(x, 3)

    W = workloads.BATCH  # n = 2^14, 16 x 60-bit, 128 polynomials: NTT, pointwise, INTT
    ps = B.find_primes(W.bits, W.n, W.limbs)
    plan = B.Plan(W.n, ps, 0)
    a = B.to_device(inputs.uniform_residues(W.shape_a, ps, W.seed_a))
    b = B.to_device(inputs.uniform_residues(W.shape_a, ps, W.seed_b))
    pairs = [(a, b), (a.clone(), b.clone())]
    c = torch.empty_like(a)
    limbs = a.numel() // W.n
    f_ms = time_cycle([lambda x=x: B.ntt_forward(plan, x) for x, _ in pairs], reps)
    p_ms = time_cycle([lambda x=x, y=y: B.poly_mul_ntt(plan, c, x, y) for x, y in pairs], reps)
    i_ms = time_cycle([lambda x=x: B.ntt_inverse(plan, x) for x, _ in pairs], reps)
    out[W.name] = {"ntt_forward_us": r3(f_ms * 1e3), "ntt_forward_limb_ntt_per_s": round(limbs / (f_ms * 1e-3)),
                   "ntt_forward_alg_GBps": round(16 * a.numel() / (f_ms * 1e-3) / 1e9, 1),
                   "poly_mul_us": r3(p_ms * 1e3), "poly_mul_alg_GBps": round(24 * a.numel() / (p_ms * 1e-3) / 1e9, 1),
                   "ntt_inverse_us": r3(i_ms * 1e3), "ntt_inverse_limb_ntt_per_s": round(limbs / (i_ms * 1e-3))}
    del pairs, a, b, c, plan

    W = workloads.CHAIN  # n = 2048, 112 x 30-bit, 4 tokens x 2 components: NTT, tensor, INTT
    ps = B.find_primes(W.bits, W.n, W.limbs)
    plan = B.Plan(W.n, ps, 0)
    a = B.to_device(inputs.uniform_residues(W.shape_a, ps, W.seed_a))
    b = B.to_device(inputs.uniform_residues(W.shape_a, ps, W.seed_b))
    copies = [(a, b)] + [(a.clone(), b.clone()) for _ in range(34)]  # 35 x 29 MB
    d = torch.empty((W.shape_a[0], 3) + tuple(W.shape_a[2:]), dtype=torch.int64, device=a.device)
    limbs = a.numel() // W.n
    fwd = [lambda x=x: B.ntt_forward(plan, x) for x, _ in copies]
    f_ms = time_cycle(fwd, max(reps, len(fwd)))
    f_graph_ms = time_graph(fwd)
    t_ms = time_cycle([lambda x=x, y=y: B.ct_tensor_ntt(plan, d, x, y) for x, y in copies], max(reps, len(copies)))
    i_ms = time_cycle([lambda: B.ntt_inverse(plan, d)], reps)
    # the whole chain (NTT of both operands, tensor, INTT of the three outputs) in one launch
    prod = [lambda x=x, y=y: B.ct_tensor_coeff(plan, d, x, y) for x, y in copies]
    c_ms = time_cycle(prod, max(reps, len(copies)))
    c_graph_ms = time_graph(prod)
    out[W.name] = {"ntt_forward_us": r3(f_ms * 1e3), "ntt_forward_graph_us": r3(f_graph_ms * 1e3),
                   "ntt_forward_limb_ntt_per_s": round(limbs / (f_ms * 1e-3)),
                   "ntt_forward_graph_limb_ntt_per_s": round(limbs / (f_graph_ms * 1e-3)),
                   "ct_tensor_us": r3(t_ms * 1e3),
                   "ct_tensor_alg_GBps": round(56 * (a.numel() // 2) / (t_ms * 1e-3) / 1e9, 1),
                   "ntt_inverse_of_tensor_us": r3(i_ms * 1e3),
                   "ntt_inverse_limb_ntt_per_s": round(d.numel() // W.n / (i_ms * 1e-3)),
                   "chain_4_launches_us": r3((2 * f_ms + t_ms + i_ms) * 1e3),
                   "ct_tensor_coeff_us": r3(c_ms * 1e3), "ct_tensor_coeff_graph_us": r3(c_graph_ms * 1e3),
                   "ct_tensor_coeff_alg_GBps": round(56 * (a.numel() // 2) / (c_ms * 1e-3) / 1e9, 1),
                   "ct_tensor_coeff_limb_transforms_per_s": round(7 * (a.numel() // 2) // W.n / (c_ms * 1e-3))}
    del copies, a, b, d, plan

    W = workloads.POLYMUL  # n = 2048, 4 x 30-bit: NTT(A), NTT(B), pointwise, INTT
    ps = B.find_primes(W.bits, W.n, W.limbs)
    plan = B.Plan(W.n, ps, 0)
    a = B.to_device(inputs.uniform_residues(W.shape_a, ps, W.seed_a))
    b = B.to_device(inputs.uniform_residues(W.shape_a, ps, W.seed_b))
    c = torch.empty_like(a)

    def chain():
        B.ntt_forward(plan, a)
        B.ntt_forward(plan, b)
        B.poly_mul_ntt(plan, c, a, b)
        B.ntt_inverse(plan, c)
    m_ms = time_cycle([chain], reps)
    m_graph_ms = time_graph([chain] * 16)
    out[W.name] = {"multiply_us": r3(m_ms * 1e3), "multiply_graph_us": r3(m_graph_ms * 1e3),
                   "launches_per_multiply": 4}
    return out


def device_info():
    import torch
    p = torch.cuda.get_device_properties(0)
    info = {"name": p.name, "arch": getattr(p, "gcnArchName", None), "cus": p.multi_processor_count,
            "hbm_GB": round(p.total_memory / 1e9, 1), "hip": torch.version.hip, "torch": torch.__version__}
    peak = hip_clock_rate_khz()
    if peak:
        info["peak_sclk_MHz"] = round(peak / 1e3)
    return info


def hip_clock_rate_khz():
    """hipDeviceAttributeClockRate of device 0 (the peak shader clock, kHz), or None."""
    import ctypes
    import re
    try:
        hdr = open("/opt/rocm/include/hip/hip_runtime_api.h").read()
        body = hdr[hdr.index("typedef enum hipDeviceAttribute_t"):]
        body = body[body.index("{") + 1: body.index("}")]
        idx, value, seen = None, -1, {}
        for line in re.sub(r"//[^\n]*|/\*.*?\*/", "", body, flags=re.S).split(","):
            m = re.match(r"\s*(\w+)\s*(?:=\s*(\w+))?\s*$", line)
            if not m:
                continue
            if m.group(2):  # an explicit value: a number or an earlier enumerator
                value = seen[m.group(2)] if m.group(2) in seen else int(m.group(2), 0)
            else:
                value += 1
            seen[m.group(1)] = value
            if m.group(1) == "hipDeviceAttributeClockRate":
                idx = value
                break
        if idx is None:
            return None
        lib = ctypes.CDLL("libamdhip64.so")
        v = ctypes.c_int(0)
        if lib.hipDeviceGetAttribute(ctypes.byref(v), idx, 0) != 0 or v.value <= 0:
            return None
        return v.value
    except (OSError, ValueError, AttributeError):
        return None


class ClockSampler:
    """Samples the current shader clock (the starred level of the GPU's pp_dpm_sclk in
    sysfs) every 2 ms in a background thread while the timed steps run."""

    def __init__(self):
        import glob
        import threading
        self.path = self._find(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
        self.samples = []
        self._stop = threading.Event()
        self._t = threading.Thread(target=self._run, daemon=True) if self.path else None

    @staticmethod
    def _find(paths):
        import torch
        try:
            props = torch.cuda.get_device_properties(0)
            bus = getattr(props, "pci_bus_id", None)
        except RuntimeError:
            bus = None
        for pth in sorted(paths):
            dev = os.path.realpath(os.path.dirname(pth))
            if bus is None and len(paths) == 1:
                return pth
            if bus is not None and os.path.basename(dev).split(":")[-2:-1] == [f"{bus:02x}"]:
                return pth
        return None

    def _read(self):
        try:
            for line in open(self.path):
                if line.rstrip().endswith("*"):
                    return int("".join(ch for ch in line.split(":", 1)[1] if ch.isdigit()))
        except (OSError, ValueError, IndexError):
            return None
        return None

    def _run(self):
        while not self._stop.is_set():
            v = self._read()
            if v:
                self.samples.append(v)
            self._stop.wait(0.002)

    def __enter__(self):
        if self._t:
            self._t.start()
        return self

    def __exit__(self, *exc):
        if self._t:
            self._stop.set()
            self._t.join()

    def summary(self):
        if not self.samples:
            return {"source": self.path, "samples": 0}
        v = sorted(self.samples)
        return {"source": self.path, "samples": len(v), "min_MHz": v[0], "median_MHz": v[len(v) // 2],
                "max_MHz": v[-1]}


def sustained(B, calls):
    """K back-to-back forward transforms of the large-ring batch over four resident copies.
    Events between calls add no gaps; one JSON line with every call's duration."""
    import torch
    from negacyclic_ntt_amd import inputs, workloads
    W = workloads.RING
    primes = B.find_primes(W.bits, W.n, W.limbs)
    plan = B.Plan(W.n, primes, 0)
    a0 = B.to_device(inputs.uniform_residues(W.shape_a, primes, W.seed_a))
    sets = [a0] + [a0.clone() for _ in range(3)]
    B.ntt_forward(plan, sets[3])  # loads the kernels; untimed
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(calls + 1)]
    ev[0].record()
    for i in range(calls):
        B.ntt_forward(plan, sets[i % 4])
        ev[i + 1].record()
    torch.cuda.synchronize()
    us = [round(ev[i].elapsed_time(ev[i + 1]) * 1e3, 1) for i in range(calls)]
    head, tail = us[: min(8, calls)], us[-min(10, calls):]
    return {"mode": "sustained_ntt_forward", "workload": W.name, "calls": calls, "us_per_call": us,
            "first_calls_mean_us": round(sum(head) / len(head), 1),
            "last_calls_mean_us": round(sum(tail) / len(tail), 1)}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1", "n_gpus": args.gpus}))
        sys.exit(2)
    import numpy as np
    import torch

    from negacyclic_ntt_amd import binding as B
    from negacyclic_ntt_amd import inputs, workloads

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    if args.sustained > 0:
        print(json.dumps(sustained(B, args.sustained)), flush=True)
        return
    dev = torch.device("cuda:0")
    W, KS = workloads.RING, workloads.KEYSWITCH
    n, L, nq, npr, dnum = W.n, W.limbs, KS.limbs, KS.special, KS.dnum
    primes = B.find_primes(W.bits, n, nq + npr)  # the ring's 24 primes are the first 24 of this list
    plan = B.Plan(n, primes, 0)
    galois = W.galois

    # ---- inputs (host generation, then resident on the device) ----
    t_gen = time.perf_counter()
    a_host = inputs.uniform_residues(W.shape_a, primes[:L], W.seed_a)
    b_host = inputs.uniform_residues(W.shape_a, primes[:L], W.seed_a + 1)
    ct_host = inputs.uniform_residues(KS.shape_a, primes[:nq], KS.seed_a)
    ksk_host = inputs.uniform_residues((dnum, 2, nq + npr, n), primes[: nq + npr], KS.seed_b)
    a0, b0 = B.to_device(a_host), B.to_device(b_host)
    sets = [(a0, b0)] + [(a0.clone(), b0.clone()) for _ in range(args.rotate - 1)]
    ct = B.to_device(ct_host)
    ksk0 = B.to_device(ksk_host)
    nks = max(1, args.ks_rotate)
    keys = [ksk0] + [ksk0.clone() for _ in range(nks - 1)]
    cts = [ct] + [ct.clone() for _ in range(nks - 1)]
    C = torch.empty_like(a0)
    E = torch.empty_like(a0)
    D = torch.empty((W.shape_a[0], 3, L, n), dtype=torch.int64, device=dev)
    ks_out = torch.empty_like(ct)
    try:
        ksp = B.KeySwitchPlan(plan, nq, npr, dnum)
        ws = B.workspace(ksp, 1)
    except B.NttError:
        ksp = None
    # A plain device copy of known size: its FETCH_SIZE / WRITE_SIZE counters
    # calibrate the HBM byte counters of the other kernels.
    cal_src = torch.empty(CALIBRATION_COPY_BYTES // 8, dtype=torch.int64, device=dev).fill_(1)
    cal_dst = torch.empty_like(cal_src)
    cal_dst.copy_(cal_src)
    del cal_src, cal_dst
    torch.cuda.synchronize()
    gen_s = time.perf_counter() - t_gen
    resident_bytes = (sum(t.numel() * 8 for pair in sets for t in pair) + sum(k.numel() * 8 for k in keys)
                      + sum(c.numel() * 8 for c in cts))

    rows = ["ntt_forward", "poly_mul_ntt", "ct_tensor_ntt", "ntt_inverse", "automorph", "keyswitch"]
    ev = {r: [] for r in rows}
    # One event between consecutive rows, across steps too (6 markers per step and one
    # before the first timed row): row i is timed from the event before it to the event
    # after it, on the stream the library uses.  A fresh event at the start of every step
    # put two markers (~10 us of idle GPU) in front of each step's forward NTT.
    last = [None]

    def step(s, timed):
        a, b = sets[s % len(sets)]
        g = galois[s % len(galois)]

        def run(name, fn):
            if timed:
                if last[0] is None:
                    last[0] = torch.cuda.Event(enable_timing=True)
                    last[0].record()
                fn()
                e1 = torch.cuda.Event(enable_timing=True)
                e1.record()
                ev[name].append((last[0], e1))
                last[0] = e1
            else:
                fn()

        run("ntt_forward", lambda: B.ntt_forward(plan, a))
        run("poly_mul_ntt", lambda: B.poly_mul_ntt(plan, C, a, b))
        run("ct_tensor_ntt", lambda: B.ct_tensor_ntt(plan, D, a, b))
        run("ntt_inverse", lambda: B.ntt_inverse(plan, C))
        # the B operand of the next set: last touched a whole step (> 1 GB of traffic) ago
        run("automorph", lambda: B.automorph(plan, E, sets[(s + 1) % len(sets)][1], g, 0))
        if ksp is not None:
            run("keyswitch", lambda: B.keyswitch(ksp, ks_out, cts[s % len(cts)], keys[s % len(keys)], g, ws))

    for s in range(args.warmup):
        step(s, False)
    torch.cuda.synchronize()
    with ClockSampler() as clock:
        t0 = time.perf_counter()
        for s in range(args.steps):
            step(args.warmup + s, True)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0

    ms = {r: [e0.elapsed_time(e1) for e0, e1 in ev[r]] for r in rows if ev[r]}
    mean_ms = {r: sum(v) / len(v) for r, v in ms.items()}
    polys = W.shape_a[0] * W.shape_a[1]
    limb = polys * L
    ks_limb_ntts = (dnum * (nq + npr) + 2 * (nq + npr)) if ksp is not None else 0
    limb_ntts_per_step = 2 * limb + ks_limb_ntts
    ms_per_step = wall * 1e3 / args.steps
    value = limb_ntts_per_step / (ms_per_step * 1e-3)

    # algorithmic bytes per call (each residue read and written once; 8 B each)
    elem = limb * n
    alg_bytes = {
        "ntt_forward": 16 * elem,
        "ntt_inverse": 16 * elem,
        "poly_mul_ntt": 24 * elem,
        "ct_tensor_ntt": 56 * elem // 2,
        "automorph": 16 * elem,
        "keyswitch": 8 * n * (2 * nq + dnum * 2 * (nq + npr) + 2 * nq),
    }
    per_row = {}
    for r, m in mean_ms.items():
        gbps = alg_bytes[r] / (m * 1e-3) / 1e9
        per_row[r] = {"ms": round(m, 4), "alg_GBps": round(gbps, 1), "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4)}
    per_row["ntt_forward"]["limb_ntt_per_s"] = round(limb / (mean_ms["ntt_forward"] * 1e-3))
    per_row["ntt_inverse"]["limb_ntt_per_s"] = round(limb / (mean_ms["ntt_inverse"] * 1e-3))
    if "keyswitch" in mean_ms:
        per_row["keyswitch"]["keyswitch_per_s"] = round(1e3 / mean_ms["keyswitch"], 1)

    # Dominant operation: the forward NTT (two launches: column pass + row pass).
    # Its algorithmic work per call: limb * (n/2) log2(n) butterflies, 16 n bytes per limb.
    fwd_s = mean_ms["ntt_forward"] * 1e-3
    butterflies = limb * (n // 2) * (n.bit_length() - 1)
    alu_tops = butterflies * MUL32_PER_BUTTERFLY / fwd_s / 1e12
    fwd_gbps = alg_bytes["ntt_forward"] / fwd_s / 1e9
    traffic = recorded_traffic()
    kname = "ntt_forward (ntt_col_kernel + ntt_row_kernel, n=2^16, 384 limbs)"
    roofline = {
        "kernel": kname,
        "bound": "hbm",
        "achieved": round(fwd_gbps, 1),
        "peak": HBM_PEAK_GBPS,
        "unit": "GB/s",
        "frac": round(fwd_gbps / HBM_PEAK_GBPS, 4),
        "traffic": traffic,
        "bytes": "16 n per limb-NTT (each residue read and written once) x 384 limb-NTTs per call",
        "us_per_call": round(fwd_s * 1e6, 2),
        "limiter": "VALU issue, not HBM (alu_issue)",
    }
    clk = clock.summary()
    alu_issue = {
        "kernel": kname,
        "achieved": round(alu_tops, 3),
        "peak": round(MUL32_PEAK_TOPS, 2),
        "unit": "TOP/s",
        "frac": round(alu_tops / MUL32_PEAK_TOPS, 4),
        "ops": "32-bit multiplies, 10 per 64-bit Shoup butterfly",
        "peak_assumes": "256 CUs x 64 lanes x 2400 MHz, one 32-bit multiply per lane per clock",
        "sampled_sclk": clk,
    }
    if clk.get("median_MHz"):
        alu_issue["frac_at_sampled_median_sclk"] = round(alu_tops / (256 * 64 * clk["median_MHz"] * 1e6 / 1e12), 4)
    valu = recorded_valu()
    alu_issue["counters"] = valu
    rt_ms = mean_ms["ntt_forward"] + mean_ms["ntt_inverse"]
    out = {
        "metric": "limb-NTTs/sec + achieved HBM GB/s (N=2^16, 60-bit, 1 GPU); keyswitches/sec",
        "value": round(value, 1),
        "unit": "limb-NTT/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u64",
        "data": "synthetic",
        "config": {"workload": W.name, "n": n, "primes": f"{L} x 60-bit", "batch": list(W.shape_a),
                   "keyswitch": KS.name, "rotated_sets": len(sets), "resident_GB": round(resident_bytes / 1e9, 2)},
        "ntt_round_trip": {"limb_ntt_per_s": round(2 * limb / (rt_ms * 1e-3)),
                           "alg_GBps": round(32 * elem / (rt_ms * 1e-3) / 1e9, 1)},
        "keyswitches_per_s": per_row.get("keyswitch", {}).get("keyswitch_per_s"),
        "rows": per_row,
        "roofline": roofline,
        "alu_issue": alu_issue,
        "input_gen_s": round(gen_s, 2),
    }
    out["device"] = device_info()
    out["galois"] = galois_rows(B, plan, sets, E, galois, args.next_reps)
    if not args.no_next_rows:
        out["next_rows"] = next_rows(B, plan, ksp, ws, primes, W, KS, C, ct, ksk0, galois, args.next_reps)
    if not args.no_other_configs:
        del sets, keys, cts, C, E, D
        out["other_configs"] = other_configs(B, args.next_reps)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(primes, n, nq, npr, dnum, args.cpu_sample_limbs, a_host, b_host,
                                           ct_host, ksk_host, galois[0])
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
