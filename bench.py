#!/usr/bin/env python3
"""Throughput benchmark on one MI355X.

One step = one pass of every hot-path operation over one batch of the
large-ring workload (n = 2^16, 24 primes of 60 bits, 8 ciphertexts = 16
polynomials, tensor [8][2][24][65536], seeded uniform residues):
  1. forward NTT of A                                  (384 limb-NTTs)
  2. pointwise product  C = A_hat * B_hat              (NTT domain)
  3. ciphertext tensor product D = (A_hat, B_hat)      ([8][3][24][n])
  4. inverse NTT of C                                  (384 limb-INTTs)
  5. coefficient-domain automorphism E = sigma_g(C), g = 5^(2^(s mod 16)) mod 2n
  6. one rotation key-switch of a 1-ciphertext batch (Q = 24, P = 8, dnum = 3)
     with the same g (96 forward + 64 inverse limb transforms inside)
`value` is limb-NTTs per second over whole steps (forward and inverse
transforms, those inside the key-switch included).  Inputs are resident in HBM
before timing; the timed steps rotate over enough distinct buffers and keys
(> 1 GB) that the 256 MB Infinity Cache cannot hold them.
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
    """sha256/16 over the code text of modarith.h + ntt.hip (comments excluded, so a
    comment edit does not invalidate counters taken on the same kernels)."""
    import hashlib
    if read is None:
        def read(name):
            with open(os.path.join(ROOT, "negacyclic_ntt_amd", "csrc", name)) as fh:
                return fh.read()
    h = hashlib.sha256()
    for f in ("modarith.h", "ntt.hip"):
        h.update(code_text(read(f)).encode())
    return h.hexdigest()[:16]


def recorded_traffic():
    """HBM bytes per forward-NTT call from the committed counter summary, if it was
    taken on the current kernel sources (else None)."""
    path = os.path.join(PROFILES, "ntt_forward_n65536_q24x60_traffic.md")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if line.startswith("- ") and ":" in line:
            k, v = line[2:].split(":", 1)
            fields[k.strip()] = v.strip().strip("`")
    if fields.get("kernel_sources_sha256_16") != kernel_sources_digest():
        return None
    try:
        return int(fields["hbm_bytes_per_call"])
    except (KeyError, ValueError):
        return None


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--rotate", type=int, default=3, help="distinct input sets cycled through")
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


def cpu_baseline(primes, n, nq, npr, dnum, sample_limbs, a_host, b_host, ct_host, ksk_host, g, min_seconds=10.0,
                 max_passes=40):
    """The plain-C oracle on a bounded sample of one step, timed on the host cores."""
    import numpy as np

    import oracle as orc
    threads = orc.default_threads()
    L = nq
    rows = max(2, min(a_host.size // (L * n), sample_limbs // L))  # whole polynomials of the batch
    a = np.ascontiguousarray(a_host.reshape(-1, L, n)[:rows])
    b = np.ascontiguousarray(b_host.reshape(-1, L, n)[:rows])
    qs = primes[:L]
    per_pass = 2 * rows * L + dnum * (nq + npr) + 2 * (nq + npr)
    passes = 0
    t0 = time.perf_counter()
    # Whole passes until at least min_seconds of CPU work (bounded by max_passes).
    while passes < max_passes and (passes == 0 or time.perf_counter() - t0 < min_seconds):
        ah = orc.batch_ntt(a, qs, threads=threads)
        c = orc.batch_pointwise(ah, b, qs)
        if rows % 2 == 0:
            orc.batch_tensor(ah.reshape(-1, 2, L, n), b.reshape(-1, 2, L, n), qs)
        c = orc.batch_ntt(c, qs, inverse=True, threads=threads)
        orc.batch_automorph(c, g, 0, qs)
        orc.keyswitch(ct_host, ksk_host, g, primes[: nq + npr], nq, dnum, threads=threads)
        passes += 1
    dt = time.perf_counter() - t0
    limb_ntts = per_pass * passes
    return {
        "value": limb_ntts / dt,
        "unit": "limb-NTT/s",
        "cores": threads,
        "kind": "oracle",
        "sample": (f"{passes} passes over {rows} of the 16 polynomials (forward NTT, pointwise, tensor, inverse "
                   f"NTT, automorphism) plus one key-switch: {limb_ntts} limb transforms in {dt:.1f} s"),
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
    out[W.name] = {"ntt_forward_us": r3(f_ms * 1e3), "ntt_forward_graph_us": r3(f_graph_ms * 1e3),
                   "ntt_forward_limb_ntt_per_s": round(limbs / (f_ms * 1e-3)),
                   "ntt_forward_graph_limb_ntt_per_s": round(limbs / (f_graph_ms * 1e-3)),
                   "ct_tensor_us": r3(t_ms * 1e3),
                   "ct_tensor_alg_GBps": round(56 * (a.numel() // 2) / (t_ms * 1e-3) / 1e9, 1),
                   "ntt_inverse_of_tensor_us": r3(i_ms * 1e3),
                   "ntt_inverse_limb_ntt_per_s": round(d.numel() // W.n / (i_ms * 1e-3))}
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
    clock = getattr(p, "clock_rate", None)
    if clock:
        info["clock_MHz"] = round(clock / 1e3)
    return info


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
            "first_calls_mean_us": round(sum(head) / len(head), 1), "last_calls_mean_us": round(sum(tail) / len(tail), 1)}


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
    keys = [ksk0] + [ksk0.clone() for _ in range(max(0, 2 * args.rotate - 1))]
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
    resident_bytes = sum(t.numel() * 8 for pair in sets for t in pair) + sum(k.numel() * 8 for k in keys)

    rows = ["ntt_forward", "poly_mul_ntt", "ct_tensor_ntt", "ntt_inverse", "automorph", "keyswitch"]
    ev = {r: [] for r in rows}

    def step(s, timed):
        a, b = sets[s % len(sets)]
        g = galois[s % len(galois)]

        # One event between consecutive rows (7 markers per step): row i is timed from
        # the event before it to the event after it, on the stream the library uses.
        last = [None]

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
        run("automorph", lambda: B.automorph(plan, E, C, g, 0))
        if ksp is not None:
            run("keyswitch", lambda: B.keyswitch(ksp, ks_out, ct, keys[s % len(keys)], g, ws))

    for s in range(args.warmup):
        step(s, False)
    torch.cuda.synchronize()
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
    roofline = {
        "kernel": "ntt_forward (ntt_col_kernel + ntt_row_kernel, n=2^16, 384 limbs)",
        "bound": "alu",
        "achieved": round(alu_tops, 3),
        "peak": round(MUL32_PEAK_TOPS, 2),
        "unit": "TOP/s",
        "frac": round(alu_tops / MUL32_PEAK_TOPS, 4),
        "traffic": traffic,
        "ops": "32-bit multiplies, 10 per 64-bit Shoup butterfly",
        "hbm_alg_GBps": round(fwd_gbps, 1),
        "hbm_frac": round(fwd_gbps / HBM_PEAK_GBPS, 4),
        "us_per_call": round(fwd_s * 1e6, 2),
    }
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
        "input_gen_s": round(gen_s, 2),
    }
    out["device"] = device_info()
    if not args.no_next_rows:
        out["next_rows"] = next_rows(B, plan, ksp, ws, primes, W, KS, C, ct, ksk0, galois, args.next_reps)
    if not args.no_other_configs:
        del sets, keys, C, E, D
        out["other_configs"] = other_configs(B, args.next_reps)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(primes, n, nq, npr, dnum, args.cpu_sample_limbs, a_host, b_host,
                                           ct_host, ksk_host, galois[0])
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
