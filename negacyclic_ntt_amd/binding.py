"""Thin ctypes binding over the C ABI in ``include/negacyclic_ntt.h``.

Argument marshalling only: every step of every operation runs in the HIP
library.  Tensors are torch ``int64`` tensors on the plan's GPU holding uint64
residues (all residues are below 2^62, so the sign bit is never set), C-contiguous,
shaped ``[..., limbs, n]``.  Work is enqueued on torch's current stream of that
device and the calls return without synchronising.
"""
import ctypes
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libnegacyclic_ntt.so")

NTT_OK, NTT_EINVAL, NTT_EUNSUPPORTED, NTT_ENOMEM, NTT_EDEVICE, NTT_EOVERLAP = 0, -1, -2, -3, -4, -5

_lib = None
_U64P = ctypes.POINTER(ctypes.c_uint64)
_VP = ctypes.c_void_p


class NttError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {lib().ntt_status_string(status).decode()} ({status})")


def lib():
    """Load the HIP library (building it first if it was never built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            from . import build as _build
            _build.build()
        L = ctypes.CDLL(LIB_PATH)
        u64, u32, i32, sz = ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int, ctypes.c_size_t
        sig = {
            "ntt_status_string": (ctypes.c_char_p, [i32]),
            "ntt_find_primes": (i32, [u32, u32, u32, _U64P]),
            "ntt_plan_create": (i32, [ctypes.POINTER(_VP), u32, _U64P, u32, _U64P, i32]),
            "ntt_plan_get_tables": (i32, [_VP, u32, _U64P, _U64P, _U64P, _U64P, _U64P]),
            "ntt_plan_info": (i32, [_VP, ctypes.POINTER(u32), ctypes.POINTER(u32), ctypes.POINTER(i32)]),
            "ntt_plan_prime": (i32, [_VP, u32, _U64P]),
            "ntt_plan_destroy": (None, [_VP]),
            "ntt_forward": (i32, [_VP, _VP, u64, u32, u32, _VP]),
            "ntt_inverse": (i32, [_VP, _VP, u64, u32, u32, _VP]),
            "ntt_forward_galois": (i32, [_VP, _VP, _VP, u64, u64, u32, u32, _VP]),
            "poly_mul_ntt": (i32, [_VP, _VP, _VP, _VP, u64, u32, u32, _VP]),
            "ct_tensor_ntt": (i32, [_VP, _VP, _VP, _VP, u64, u32, u32, _VP]),
            "ct_tensor_coeff": (i32, [_VP, _VP, _VP, _VP, u64, u32, u32, _VP]),
            "automorph": (i32, [_VP, _VP, _VP, u64, i32, u64, u32, u32, _VP]),
            "keyswitch_plan_create": (i32, [ctypes.POINTER(_VP), _VP, u32, u32, u32]),
            "keyswitch_workspace_size": (i32, [_VP, u64, ctypes.POINTER(sz)]),
            "keyswitch": (i32, [_VP, _VP, _VP, _VP, u64, u64, _VP, sz, _VP]),
            "keyswitch_noalloc": (i32, [_VP, _VP, _VP, _VP, u64, u64, _VP]),
            "keyswitch_plan_destroy": (None, [_VP]),
            "relinearize": (i32, [_VP, _VP, _VP, _VP, u64, _VP, sz, _VP]),
            "modraise_plan_create": (i32, [ctypes.POINTER(_VP), _VP, u32, u32]),
            "modraise": (i32, [_VP, _VP, _VP, u64, _VP]),
            "modraise_plan_destroy": (None, [_VP]),
            "keyswitch_hoisted_workspace_size": (i32, [_VP, u32, u64, ctypes.POINTER(sz)]),
            "keyswitch_hoisted": (i32, [_VP, _VP, _VP, _VP, _U64P, u32, u64, _VP, sz, _VP]),
            "rescale": (i32, [_VP, _VP, _VP, i32, u64, u32, u32, _VP]),
            "ntt_count_noncanonical": (i32, [_VP, _VP, u64, u32, u32, _VP, _VP]),
            "ntt_set_debug_checks": (None, [i32]),
            "ntt_set_max_launch_threads": (i32, [u64]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _check(status: int, what: str):
    if status != NTT_OK:
        raise NttError(status, what)


def _u64arr(values):
    arr = np.ascontiguousarray(np.asarray(values, dtype=np.uint64))
    return arr, arr.ctypes.data_as(_U64P)


def find_primes(bits: int, n: int, count: int) -> list:
    """First `count` primes below 2^bits that are 1 mod 2n, descending."""
    arr = np.zeros(max(count, 1), dtype=np.uint64)
    _check(lib().ntt_find_primes(bits, n, count, arr.ctypes.data_as(_U64P)), "ntt_find_primes")
    return [int(v) for v in arr[:count]]


class Plan:
    """Transform plan for ring degree n over a list of primes (see ntt_plan_create).

    device: a CUDA/HIP device index, a torch.device, or -1 for a host-only plan.
    """

    def __init__(self, n: int, primes, device=0, psi=None):
        if hasattr(device, "index"):
            device = device.index if device.index is not None else 0
        self.n = int(n)
        self.primes = [int(p) for p in primes]
        self.device = int(device)
        parr, pp = _u64arr(self.primes)
        psi_p = None
        if psi is not None:
            self._psi_arr, psi_p = _u64arr(psi)
        h = _VP()
        _check(lib().ntt_plan_create(ctypes.byref(h), self.n, pp, len(self.primes), psi_p, self.device),
               "ntt_plan_create")
        self._h = h

    @property
    def handle(self):
        if self._h is None:
            raise ValueError("plan destroyed")
        return self._h

    def destroy(self):
        if getattr(self, "_h", None) is not None:
            lib().ntt_plan_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass

    def tables(self, limb: int) -> dict:
        out = {k: np.zeros(self.n, dtype=np.uint64) for k in ("fwd", "fwd_shoup", "inv", "inv_shoup")}
        psi = ctypes.c_uint64()
        _check(lib().ntt_plan_get_tables(self.handle, limb, ctypes.byref(psi),
                                         *(out[k].ctypes.data_as(_U64P) for k in ("fwd", "fwd_shoup", "inv",
                                                                                 "inv_shoup"))),
               "ntt_plan_get_tables")
        out["psi"] = int(psi.value)
        return out


def _stream_ptr(t, stream):
    if stream is not None:
        return _VP(stream if isinstance(stream, int) else stream.cuda_stream)
    import torch
    return _VP(torch.cuda.current_stream(t.device).cuda_stream)


def _on_stream(t, stream):
    """Context that makes `stream` torch's current stream on t's device (a no-op when
    stream is None).  Temporaries a call allocates for itself (key-switch workspaces,
    the count of non-canonical residues) are created inside it, so that torch's
    caching allocator orders their reuse, and their initialisation and read-back, on
    the stream the library launches on."""
    import contextlib

    import torch
    if stream is None:
        return contextlib.nullcontext()
    if isinstance(stream, int):
        stream = torch.cuda.ExternalStream(stream, device=t.device)
    return torch.cuda.stream(stream)


def _check_tensor(t, plan: Plan, name: str, lead: int = 0):
    """Validate a residue tensor and return (batch, num_limbs)."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != torch.int64:
        raise TypeError(f"{name} must be int64 (uint64 residues), got {t.dtype}")
    if t.device.type != "cuda" or t.device.index != plan.device:
        raise ValueError(f"{name} must be on cuda:{plan.device}, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.dim() < 2 + lead or t.shape[-1] != plan.n:
        raise ValueError(f"{name} must have shape [..., limbs, {plan.n}], got {tuple(t.shape)}")
    limbs = t.shape[-2]
    per = limbs * plan.n * (t.shape[-3] if lead else 1)
    batch = t.numel() // per if per else 0
    return batch, limbs


def ntt_forward(plan: Plan, x, limb_begin: int = 0, stream=None):
    """In-place forward NTT of x [..., limbs, n]; returns x."""
    batch, limbs = _check_tensor(x, plan, "x")
    _check(lib().ntt_forward(plan.handle, _VP(x.data_ptr()), batch, limb_begin, limbs, _stream_ptr(x, stream)),
           "ntt_forward")
    return x


def ntt_inverse(plan: Plan, x, limb_begin: int = 0, stream=None):
    """In-place inverse NTT of x [..., limbs, n]; returns x."""
    batch, limbs = _check_tensor(x, plan, "x")
    _check(lib().ntt_inverse(plan.handle, _VP(x.data_ptr()), batch, limb_begin, limbs, _stream_ptr(x, stream)),
           "ntt_inverse")
    return x


def ntt_forward_galois(plan: Plan, out, x, galois_elt: int, limb_begin: int = 0, stream=None):
    """out = NTT(sigma_g(x)); out may be x itself."""
    batch, limbs = _check_tensor(x, plan, "x")
    _check_tensor(out, plan, "out")
    if out.shape != x.shape:
        raise ValueError("out and x shapes differ")
    _check(lib().ntt_forward_galois(plan.handle, _VP(out.data_ptr()), _VP(x.data_ptr()), galois_elt, batch,
                                    limb_begin, limbs, _stream_ptr(x, stream)), "ntt_forward_galois")
    return out


def poly_mul_ntt(plan: Plan, out, a, b, limb_begin: int = 0, stream=None):
    batch, limbs = _check_tensor(a, plan, "a")
    _check_tensor(b, plan, "b")
    _check_tensor(out, plan, "out")
    if not (a.shape == b.shape == out.shape):
        raise ValueError("a, b and out must have the same shape")
    _check(lib().poly_mul_ntt(plan.handle, _VP(out.data_ptr()), _VP(a.data_ptr()), _VP(b.data_ptr()), batch,
                              limb_begin, limbs, _stream_ptr(a, stream)), "poly_mul_ntt")
    return out


def ct_tensor_ntt(plan: Plan, out, a, b, limb_begin: int = 0, stream=None):
    """a, b: [..., 2, limbs, n] -> out [..., 3, limbs, n]."""
    batch, limbs = _check_tensor(a, plan, "a", lead=1)
    _check_tensor(b, plan, "b", lead=1)
    _check_tensor(out, plan, "out", lead=1)
    if (a.shape != b.shape or a.shape[-3] != 2 or out.shape[:-3] != a.shape[:-3]
            or out.shape[-3:] != (3, limbs, plan.n)):
        raise ValueError("expected a, b [..., 2, L, n] and out [..., 3, L, n]")
    _check(lib().ct_tensor_ntt(plan.handle, _VP(out.data_ptr()), _VP(a.data_ptr()), _VP(b.data_ptr()), batch,
                               limb_begin, limbs, _stream_ptr(a, stream)), "ct_tensor_ntt")
    return out


def ct_tensor_coeff(plan: Plan, out, a, b, limb_begin: int = 0, stream=None):
    """Coefficient-domain ciphertext product: a, b [..., 2, limbs, n] -> out [..., 3, limbs, n]
    (negacyclic products d0 = a0 b0, d1 = a0 b1 + a1 b0, d2 = a1 b1; n <= 4096)."""
    batch, limbs = _check_tensor(a, plan, "a", lead=1)
    _check_tensor(b, plan, "b", lead=1)
    _check_tensor(out, plan, "out", lead=1)
    if (a.shape != b.shape or a.shape[-3] != 2 or out.shape[:-3] != a.shape[:-3]
            or out.shape[-3:] != (3, limbs, plan.n)):
        raise ValueError("expected a, b [..., 2, L, n] and out [..., 3, L, n]")
    _check(lib().ct_tensor_coeff(plan.handle, _VP(out.data_ptr()), _VP(a.data_ptr()), _VP(b.data_ptr()), batch,
                                 limb_begin, limbs, _stream_ptr(a, stream)), "ct_tensor_coeff")
    return out


def automorph(plan: Plan, out, x, galois_elt: int, domain: int = 0, limb_begin: int = 0, stream=None):
    """out = sigma_g(x); domain 0 = coefficient, 1 = NTT (bit-reversed)."""
    batch, limbs = _check_tensor(x, plan, "x")
    _check_tensor(out, plan, "out")
    if out.shape != x.shape:
        raise ValueError("out and x shapes differ")
    _check(lib().automorph(plan.handle, _VP(out.data_ptr()), _VP(x.data_ptr()), galois_elt, domain, batch,
                           limb_begin, limbs, _stream_ptr(x, stream)), "automorph")
    return out


def count_noncanonical(plan: Plan, x, limb_begin: int = 0, stream=None) -> int:
    """Number of residues of x [..., limbs, n] that are >= their prime (synchronises)."""
    import torch
    batch, limbs = _check_tensor(x, plan, "x")
    with _on_stream(x, stream):  # zero fill, count and read-back all on the launch stream
        cnt = torch.zeros(1, dtype=torch.int64, device=x.device)
        _check(lib().ntt_count_noncanonical(plan.handle, _VP(x.data_ptr()), batch, limb_begin, limbs,
                                            _VP(cnt.data_ptr()), _stream_ptr(x, stream)), "ntt_count_noncanonical")
        return int(cnt.item())


def set_debug_checks(on: bool):
    """Turn the library's input checks on or off for this process (see ntt_set_debug_checks)."""
    lib().ntt_set_debug_checks(1 if on else 0)


def set_max_launch_threads(threads: int = 0):
    """Cap the threads of one kernel launch (0: the hardware default); larger calls
    are split into several launches (see ntt_set_max_launch_threads)."""
    _check(lib().ntt_set_max_launch_threads(int(threads)), "ntt_set_max_launch_threads")


def rescale(plan: Plan, out, x, mode: int = 0, limb_begin: int = 0, stream=None):
    """out [..., limbs - 1, n] = x [..., limbs, n] divided by its last prime;
    mode 0 truncating (floor), 1 nearest (floor of X / q + 1/2)."""
    batch, limbs = _check_tensor(x, plan, "x")
    _check_tensor(out, plan, "out")
    if tuple(out.shape) != tuple(x.shape[:-2]) + (limbs - 1, plan.n):
        raise ValueError("out must be [..., limbs - 1, n]")
    _check(lib().rescale(plan.handle, _VP(out.data_ptr()), _VP(x.data_ptr()), mode, batch, limb_begin, limbs,
                         _stream_ptr(x, stream)), "rescale")
    return out


class KeySwitchPlan:
    """Hybrid key-switch constants over a Q u P plan (see keyswitch_plan_create)."""

    def __init__(self, qp_plan: Plan, num_q: int, num_p: int, dnum: int):
        self.qp_plan = qp_plan  # keeps the device tables alive
        self.num_q, self.num_p, self.dnum = int(num_q), int(num_p), int(dnum)
        h = _VP()
        _check(lib().keyswitch_plan_create(ctypes.byref(h), qp_plan.handle, num_q, num_p, dnum),
               "keyswitch_plan_create")
        self._h = h

    @property
    def handle(self):
        if self._h is None:
            raise ValueError("plan destroyed")
        return self._h

    def workspace_bytes(self, batch: int = 1) -> int:
        v = ctypes.c_size_t()
        _check(lib().keyswitch_workspace_size(self.handle, batch, ctypes.byref(v)), "keyswitch_workspace_size")
        return int(v.value)

    def destroy(self):
        if getattr(self, "_h", None) is not None:
            lib().keyswitch_plan_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass


def workspace(ks: KeySwitchPlan, batch: int = 1):
    """A device workspace tensor (uint8) big enough for keyswitch on `batch` ciphertexts."""
    import torch
    nbytes = ks.workspace_bytes(batch)
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=f"cuda:{ks.qp_plan.device}")


def keyswitch(ks: KeySwitchPlan, out, ct, ksk, galois_elt: int, ws=None, stream=None):
    """Rotation key-switch; ct, out [batch, 2, num_q, n]; ksk [dnum, 2, num_q + num_p, n]."""
    plan = ks.qp_plan
    batch, limbs = _check_tensor(ct, plan, "ct", lead=1)
    _check_tensor(out, plan, "out", lead=1)
    _check_tensor(ksk, plan, "ksk", lead=1)
    if limbs != ks.num_q or ct.shape[-3] != 2 or out.shape != ct.shape:
        raise ValueError("ct/out must be [batch, 2, num_q, n]")
    if tuple(ksk.shape) != (ks.dnum, 2, ks.num_q + ks.num_p, plan.n):
        raise ValueError("ksk must be [dnum, 2, num_q + num_p, n]")
    if ws is None:
        with _on_stream(ct, stream):
            ws = workspace(ks, batch)
    _check(lib().keyswitch(ks.handle, _VP(out.data_ptr()), _VP(ct.data_ptr()), _VP(ksk.data_ptr()), galois_elt,
                           batch, _VP(ws.data_ptr()), ws.numel() * ws.element_size(), _stream_ptr(ct, stream)),
           "keyswitch")
    return out


def keyswitch_noalloc(ks: KeySwitchPlan, out, ct, ksk, galois_elt: int, stream=None):
    """keyswitch() with the library's static device workspace (allocates nothing; see
    keyswitch_noalloc in the header for its size limit and sharing rule)."""
    plan = ks.qp_plan
    batch, limbs = _check_tensor(ct, plan, "ct", lead=1)
    _check_tensor(out, plan, "out", lead=1)
    _check_tensor(ksk, plan, "ksk", lead=1)
    if limbs != ks.num_q or ct.shape[-3] != 2 or out.shape != ct.shape:
        raise ValueError("ct/out must be [batch, 2, num_q, n]")
    if tuple(ksk.shape) != (ks.dnum, 2, ks.num_q + ks.num_p, plan.n):
        raise ValueError("ksk must be [dnum, 2, num_q + num_p, n]")
    _check(lib().keyswitch_noalloc(ks.handle, _VP(out.data_ptr()), _VP(ct.data_ptr()), _VP(ksk.data_ptr()),
                                   galois_elt, batch, _stream_ptr(ct, stream)), "keyswitch_noalloc")
    return out


def hoisted_workspace(ks: KeySwitchPlan, num_rot: int, batch: int = 1):
    """A device workspace (uint8) for keyswitch_hoisted with num_rot rotations of `batch` ciphertexts."""
    import torch
    v = ctypes.c_size_t()
    _check(lib().keyswitch_hoisted_workspace_size(ks.handle, num_rot, batch, ctypes.byref(v)),
           "keyswitch_hoisted_workspace_size")
    return torch.empty(max(int(v.value), 1), dtype=torch.uint8, device=f"cuda:{ks.qp_plan.device}")


def keyswitch_hoisted(ks: KeySwitchPlan, out, ct, ksk, galois_elts, ws=None, stream=None):
    """Hoisted rotations; ct [batch, 2, num_q, n], ksk [R, dnum, 2, num_q + num_p, n] -> out [R, batch, 2, num_q, n]."""
    plan = ks.qp_plan
    batch, limbs = _check_tensor(ct, plan, "ct", lead=1)
    _check_tensor(out, plan, "out", lead=1)
    _check_tensor(ksk, plan, "ksk", lead=1)
    R = len(galois_elts)
    if limbs != ks.num_q or ct.dim() != 4 or ct.shape[1] != 2:
        raise ValueError("ct must be [batch, 2, num_q, n]")
    if tuple(out.shape) != (R,) + tuple(ct.shape):
        raise ValueError("out must be [R, batch, 2, num_q, n]")
    if tuple(ksk.shape) != (R, ks.dnum, 2, ks.num_q + ks.num_p, plan.n):
        raise ValueError("ksk must be [R, dnum, 2, num_q + num_p, n]")
    if ws is None:
        with _on_stream(ct, stream):
            ws = hoisted_workspace(ks, R, batch)
    _gs_arr, gs_ptr = _u64arr(galois_elts)
    _check(lib().keyswitch_hoisted(ks.handle, _VP(out.data_ptr()), _VP(ct.data_ptr()), _VP(ksk.data_ptr()),
                                   gs_ptr, R, batch, _VP(ws.data_ptr()),
                                   ws.numel() * ws.element_size(), _stream_ptr(ct, stream)), "keyswitch_hoisted")
    return out


def relinearize(ks: KeySwitchPlan, out, d, rlk, ws=None, stream=None):
    """Relinearisation; d [batch, 3, num_q, n] -> out [batch, 2, num_q, n]; rlk [dnum, 2, num_q + num_p, n]."""
    plan = ks.qp_plan
    batch, limbs = _check_tensor(d, plan, "d", lead=1)
    _check_tensor(out, plan, "out", lead=1)
    _check_tensor(rlk, plan, "rlk", lead=1)
    if limbs != ks.num_q or d.shape[-3] != 3:
        raise ValueError("d must be [batch, 3, num_q, n]")
    if tuple(out.shape) != tuple(d.shape[:-3]) + (2, ks.num_q, plan.n):
        raise ValueError("out must be [batch, 2, num_q, n]")
    if tuple(rlk.shape) != (ks.dnum, 2, ks.num_q + ks.num_p, plan.n):
        raise ValueError("rlk must be [dnum, 2, num_q + num_p, n]")
    if ws is None:
        with _on_stream(d, stream):
            ws = workspace(ks, batch)
    _check(lib().relinearize(ks.handle, _VP(out.data_ptr()), _VP(d.data_ptr()), _VP(rlk.data_ptr()), batch,
                             _VP(ws.data_ptr()), ws.numel() * ws.element_size(), _stream_ptr(d, stream)),
           "relinearize")
    return out


class ModRaisePlan:
    """Garner constants to lift from the first num_from primes of a plan to its first num_to."""

    def __init__(self, plan: Plan, num_from: int, num_to: int):
        self.plan = plan  # keeps the device tables alive
        self.num_from, self.num_to = int(num_from), int(num_to)
        h = _VP()
        _check(lib().modraise_plan_create(ctypes.byref(h), plan.handle, num_from, num_to), "modraise_plan_create")
        self._h = h

    @property
    def handle(self):
        if self._h is None:
            raise ValueError("plan destroyed")
        return self._h

    def destroy(self):
        if getattr(self, "_h", None) is not None:
            lib().modraise_plan_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass


def modraise(mr: ModRaisePlan, out, x, stream=None):
    """x [..., num_from, n] -> out [..., num_to, n] (exact lift onto the longer chain)."""
    batch, limbs = _check_tensor(x, mr.plan, "x")
    _check_tensor(out, mr.plan, "out")
    if limbs != mr.num_from or tuple(out.shape) != tuple(x.shape[:-2]) + (mr.num_to, mr.plan.n):
        raise ValueError("x must be [..., num_from, n] and out [..., num_to, n]")
    _check(lib().modraise(mr.handle, _VP(out.data_ptr()), _VP(x.data_ptr()), batch, _stream_ptr(x, stream)),
           "modraise")
    return out


def to_device(arr: np.ndarray, device="cuda:0"):
    """uint64 numpy array -> int64 torch tensor on the device (bit-identical)."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(arr).view(np.int64)).to(device)


def to_host(t) -> np.ndarray:
    """int64 torch tensor -> uint64 numpy array (bit-identical)."""
    return t.detach().cpu().numpy().view(np.uint64)
