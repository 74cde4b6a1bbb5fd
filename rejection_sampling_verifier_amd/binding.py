"""ctypes binding of libspecverify.so.

Argument marshalling only: every step of the verify computation runs in the
library's HIP kernels.  PyTorch provides device memory and the current
stream.  There is no fallback: when the library is missing or no GPU is
present, the calls raise.
"""

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libspecverify.so")

SV_F32, SV_BF16 = 0, 1
PROBE_POS, PROBE_ROW = 8, 4
STATUS = {0: "SV_OK", -1: "SV_EINVAL", -2: "SV_ESHAPE", -3: "SV_EDTYPE", -4: "SV_EHIP", -5: "SV_ENOMEM",
          -6: "SV_EALIGN", -7: "SV_ECAPTURE", -8: "SV_ETOOBIG"}
KERNEL_KINDS = ("stats", "topp", "rows", "smc", "produce")

EXPORTS = ("spec_verify", "spec_verify_noalloc", "spec_verify_probe", "spec_greedy_verify", "spec_hispec_verify", "spec_smc_step",
           "spec_draft_produce",
           "spec_verify_strerror",
           "spec_verify_release",
           "spec_verify_abi_version", "spec_verify_profile_enable", "spec_verify_profile_read",
           "spec_verify_stream_read")


class SvLogits(ctypes.Structure):
    _fields_ = [
        ("data", ctypes.c_void_p),
        ("dtype", ctypes.c_int32),
        ("B", ctypes.c_int32),
        ("P", ctypes.c_int32),
        ("V", ctypes.c_int32),
        ("stride_b", ctypes.c_int64),
        ("stride_p", ctypes.c_int64),
    ]


class SpecVerifyError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


_lib = None


def load(path=LIB_PATH):
    """Load the library once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m rejection_sampling_verifier_amd.build`")
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER
    lib.spec_verify.argtypes = [P(SvLogits), P(SvLogits), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_float,
                                ctypes.c_float, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    lib.spec_verify.restype = ctypes.c_int
    lib.spec_verify_noalloc.argtypes = lib.spec_verify.argtypes
    lib.spec_verify_noalloc.restype = ctypes.c_int
    lib.spec_verify_probe.argtypes = lib.spec_verify.argtypes[:9] + [ctypes.c_void_p] * 3
    lib.spec_verify_probe.restype = ctypes.c_int
    lib.spec_greedy_verify.argtypes = [P(SvLogits), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32] + \
        [ctypes.c_void_p] * 4
    lib.spec_greedy_verify.restype = ctypes.c_int
    lib.spec_hispec_verify.argtypes = [P(SvLogits)] * 3 + [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_float,
                                                            ctypes.c_float, ctypes.c_uint64] + [ctypes.c_void_p] * 4
    lib.spec_hispec_verify.restype = ctypes.c_int
    lib.spec_smc_step.argtypes = [P(SvLogits), P(SvLogits), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_float,
                                  ctypes.c_double, ctypes.c_uint64] + [ctypes.c_void_p] * 6
    lib.spec_smc_step.restype = ctypes.c_int
    lib.spec_draft_produce.argtypes = [P(SvLogits), ctypes.c_int32, ctypes.c_uint64, ctypes.c_void_p,
                                       ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
    lib.spec_draft_produce.restype = ctypes.c_int
    lib.spec_verify_strerror.argtypes = [ctypes.c_int]
    lib.spec_verify_strerror.restype = ctypes.c_char_p
    lib.spec_verify_release.argtypes = []
    lib.spec_verify_release.restype = None
    lib.spec_verify_abi_version.argtypes = []
    lib.spec_verify_abi_version.restype = ctypes.c_int
    lib.spec_verify_profile_enable.argtypes = [ctypes.c_int]
    lib.spec_verify_profile_enable.restype = ctypes.c_int
    lib.spec_verify_profile_read.argtypes = [P(ctypes.c_double), P(ctypes.c_int64), ctypes.c_int]
    lib.spec_verify_profile_read.restype = ctypes.c_int
    lib.spec_verify_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int,
                                            ctypes.c_void_p]
    lib.spec_verify_stream_read.restype = ctypes.c_int
    _lib = lib
    return lib


def _desc(t, name):
    if t.dim() != 3:
        raise ValueError(f"{name} must be [B, P, V]")
    if t.stride(2) != 1:
        raise ValueError(f"{name} must be contiguous along V")
    if t.dtype == torch.float32:
        dt = SV_F32
    elif t.dtype == torch.bfloat16:
        dt = SV_BF16
    else:
        raise ValueError(f"{name}: dtype {t.dtype} is not float32 or bfloat16")
    B, P, V = t.shape
    return SvLogits(t.data_ptr(), dt, B, P, V, t.stride(0), t.stride(1))


def _stream_handle(stream, device):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def _check(lib, rc):
    if rc < 0:
        raise SpecVerifyError(rc, lib.spec_verify_strerror(rc).decode())


def verify(target, draft, draft_tokens, draft_len=None, temperature=1.0, top_p=1.0, seed=0, *, stream=None,
           out_tokens=None, out_n_accepted=None, probe=False, noalloc=False):
    """The verify step on device tensors.

    target [B, K+1, V] and draft [B, K, V]: bfloat16 or float32, V contiguous.
    draft_tokens [B, K] int32 contiguous; draft_len [B] int32 or None.
    Returns (tokens [B, K+1] int32, n_accepted [B] int32), plus
    (probe_pos [B, K+1, 8], probe_row [B, 4]) float64 when probe is set.
    noalloc: call spec_verify_noalloc (no device allocation by the library;
    the caller passes out_tokens and out_n_accepted to allocate nothing at
    all).
    """
    lib = load()
    if draft_tokens.dtype != torch.int32 or not draft_tokens.is_contiguous():
        raise ValueError("draft_tokens must be contiguous int32")
    if draft_len is not None and (draft_len.dtype != torch.int32 or not draft_len.is_contiguous()):
        raise ValueError("draft_len must be contiguous int32")
    if noalloc and probe:
        raise ValueError("the no-allocation entry point has no probe")
    dev = target.device
    B, K1 = target.shape[0], target.shape[1]
    if out_tokens is None:
        out_tokens = torch.empty((B, K1), dtype=torch.int32, device=dev)
    if out_n_accepted is None:
        out_n_accepted = torch.empty((B,), dtype=torch.int32, device=dev)
    td, dd = _desc(target, "target"), _desc(draft, "draft")
    args = [ctypes.byref(td), ctypes.byref(dd), ctypes.c_void_p(draft_tokens.data_ptr()),
            ctypes.c_void_p(draft_len.data_ptr() if draft_len is not None else None),
            ctypes.c_float(temperature), ctypes.c_float(top_p), ctypes.c_uint64(int(seed) & (2 ** 64 - 1)),
            ctypes.c_void_p(out_tokens.data_ptr()), ctypes.c_void_p(out_n_accepted.data_ptr())]
    sh = _stream_handle(stream, dev)
    if probe:
        pp = torch.empty((B, K1, PROBE_POS), dtype=torch.float64, device=dev)
        pr = torch.empty((B, PROBE_ROW), dtype=torch.float64, device=dev)
        _check(lib, lib.spec_verify_probe(*args, ctypes.c_void_p(pp.data_ptr()), ctypes.c_void_p(pr.data_ptr()), sh))
        return out_tokens, out_n_accepted, pp, pr
    if noalloc:
        _check(lib, lib.spec_verify_noalloc(*args, sh))
    else:
        _check(lib, lib.spec_verify(*args, sh))
    return out_tokens, out_n_accepted


def greedy_verify(target, draft_tokens, draft_len=None, k=0, *, stream=None, out_tokens=None, out_n_accepted=None,
                  out_topk=None):
    """Greedy verify on device tensors: target [B, K+1, V] (bfloat16 or
    float32, V contiguous), draft_tokens [B, K] int32.  Returns (tokens
    [B, K+1] int32, n_accepted [B] int32, topk [B, k] int32)."""
    lib = load()
    if draft_tokens.dtype != torch.int32 or not draft_tokens.is_contiguous():
        raise ValueError("draft_tokens must be contiguous int32")
    if draft_len is not None and (draft_len.dtype != torch.int32 or not draft_len.is_contiguous()):
        raise ValueError("draft_len must be contiguous int32")
    dev = target.device
    B, K1 = target.shape[0], target.shape[1]
    if out_tokens is None:
        out_tokens = torch.empty((B, K1), dtype=torch.int32, device=dev)
    if out_n_accepted is None:
        out_n_accepted = torch.empty((B,), dtype=torch.int32, device=dev)
    if out_topk is None:
        out_topk = torch.empty((B, max(k, 1)), dtype=torch.int32, device=dev)
    td = _desc(target, "target")
    _check(lib, lib.spec_greedy_verify(ctypes.byref(td), ctypes.c_void_p(draft_tokens.data_ptr()),
                                       ctypes.c_void_p(draft_len.data_ptr() if draft_len is not None else None),
                                       ctypes.c_int32(k), ctypes.c_void_p(out_tokens.data_ptr()),
                                       ctypes.c_void_p(out_n_accepted.data_ptr()),
                                       ctypes.c_void_p(out_topk.data_ptr()), _stream_handle(stream, dev)))
    return out_tokens, out_n_accepted, out_topk[:, :k]


def draft_produce(target, K, seed=0, *, stream=None, out=None, out_tokens=None):
    """The synthetic draft producer on device tensors: target [B, P, V]
    (bfloat16 or float32, V contiguous), K <= P.  Returns (draft [B, K, V] of
    the target's dtype, tokens [B, K] int32); `out` may be any [B, K, V] view
    of that dtype with V contiguous."""
    lib = load()
    dev = target.device
    B, _, V = target.shape
    if out is None:
        out = torch.empty((B, K, V), dtype=target.dtype, device=dev)
    if out.dim() != 3 or tuple(out.shape) != (B, K, V) or out.dtype != target.dtype or out.stride(2) != 1:
        raise ValueError("out must be [B, K, V] of the target's dtype, contiguous along V")
    if out_tokens is None:
        out_tokens = torch.empty((B, K), dtype=torch.int32, device=dev)
    if out_tokens.dtype != torch.int32 or not out_tokens.is_contiguous() or tuple(out_tokens.shape) != (B, K):
        raise ValueError("out_tokens must be contiguous int32 [B, K]")
    td = _desc(target, "target")
    _check(lib, lib.spec_draft_produce(ctypes.byref(td), ctypes.c_int32(K), ctypes.c_uint64(seed & (2**64 - 1)),
                                       ctypes.c_void_p(out.data_ptr()), out.stride(0), out.stride(1),
                                       ctypes.c_void_p(out_tokens.data_ptr()), _stream_handle(stream, dev)))
    return out, out_tokens


def hispec_verify(final, inter, draft, draft_tokens, draft_len=None, temperature=1.0, top_p=1.0, seed=0, *,
                  stream=None, out_tokens=None, out_n_accepted=None, out_n_stage1=None):
    """The two-stage verify on device tensors: final [B, K+2, V], inter
    [B, K+1, V], draft [B, K, V] logits (same dtype, V contiguous).  Returns
    (tokens [B, K+2] int32, n_accepted [B] int32, n_stage1 [B] int32)."""
    lib = load()
    if draft_tokens.dtype != torch.int32 or not draft_tokens.is_contiguous():
        raise ValueError("draft_tokens must be contiguous int32")
    if draft_len is not None and (draft_len.dtype != torch.int32 or not draft_len.is_contiguous()):
        raise ValueError("draft_len must be contiguous int32")
    dev = final.device
    B, K2 = final.shape[0], final.shape[1]
    if out_tokens is None:
        out_tokens = torch.empty((B, K2), dtype=torch.int32, device=dev)
    if out_n_accepted is None:
        out_n_accepted = torch.empty((B,), dtype=torch.int32, device=dev)
    if out_n_stage1 is None:
        out_n_stage1 = torch.empty((B,), dtype=torch.int32, device=dev)
    fd, idd, dd = _desc(final, "final"), _desc(inter, "inter"), _desc(draft, "draft")
    _check(lib, lib.spec_hispec_verify(
        ctypes.byref(fd), ctypes.byref(idd), ctypes.byref(dd), ctypes.c_void_p(draft_tokens.data_ptr()),
        ctypes.c_void_p(draft_len.data_ptr() if draft_len is not None else None), ctypes.c_float(temperature),
        ctypes.c_float(top_p), ctypes.c_uint64(int(seed) & (2 ** 64 - 1)), ctypes.c_void_p(out_tokens.data_ptr()),
        ctypes.c_void_p(out_n_accepted.data_ptr()), ctypes.c_void_p(out_n_stage1.data_ptr()),
        _stream_handle(stream, dev)))
    return out_tokens, out_n_accepted, out_n_stage1


def smc_step(target, draft, draft_tokens, logw_in, temperature=1.0, ess_fraction=0.5, seed=0, *, stream=None,
             out_bonus=None, out_logw=None, out_ancestor=None):
    """One SMC-SD reweight-and-resample step on device tensors.

    target [N, K+1, V], draft [N, K, V]: bfloat16 or float32, V contiguous;
    draft_tokens [N, K] int32 contiguous; logw_in [N] float64 contiguous.
    Returns (bonus [N] int32, logw [N] float64, ancestor [N] int32,
    ess [1] float64, resampled [1] int32), all on the device.
    """
    lib = load()
    if draft_tokens.dtype != torch.int32 or not draft_tokens.is_contiguous():
        raise ValueError("draft_tokens must be contiguous int32")
    if logw_in.dtype != torch.float64 or not logw_in.is_contiguous():
        raise ValueError("logw_in must be contiguous float64")
    dev = target.device
    N = target.shape[0]
    if out_bonus is None:
        out_bonus = torch.empty((N,), dtype=torch.int32, device=dev)
    if out_logw is None:
        out_logw = torch.empty((N,), dtype=torch.float64, device=dev)
    if out_ancestor is None:
        out_ancestor = torch.empty((N,), dtype=torch.int32, device=dev)
    ess = torch.empty((1,), dtype=torch.float64, device=dev)
    resampled = torch.empty((1,), dtype=torch.int32, device=dev)
    td, dd = _desc(target, "target"), _desc(draft, "draft")
    _check(lib, lib.spec_smc_step(ctypes.byref(td), ctypes.byref(dd), ctypes.c_void_p(draft_tokens.data_ptr()),
                                  ctypes.c_void_p(logw_in.data_ptr()), ctypes.c_float(temperature),
                                  ctypes.c_double(ess_fraction), ctypes.c_uint64(int(seed) & (2 ** 64 - 1)),
                                  ctypes.c_void_p(out_bonus.data_ptr()), ctypes.c_void_p(out_logw.data_ptr()),
                                  ctypes.c_void_p(out_ancestor.data_ptr()), ctypes.c_void_p(ess.data_ptr()),
                                  ctypes.c_void_p(resampled.data_ptr()), _stream_handle(stream, dev)))
    return out_bonus, out_logw, out_ancestor, ess, resampled


def profile_enable(on=True):
    load().spec_verify_profile_enable(1 if on else 0)


def profile_read():
    """{kind: (summed ms, launches)} since the previous read (synchronises)."""
    lib = load()
    n = len(KERNEL_KINDS)
    ms = (ctypes.c_double * n)()
    cnt = (ctypes.c_int64 * n)()
    rc = lib.spec_verify_profile_read(ms, cnt, n)
    _check(lib, rc)
    return {KERNEL_KINDS[i]: (ms[i], cnt[i]) for i in range(n)}


def release():
    load().spec_verify_release()


def stream_read(buf, sink, unroll=4, stream=None):
    """Launch the streaming-read calibration kernel over a device tensor."""
    lib = load()
    sh = _stream_handle(stream, buf.device)
    _check(lib, lib.spec_verify_stream_read(ctypes.c_void_p(buf.data_ptr()), buf.numel() * buf.element_size(),
                                            ctypes.c_void_p(sink.data_ptr()), unroll, sh))
