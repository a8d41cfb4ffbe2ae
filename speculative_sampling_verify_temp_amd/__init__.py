"""Speculative-sampling verify step on MI355X (gfx950): Python binding.

A thin ctypes layer over libsdverify.so (the C ABI in include/sd_verify.h).
It only marshals arguments: torch tensors provide device memory and the
current HIP stream; every step of the verify runs in the HIP kernels.  There
is no fallback: if the library is missing, importing this package raises.

Functions mirror the C entry points:
    verify_sample(...)   -> sd_verify_sample
    verify_sample_noalloc(...) -> sd_verify_sample_noalloc (outputs preallocated
                            by the caller, no workspace)
    verify_greedy(...)   -> sd_verify_greedy
    workspace_bytes(...) -> sd_verify_workspace_bytes
    strerror(code)       -> sd_strerror
    debug_process_rows(...), debug_uniforms(...)  (test exports)
"""
import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsdverify.so")

SD_OK, SD_EINVAL, SD_EWORKSPACE, SD_EHIP, SD_EUNSUPPORTED, SD_ESCRATCH = 0, -1, -2, -3, -4, -5
SD_NOALLOC_MAX_WORKSPACE = 8 << 20
SD_F32, SD_BF16 = 0, 1
SD_NO_BONUS, SD_PENALTY_PRIOR_ONLY = 1, 2
SD_ST_BAD_K, SD_ST_BAD_TEMP, SD_ST_BAD_DRAFT_ID, SD_ST_NONFINITE = 1, 2, 4, 8
SD_ST_BAD_PRIOR, SD_ST_Q_ZERO, SD_ST_RESID_ZERO = 16, 32, 64
SD_ST_BAD_PARAM = 1 << 7
SD_ST_INVALID_MASK = 0x8F
SD_NSTAT = 8
SD_MAX_K = 32
STAT_NAMES = ("d", "theta", "p_x", "q_x", "pi_x", "u", "v", "S")


class SdVerifyArgs(ctypes.Structure):
    _fields_ = [
        ("target_logits", ctypes.c_void_p),
        ("draft_logits", ctypes.c_void_p),
        ("ld_target", ctypes.c_int64),
        ("ld_draft", ctypes.c_int64),
        ("dtype", ctypes.c_int32),
        ("B", ctypes.c_int32),
        ("K_max", ctypes.c_int32),
        ("V", ctypes.c_int32),
        ("draft_ids", ctypes.c_void_p),
        ("k_per_row", ctypes.c_void_p),
        ("temperature", ctypes.c_void_p),
        ("top_p", ctypes.c_float),
        ("rep_penalty", ctypes.c_float),
        ("tv_budget", ctypes.c_float),
        ("prior_ids", ctypes.c_void_p),
        ("prior_offsets", ctypes.c_void_p),
        ("seed", ctypes.c_uint64),
        ("offset", ctypes.c_uint64),
        ("flags", ctypes.c_uint32),
        ("top_p_per_row", ctypes.c_void_p),
        ("tv_budget_per_row", ctypes.c_void_p),
        ("V_draft", ctypes.c_int32),
    ]


class SdLmHeadArgs(ctypes.Structure):
    _fields_ = [
        ("target_hidden", ctypes.c_void_p),
        ("draft_hidden", ctypes.c_void_p),
        ("target_weight", ctypes.c_void_p),
        ("draft_weight", ctypes.c_void_p),
        ("H_target", ctypes.c_int32),
        ("H_draft", ctypes.c_int32),
        ("B", ctypes.c_int32),
        ("K_max", ctypes.c_int32),
        ("V", ctypes.c_int32),
        ("V_draft", ctypes.c_int32),
        ("draft_ids", ctypes.c_void_p),
        ("k_per_row", ctypes.c_void_p),
        ("temperature", ctypes.c_void_p),
        ("tv_budget", ctypes.c_float),
        ("flags", ctypes.c_uint32),
        ("seed", ctypes.c_uint64),
        ("offset", ctypes.c_uint64),
    ]


class SdVerifyError(RuntimeError):
    def __init__(self, code, what):
        super().__init__(f"{what}: {strerror(code)} ({code})")
        self.code = code


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with "
            "`python speculative_sampling_verify_temp_amd/build.py` "
            "(there is no CPU fallback)")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    A = ctypes.POINTER(SdVerifyArgs)
    lib.sd_verify_workspace_bytes.argtypes = [A, ctypes.POINTER(SZ)]
    lib.sd_verify_workspace_bytes.restype = ctypes.c_int
    lib.sd_verify_sample.argtypes = [A, P, SZ, P, P, P, P, P]
    lib.sd_verify_sample.restype = ctypes.c_int
    lib.sd_verify_sample_noalloc.argtypes = [A, P, P, P, P, P]
    lib.sd_verify_sample_noalloc.restype = ctypes.c_int
    lib.sd_verify_greedy.argtypes = [A, P, SZ, P, P, P, P, P]
    lib.sd_verify_greedy.restype = ctypes.c_int
    lib.sd_strerror.argtypes = [ctypes.c_int]
    lib.sd_strerror.restype = ctypes.c_char_p
    lib.sd_debug_process_rows.argtypes = [A, P, SZ, P, P, P]
    lib.sd_debug_process_rows.restype = ctypes.c_int
    lib.sd_debug_run_phase.argtypes = [A, P, SZ, ctypes.c_int, P, P, P, P, P]
    lib.sd_debug_run_phase.restype = ctypes.c_int
    lib.sd_debug_phase_kernel.argtypes = [A, ctypes.c_int]
    lib.sd_debug_phase_kernel.restype = ctypes.c_char_p
    lib.sd_debug_fallback_units.argtypes = [A, P, SZ, ctypes.POINTER(I32), P, P]
    lib.sd_debug_fallback_units.restype = ctypes.c_int
    lib.sd_debug_uniforms.argtypes = [ctypes.c_uint64, ctypes.c_uint64, I32, I32, P, P, P]
    lib.sd_debug_uniforms.restype = ctypes.c_int
    lib.sd_draft_confidence.argtypes = [P, I32, I32, I32, I32, ctypes.c_int64, P, ctypes.c_float, P, P, P]
    lib.sd_draft_confidence.restype = ctypes.c_int
    L = ctypes.POINTER(SdLmHeadArgs)
    lib.sd_lmhead_workspace_bytes.argtypes = [L, ctypes.POINTER(SZ)]
    lib.sd_lmhead_workspace_bytes.restype = ctypes.c_int
    lib.sd_lmhead_verify_sample.argtypes = [L, P, SZ, P, P, P, P, P]
    lib.sd_lmhead_verify_sample.restype = ctypes.c_int
    lib.sd_lmhead_verify_greedy.argtypes = [L, P, SZ, P, P, P, P, P]
    lib.sd_lmhead_verify_greedy.restype = ctypes.c_int
    lib.sd_debug_lmhead_logits.argtypes = [L, P, SZ, P, P, P]
    lib.sd_debug_lmhead_logits.restype = ctypes.c_int
    return lib


lib = _load()


def strerror(code):
    return lib.sd_strerror(int(code)).decode()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dtype_code(t):
    import torch
    if t.dtype == torch.float32:
        return SD_F32
    if t.dtype in (torch.bfloat16, torch.int16, torch.uint16):
        return SD_BF16
    raise TypeError(f"logits must be float32 or bfloat16 (got {t.dtype})")


def _rows_ld(t, name):
    """[B][R][V] tensor with unit element stride and rows packed per request."""
    if t.dim() != 3 or t.stride(2) != 1 or (t.shape[0] > 1 and t.stride(0) != t.shape[1] * t.stride(1)):
        raise ValueError(f"{name} must be [B][rows][V] with rows laid out back to back")
    return t.stride(1) if t.shape[1] > 1 else max(t.stride(1), t.shape[2])


def make_args(target, draft, draft_ids, k_per_row=None, temperature=None, top_p=1.0,
              rep_penalty=1.0, prior_ids=None, prior_offsets=None, tv_budget=0.0,
              seed=0, offset=0, flags=0):
    """Fill the C argument struct from tensors (device pointers, strides)."""
    B, K1, V = target.shape
    a = SdVerifyArgs()
    a.target_logits = target.data_ptr()
    a.ld_target = _rows_ld(target, "target")
    a.dtype = _dtype_code(target)
    if draft is not None and draft.numel() > 0:
        if _dtype_code(draft) != a.dtype:
            raise TypeError("target and draft logits must share a dtype")
        a.draft_logits = draft.data_ptr()
        a.ld_draft = _rows_ld(draft, "draft")
        if draft.shape[2] > V:
            raise ValueError("draft rows longer than the target's vocabulary")
        a.V_draft = draft.shape[2]   # a shorter draft vocabulary: q = 0 past it
    else:
        a.draft_logits = None
        a.ld_draft = a.ld_target
    a.B, a.K_max, a.V = B, K1 - 1, V
    a.draft_ids = draft_ids.data_ptr() if draft_ids is not None and draft_ids.numel() else None
    a.k_per_row = None if k_per_row is None else k_per_row.data_ptr()
    a.temperature = None if temperature is None else temperature.data_ptr()
    # top_p and tv_budget: a float, or a [B] float32 device tensor of
    # per-request values (the scalar field is then unused)
    if hasattr(top_p, "data_ptr"):
        a.top_p, a.top_p_per_row = 1.0, top_p.data_ptr()
    else:
        a.top_p, a.top_p_per_row = float(top_p), None
    if hasattr(tv_budget, "data_ptr"):
        a.tv_budget, a.tv_budget_per_row = 0.0, tv_budget.data_ptr()
    else:
        a.tv_budget, a.tv_budget_per_row = float(tv_budget), None
    a.rep_penalty = float(rep_penalty)
    a.prior_ids = None if prior_ids is None else prior_ids.data_ptr()
    a.prior_offsets = None if prior_offsets is None else prior_offsets.data_ptr()
    a.seed = int(seed) & (2**64 - 1)
    a.offset = int(offset) & (2**64 - 1)
    a.flags = int(flags)
    return a


def workspace_bytes(args):
    n = ctypes.c_size_t()
    rc = lib.sd_verify_workspace_bytes(ctypes.byref(args), ctypes.byref(n))
    if rc != SD_OK:
        raise SdVerifyError(rc, "sd_verify_workspace_bytes")
    return n.value


def alloc_workspace(args, device):
    import torch
    return torch.zeros(max(1, workspace_bytes(args)), dtype=torch.uint8, device=device)


def verify_sample(target, draft, draft_ids, k_per_row=None, temperature=None, top_p=1.0,
                  rep_penalty=1.0, prior_ids=None, prior_offsets=None, tv_budget=0.0,
                  seed=0, offset=0, flags=0, stats=False, workspace=None, out=None,
                  stream=None):
    """Sampling verify on device tensors; returns (accepted, tokens, status, stats).

    out: optional dict of preallocated outputs (accepted, tokens, status, stats).
    """
    import torch
    args = make_args(target, draft, draft_ids, k_per_row, temperature, top_p, rep_penalty,
                     prior_ids, prior_offsets, tv_budget, seed, offset, flags)
    dev = target.device
    B, K1 = args.B, args.K_max + 1
    if workspace is None:
        workspace = alloc_workspace(args, dev)
    o = out or {}
    acc = o.get("accepted") if o.get("accepted") is not None else torch.empty(B, dtype=torch.int32, device=dev)
    tok = o.get("tokens") if o.get("tokens") is not None else torch.empty((B, K1), dtype=torch.int32, device=dev)
    st = o.get("status") if o.get("status") is not None else torch.empty(B, dtype=torch.int32, device=dev)
    sts = None
    if stats:
        sts = o.get("stats") if o.get("stats") is not None else torch.empty((B, K1, SD_NSTAT), dtype=torch.float32, device=dev)
    rc = lib.sd_verify_sample(ctypes.byref(args), _ptr(workspace), workspace.numel(),
                              _ptr(acc), _ptr(tok), _ptr(st), _ptr(sts), _stream(stream))
    if rc != SD_OK:
        raise SdVerifyError(rc, "sd_verify_sample")
    return acc, tok, st, sts


def verify_sample_noalloc(args, accepted, tokens, status=None, stats=None, stream=None):
    """sd_verify_sample_noalloc on a filled argument struct (make_args) and
    caller-allocated outputs: nothing is allocated, by this function or the
    library."""
    rc = lib.sd_verify_sample_noalloc(ctypes.byref(args), _ptr(accepted), _ptr(tokens),
                                      _ptr(status), _ptr(stats), _stream(stream))
    if rc != SD_OK:
        raise SdVerifyError(rc, "sd_verify_sample_noalloc")


def verify_greedy(target, draft_ids, k_per_row=None, rep_penalty=1.0, prior_ids=None,
                  prior_offsets=None, flags=0, workspace=None, argmax=False, out=None,
                  stream=None):
    """Greedy verify; returns (accepted, tokens, status, argmax or None)."""
    import torch
    args = make_args(target, None, draft_ids, k_per_row, None, 1.0, rep_penalty,
                     prior_ids, prior_offsets, 0.0, 0, 0, flags)
    dev = target.device
    B, K1 = args.B, args.K_max + 1
    if workspace is None:
        workspace = alloc_workspace(args, dev)
    o = out or {}
    acc = o.get("accepted") if o.get("accepted") is not None else torch.empty(B, dtype=torch.int32, device=dev)
    tok = o.get("tokens") if o.get("tokens") is not None else torch.empty((B, K1), dtype=torch.int32, device=dev)
    st = o.get("status") if o.get("status") is not None else torch.empty(B, dtype=torch.int32, device=dev)
    am = torch.empty((B, K1), dtype=torch.int32, device=dev) if argmax else None
    rc = lib.sd_verify_greedy(ctypes.byref(args), _ptr(workspace), workspace.numel(),
                              _ptr(acc), _ptr(tok), _ptr(st), _ptr(am), _stream(stream))
    if rc != SD_OK:
        raise SdVerifyError(rc, "sd_verify_greedy")
    return acc, tok, st, am


def debug_process_rows(target, draft, draft_ids, k_per_row=None, temperature=None, top_p=1.0,
                       rep_penalty=1.0, prior_ids=None, prior_offsets=None, flags=0,
                       stream=None):
    """Processed (penalized, tempered, truncated, renormalized) p and q rows."""
    import torch
    args = make_args(target, draft, draft_ids, k_per_row, temperature, top_p, rep_penalty,
                     prior_ids, prior_offsets, 0.0, 0, 0, flags)
    dev = target.device
    ws = alloc_workspace(args, dev)
    B, K1, V = target.shape
    p = torch.zeros((B, K1, V), dtype=torch.float32, device=dev)
    q = torch.zeros((B, max(K1 - 1, 0), V), dtype=torch.float32, device=dev)
    rc = lib.sd_debug_process_rows(ctypes.byref(args), _ptr(ws), ws.numel(), _ptr(p),
                                   _ptr(q) if q.numel() else None, _stream(stream))
    if rc != SD_OK:
        raise SdVerifyError(rc, "sd_debug_process_rows")
    return p, q


def run_phase(args, workspace, phase, accepted, tokens, status=None, stats=None,
              stream=None):
    """One phase (0, 1 or 2) of sd_verify_sample, for timing; phase_kernel names it."""
    rc = lib.sd_debug_run_phase(ctypes.byref(args), _ptr(workspace), workspace.numel(),
                                int(phase), _ptr(accepted), _ptr(tokens), _ptr(status),
                                _ptr(stats), _stream(stream))
    if rc != SD_OK:
        raise SdVerifyError(rc, "sd_debug_run_phase")


def phase_kernel(args, phase):
    """Name of the kernel run_phase launches for `phase` (None: no launch)."""
    name = lib.sd_debug_phase_kernel(ctypes.byref(args), int(phase))
    return name.decode() if name is not None else None


def fallback_units(args, workspace, stream=None, why=False):
    """After run_phase(..., 0, ...) on the single-pass path: how many units
    that phase settled by its exact route (and, with why=True, the reason
    bits per unit as a numpy array)."""
    import numpy as np
    n = ctypes.c_int32(0)
    nunits = args.B * (args.K_max + 1)
    w = np.zeros(nunits, dtype=np.uint32)
    rc = lib.sd_debug_fallback_units(ctypes.byref(args), _ptr(workspace), workspace.numel(),
                                     ctypes.byref(n), w.ctypes.data if why else None,
                                     _stream(stream))
    if rc != SD_OK:
        raise SdVerifyError(rc, "sd_debug_fallback_units")
    return (int(n.value), w) if why else int(n.value)


def debug_uniforms(seed, offset, B, npos, device="cuda", stream=None):
    import torch
    u = torch.empty((B, npos), dtype=torch.float32, device=device)
    v = torch.empty((B, npos), dtype=torch.float32, device=device)
    rc = lib.sd_debug_uniforms(int(seed) & (2**64 - 1), int(offset) & (2**64 - 1), B, npos,
                               _ptr(u), _ptr(v), _stream(stream))
    if rc != SD_OK:
        raise SdVerifyError(rc, "sd_debug_uniforms")
    return u, v


def draft_confidence(draft, temperature=None, threshold=0.6, stream=None, lengths=True):
    """Top-1 probability of each draft row and the early-stop draft length.

    draft: [B][K_max][V] float32 or bfloat16 device tensor (rows back to
    back); temperature: [B] float32 device tensor or None (T = 1).  Returns
    (top1 [B][K_max] float32, K [B] int32) from sd_draft_confidence; with
    lengths=False, K is None and only the row kernel runs."""
    import torch
    B, K, V = draft.shape
    ld = _rows_ld(draft, "draft")
    top1 = torch.empty((B, K), dtype=torch.float32, device=draft.device)
    kout = torch.empty(B, dtype=torch.int32, device=draft.device) if lengths else None
    rc = lib.sd_draft_confidence(_ptr(draft), _dtype_code(draft), B, K, V, ld,
                                 _ptr(temperature), float(threshold), _ptr(top1), _ptr(kout),
                                 _stream(stream))
    if rc != 0:
        raise SdVerifyError(rc, "sd_draft_confidence")
    return top1, kout


# ---------------------------------------------------------------------------
# Verify fed from hidden states through the LM heads (sd_lmhead_*).
# ---------------------------------------------------------------------------

def make_lmhead_args(target_hidden, target_weight, draft_ids, draft_hidden=None, draft_weight=None,
                     k_per_row=None, temperature=None, tv_budget=0.0, seed=0, offset=0, flags=0):
    """Fill sd_lmhead_args_t from bf16 device tensors: target_hidden
    [B][K_max+1][H_t], target_weight [V][H_t], draft_hidden [B][K_max][H_d],
    draft_weight [V_draft][H_d] (all contiguous)."""
    for t in (target_hidden, target_weight, draft_hidden, draft_weight):
        if t is not None and not t.is_contiguous():
            raise ValueError("LM-head tensors must be contiguous")
    a = SdLmHeadArgs()
    B, K1, Ht = target_hidden.shape
    a.target_hidden, a.target_weight = target_hidden.data_ptr(), target_weight.data_ptr()
    a.H_target, a.B, a.K_max, a.V = Ht, B, K1 - 1, target_weight.shape[0]
    if draft_hidden is not None:
        a.draft_hidden, a.draft_weight = draft_hidden.data_ptr(), draft_weight.data_ptr()
        a.H_draft, a.V_draft = draft_hidden.shape[2], draft_weight.shape[0]
    a.draft_ids = draft_ids.data_ptr() if draft_ids is not None and draft_ids.numel() else None
    a.k_per_row = None if k_per_row is None else k_per_row.data_ptr()
    a.temperature = None if temperature is None else temperature.data_ptr()
    a.tv_budget = float(tv_budget)
    a.flags = int(flags)
    a.seed = int(seed) & (2**64 - 1)
    a.offset = int(offset) & (2**64 - 1)
    return a


def lmhead_workspace(args, device):
    import torch
    n = ctypes.c_size_t()
    rc = lib.sd_lmhead_workspace_bytes(ctypes.byref(args), ctypes.byref(n))
    if rc != SD_OK:
        raise SdVerifyError(rc, "sd_lmhead_workspace_bytes")
    return torch.empty(max(1, n.value), dtype=torch.uint8, device=device)


def lmhead_verify_sample(args, accepted, tokens, status=None, stats=None, workspace=None,
                         stream=None):
    """sd_lmhead_verify_sample into caller-allocated outputs."""
    ws = lmhead_workspace(args, accepted.device) if workspace is None else workspace
    rc = lib.sd_lmhead_verify_sample(ctypes.byref(args), _ptr(ws), ws.numel(), _ptr(accepted),
                                     _ptr(tokens), _ptr(status), _ptr(stats), _stream(stream))
    if rc != SD_OK:
        raise SdVerifyError(rc, "sd_lmhead_verify_sample")


def lmhead_verify_greedy(args, accepted, tokens, status=None, argmax=None, workspace=None,
                         stream=None):
    """sd_lmhead_verify_greedy into caller-allocated outputs."""
    ws = lmhead_workspace(args, accepted.device) if workspace is None else workspace
    rc = lib.sd_lmhead_verify_greedy(ctypes.byref(args), _ptr(ws), ws.numel(), _ptr(accepted),
                                     _ptr(tokens), _ptr(status), _ptr(argmax), _stream(stream))
    if rc != SD_OK:
        raise SdVerifyError(rc, "sd_lmhead_verify_greedy")


def debug_lmhead_logits(args, out_target, out_draft=None, workspace=None, stream=None):
    """The LM-head logits of the used rows (test export)."""
    ws = lmhead_workspace(args, out_target.device) if workspace is None else workspace
    rc = lib.sd_debug_lmhead_logits(ctypes.byref(args), _ptr(ws), ws.numel(), _ptr(out_target),
                                    _ptr(out_draft), _stream(stream))
    if rc != SD_OK:
        raise SdVerifyError(rc, "sd_debug_lmhead_logits")
