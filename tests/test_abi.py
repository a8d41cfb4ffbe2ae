"""The C-ABI library (CPU only, no compute calls): it loads, exports every
symbol include/sd_verify.h declares, and rejects bad host-side arguments
synchronously, before anything is enqueued."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sd_verify.h")


def _declared():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(sd_[a-z_0-9]+)\s*\(", txt)))


def test_header_declares_the_entry_points():
    names = _declared()
    for n in ("sd_verify_sample", "sd_verify_greedy", "sd_verify_workspace_bytes",
              "sd_strerror", "sd_debug_process_rows", "sd_debug_uniforms"):
        assert n in names


def test_library_loads_and_exports_every_declared_symbol():
    import speculative_sampling_verify_temp_amd as sdv
    lib = ctypes.CDLL(sdv.LIB_PATH)
    for n in _declared():
        assert hasattr(lib, n), n


def test_strerror_and_workspace_size_on_host():
    import speculative_sampling_verify_temp_amd as sdv
    assert sdv.strerror(0) == "ok"
    assert "invalid" in sdv.strerror(-1)
    a = sdv.SdVerifyArgs()
    a.B, a.K_max, a.V, a.dtype = 256, 8, 152064, sdv.SD_BF16
    n = sdv.workspace_bytes(a)
    assert n > 256 * 17 * 32
    a.K_max = 99
    with pytest.raises(sdv.SdVerifyError):
        sdv.workspace_bytes(a)


def _good_args(sdv):
    a = sdv.SdVerifyArgs()
    a.target_logits = 0x100000
    a.draft_logits = 0x200000
    a.ld_target = a.ld_draft = 1024
    a.dtype = sdv.SD_BF16
    a.B, a.K_max, a.V = 2, 3, 1000
    a.draft_ids = 0x300000
    a.top_p, a.rep_penalty, a.tv_budget = 0.9, 1.1, 0.5
    return a


@pytest.mark.parametrize("field,value,code", [
    ("B", 0, -1), ("V", 0, -1), ("K_max", -1, -1), ("K_max", 33, -4),
    ("dtype", 7, -1), ("top_p", 0.0, -1), ("top_p", 1.5, -1), ("top_p", float("nan"), -1),
    ("rep_penalty", 0.0, -1), ("rep_penalty", float("inf"), -1),
    ("tv_budget", -0.1, -1), ("ld_target", 999, -1), ("ld_target", 1001, -1),
    ("target_logits", 0x100004, -1), ("draft_logits", None, -1), ("draft_ids", None, -1),
    ("flags", 4, -1), ("V", 1 << 20, -4),
])
def test_sample_rejects_bad_arguments_synchronously(field, value, code):
    import speculative_sampling_verify_temp_amd as sdv
    a = _good_args(sdv)
    setattr(a, field, value)
    out = ctypes.c_void_p(0x400000)
    rc = sdv.lib.sd_verify_sample(ctypes.byref(a), ctypes.c_void_p(0x500000), 1 << 30,
                                  out, out, None, None, None)
    assert rc == code


def test_sample_rejects_small_workspace_and_missing_outputs():
    import speculative_sampling_verify_temp_amd as sdv
    a = _good_args(sdv)
    out = ctypes.c_void_p(0x400000)
    assert sdv.lib.sd_verify_sample(ctypes.byref(a), ctypes.c_void_p(0x500000), 16,
                                    out, out, None, None, None) == sdv.SD_EWORKSPACE
    assert sdv.lib.sd_verify_sample(ctypes.byref(a), None, 1 << 30,
                                    out, out, None, None, None) == sdv.SD_EWORKSPACE
    assert sdv.lib.sd_verify_sample(ctypes.byref(a), ctypes.c_void_p(0x500000), 1 << 30,
                                    None, out, None, None, None) == sdv.SD_EINVAL


def test_greedy_ignores_sampling_only_fields():
    import speculative_sampling_verify_temp_amd as sdv
    a = _good_args(sdv)
    a.draft_logits = None
    a.top_p = 0.0          # ignored by greedy ...
    a.tv_budget = -1.0
    a.B = 0                # ... but B is still checked
    out = ctypes.c_void_p(0x400000)
    assert sdv.lib.sd_verify_greedy(ctypes.byref(a), ctypes.c_void_p(0x500000), 1 << 30,
                                    out, out, None, None, None) == sdv.SD_EINVAL


def test_phase_kernel_names_follow_the_path_choice():
    import speculative_sampling_verify_temp_amd as sdv
    a = _good_args(sdv)
    assert [sdv.phase_kernel(a, p) for p in range(3)] == \
        ["k_pair_fast", None, "k_fast_finalize"]   # (flagged units: exact route inside k_pair_fast)
    a.top_p = 1.0   # no truncation: general path; TV needed for 0 < D < 1
    assert [sdv.phase_kernel(a, p) for p in range(3)] == \
        ["k_row_prepare", "k_pair_tv", "k_finalize"]
    a.tv_budget = 0.0
    assert sdv.phase_kernel(a, 1) is None
    a.dtype, a.top_p = sdv.SD_F32, 0.9
    assert sdv.phase_kernel(a, 0) == "k_row_prepare"
    assert sdv.phase_kernel(a, 3) is None
    a.B = 0
    assert sdv.phase_kernel(a, 0) is None


def test_draft_confidence_rejects_bad_arguments_on_host():
    """Every call here fails a host-side check, so nothing is launched (the
    pointers are never dereferenced)."""
    import speculative_sampling_verify_temp_amd as sdv
    lib = ctypes.CDLL(sdv.LIB_PATH)
    f = lib.sd_draft_confidence
    P, I32 = ctypes.c_void_p, ctypes.c_int32
    f.argtypes = [P, I32, I32, I32, I32, ctypes.c_int64, P, ctypes.c_float, P, P, P]
    f.restype = ctypes.c_int
    good, out = P(1 << 20), P(1 << 21)
    cases = [
        (None, sdv.SD_BF16, 2, 3, 64, 64, None, 0.6, out),          # no logits
        (good, sdv.SD_BF16, 2, 3, 64, 64, None, 0.6, None),         # no top-1 output
        (P((1 << 20) + 8), sdv.SD_BF16, 2, 3, 64, 64, None, 0.6, out),   # misaligned rows
        (good, sdv.SD_BF16, 2, 3, 64, 60, None, 0.6, out),          # ld < V
        (good, sdv.SD_BF16, 2, 3, 60, 60, None, 0.6, out),          # ld * 2 not a 16-byte multiple
        (good, 7, 2, 3, 64, 64, None, 0.6, out),                    # unknown dtype
        (good, sdv.SD_F32, 0, 3, 64, 64, None, 0.6, out),           # B < 1
        (good, sdv.SD_F32, 2, 0, 64, 64, None, 0.6, out),           # K_max < 1
        (good, sdv.SD_F32, 2, 3, 0, 64, None, 0.6, out),            # V < 1
        (good, sdv.SD_F32, 2, 3, 64, 64, None, float("nan"), out),  # NaN threshold
    ]
    for c in cases:
        assert f(*c, None, None) == -1, c   # SD_EINVAL


def test_args_struct_matches_the_header():
    """The ctypes mirror has every field of the C struct at the offset a C
    compiler gives it, and the same size (the header compiled here by gcc)."""
    import shutil
    import subprocess
    import tempfile
    import speculative_sampling_verify_temp_amd as sdv
    A = sdv.SdVerifyArgs
    names = [f[0] for f in A._fields_]
    assert names[-3:] == ["top_p_per_row", "tv_budget_per_row", "V_draft"]
    gcc = shutil.which("gcc") or shutil.which("cc")
    if gcc is None:
        pytest.skip("no C compiler")
    src = "#include <stdio.h>\n#include <stddef.h>\n#include \"sd_verify.h\"\nint main(void){" + \
        "printf(\"%zu\", sizeof(sd_verify_args_t));" + "".join(
            f'printf(" %zu", offsetof(sd_verify_args_t, {n}));' for n in names) + "return 0;}\n"
    with tempfile.TemporaryDirectory() as d:
        c, exe = os.path.join(d, "t.c"), os.path.join(d, "t")
        open(c, "w").write(src)
        subprocess.run([gcc, "-I", os.path.dirname(HEADER), c, "-o", exe], check=True)
        got = [int(v) for v in subprocess.run([exe], capture_output=True, text=True,
                                               check=True).stdout.split()]
    assert got[0] == ctypes.sizeof(A)
    assert got[1:] == [getattr(A, n).offset for n in names]


def test_draft_vocabulary_checked_on_host():
    """V_draft in [0, V] (0 = V) and ld_draft >= V_draft pass the host checks
    (the call then stops at the too-small workspace, SD_EWORKSPACE); other
    values fail them (SD_EINVAL).  Nothing is launched either way."""
    import speculative_sampling_verify_temp_amd as sdv
    out = ctypes.c_void_p(0x400000)
    for vd, ld, code in ((0, 1024, -2), (999, 1000, -2), (600, 600, -2), (1000, 1000, -2),
                         (1001, 1024, -1), (-1, 1024, -1), (600, 592, -1), (0, 992, -1)):
        a = _good_args(sdv)
        a.V_draft, a.ld_draft = vd, ld
        rc = sdv.lib.sd_verify_sample(ctypes.byref(a), ctypes.c_void_p(0x500000), 16,
                                      out, out, None, None, None)
        assert rc == code, (vd, ld)


def test_noalloc_rejects_on_host_before_touching_the_device():
    """sd_verify_sample_noalloc checks its arguments, then whether the call
    fits the built-in scratch array (SD_ESCRATCH), before it looks up the
    array or enqueues anything."""
    import speculative_sampling_verify_temp_amd as sdv
    f = sdv.lib.sd_verify_sample_noalloc
    out = ctypes.c_void_p(0x400000)
    a = _good_args(sdv)
    a.B = 0
    assert f(ctypes.byref(a), out, out, None, None, None) == sdv.SD_EINVAL
    a = _good_args(sdv)
    assert f(ctypes.byref(a), None, out, None, None, None) == sdv.SD_EINVAL
    a.B = 100000   # about 40 MiB of workspace
    assert sdv.workspace_bytes(a) > sdv.SD_NOALLOC_MAX_WORKSPACE
    assert f(ctypes.byref(a), out, out, None, None, None) == sdv.SD_ESCRATCH
    assert "scratch" in sdv.strerror(sdv.SD_ESCRATCH)


def _lm_args(sdv, B, K, H):
    a = sdv.SdLmHeadArgs()
    a.target_hidden, a.target_weight = 0x100000, 0x200000
    a.draft_hidden, a.draft_weight = 0x300000, 0x400000
    a.draft_ids = 0x500000
    a.H_target = a.H_draft = H
    a.B, a.K_max, a.V = B, K, 1000
    return a


def test_lmhead_rejects_bad_arguments_on_host():
    """Every check of the LM-head calls runs on the host before any work is
    enqueued: hidden sizes that are not multiples of 64, misaligned pointers,
    and hidden-state arrays of 2 GiB or more (the tile engine addresses them
    by 32-bit byte offsets)."""
    import speculative_sampling_verify_temp_amd as sdv
    lib = sdv.lib
    acc = (ctypes.c_int32 * 1)()
    call = lambda a: lib.sd_lmhead_verify_sample(ctypes.byref(a), None, 0, acc, acc, None, None, None)
    assert call(_lm_args(sdv, 4, 2, 96)) == -1                # H not a multiple of 64
    a = _lm_args(sdv, 4, 2, 128)
    a.target_weight += 8
    assert call(a) == -1                                       # misaligned
    assert call(_lm_args(sdv, 4, 2, 128)) == sdv.SD_EWORKSPACE   # passes the checks
    big = 1 << 20   # B (K + 1) H 2 bytes: 2^20 * 3 * 1024 * 2 > 2^31
    assert call(_lm_args(sdv, big, 2, 1024)) == -4
    a = _lm_args(sdv, 1 << 18, 2, 1024)   # target 1.5 GiB, draft 1 GiB: fits
    assert call(a) == sdv.SD_EWORKSPACE
    a.H_draft = 4096                      # draft 4 GiB
    assert call(a) == -4
