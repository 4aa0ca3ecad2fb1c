"""Host-side checks of the C-ABI library: it loads, exports every symbol the
header declares, and its version, capability and error paths behave as the
header documents.  No compute call is made here (no GPU is needed)."""
import ctypes
import os
import re

import pytest

from linear_recurrence_scan_fma_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lrs_abi.h")


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(lrs_[a-z_0-9]+)\s*\(", src)))


def _header_int(name):
    src = open(HEADER).read()
    m = re.search(rf"#define {name}\s+\((\d+)u\s*<<\s*(\d+)\)", src)
    if m:
        return int(m.group(1)) << int(m.group(2))
    m = re.search(rf"\b{name}\s*=\s*(-?\d+)", src) or re.search(rf"#define {name}\s+\(?(\d+)", src)
    return int(m.group(1))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.LIB_PATH):
        pytest.fail("liblrs.so is not built (run __graft_entry__.build())")
    return binding.lib()


def test_exports_every_declared_symbol(lib):
    names = _declared_functions()
    assert len(names) == 21
    for n in names:
        assert hasattr(lib, n), f"{n} declared in lrs_abi.h but not exported"
    assert set(names) == set(binding.SIGNATURES), "binding and header disagree"


def test_python_mirrors_header_constants():
    for name in ("LRS_OK", "LRS_E_INVAL", "LRS_E_NOMEM", "LRS_E_UNSUPPORTED", "LRS_E_DEVICE",
                 "LRS_PARAM_ELEM_SCHEDULE", "LRS_ELEM_SCHEDULE_STREAM", "LRS_PARAM_LOOKBACK_DELAY_SEED",
                 "LRS_ELEM_SCHEDULE_LOOKBACK", "LRS_PARAM_DIAG_SEGMENTS", "LRS_PARAM_DELTA_SEGMENTS",
                 "LRS_CAP_SCAN_FMA",
                 "LRS_CAP_SCAN_GATED", "LRS_CAP_SCAN_DIAG_OUTER", "LRS_CAP_SCAN_DELTA",
                 "LRS_CAP_ELEM_BACKWARD", "LRS_CAP_ELEM_STEP", "LRS_CAP_SCAN_DELTA_DECAY",
                 "LRS_CAP_SCAN_DIAG_KEYSCALE", "LRS_CAP_SCAN_DIAG_EPILOGUE", "LRS_CAP_SCAN_DELTA_OUT",
                 "LRS_EPILOGUE_NONE",
                 "LRS_EPILOGUE_SKIP", "LRS_EPILOGUE_NORM_GATE", "LRS_DTYPE_F32", "LRS_DTYPE_BF16"):
        assert getattr(binding, name) == _header_int(name), name
    assert binding.LRS_ABI_VERSION_MAJOR == _header_int("LRS_ABI_VERSION_MAJOR")


def test_version_and_check(lib):
    v = binding.lrs_abi_version()
    assert v == (1 << 16) | (3 << 8) | 0
    assert binding.LRS_ABI_VERSION_MAJOR == 1
    assert binding.lrs_abi_check(1) == binding.LRS_OK
    assert binding.lrs_abi_check(2) == binding.LRS_E_UNSUPPORTED
    assert binding.lrs_abi_check(0) == binding.LRS_E_UNSUPPORTED


def test_caps_and_status_strings(lib):
    caps = binding.lrs_abi_caps()
    for bit in (binding.LRS_CAP_SCAN_FMA, binding.LRS_CAP_SCAN_GATED,
                binding.LRS_CAP_SCAN_DIAG_OUTER, binding.LRS_CAP_SCAN_DELTA,
                binding.LRS_CAP_ELEM_BACKWARD, binding.LRS_CAP_ELEM_STEP,
                binding.LRS_CAP_SCAN_DELTA_DECAY, binding.LRS_CAP_SCAN_DIAG_KEYSCALE,
                binding.LRS_CAP_SCAN_DIAG_EPILOGUE, binding.LRS_CAP_SCAN_DELTA_OUT):
        assert caps & bit
    for st in (0, -1, -2, -3, -4, -5, -6, 17, -99):
        s = binding.lrs_status_string(st)
        assert isinstance(s, str) and s
    assert binding.lrs_status_string(-1) == "invalid argument"


def test_null_context_and_null_out_are_rejected(lib):
    P = ctypes.c_void_p
    fake = P(0x1000)
    assert lib.lrs_scan_fma(None, fake, fake, None, fake, fake, 1, 1, 1, None) == binding.LRS_E_INVAL
    assert lib.lrs_scan_gated(None, fake, fake, None, fake, fake, 1, 1, 1, None) == binding.LRS_E_INVAL
    assert lib.lrs_scan_fma_backward(None, fake, None, fake, fake, None, fake, fake, None,
                                     1, 1, 1, None) == binding.LRS_E_INVAL
    assert lib.lrs_scan_gated_backward(None, fake, fake, None, fake, fake, None, fake, fake, None,
                                       1, 1, 1, None) == binding.LRS_E_INVAL
    assert lib.lrs_step_fma(None, fake, fake, fake, 1, 1, None) == binding.LRS_E_INVAL
    assert lib.lrs_scan_delta_decay(None, fake, fake, fake, fake, fake, 1.0, None, fake, fake,
                                    1, 1, 1, 1, 1, None) == binding.LRS_E_INVAL
    assert lib.lrs_scan_diag_outer_keyscale(None, fake, fake, fake, fake, fake, 1.0, None, fake, fake,
                                            1, 1, 1, 1, 1, 1, None) == binding.LRS_E_INVAL
    assert lib.lrs_scan_diag_outer_epilogue(None, fake, fake, fake, fake, 0, None, 1.0, None, 0, None, None,
                                            None, 0.0, 0, fake, fake, 1, 1, 1, 1, 1, 1,
                                            None) == binding.LRS_E_INVAL
    assert lib.lrs_step_gated(None, fake, fake, fake, 1, 1, None) == binding.LRS_E_INVAL
    assert lib.lrs_scan_delta_out(None, fake, fake, fake, None, fake, 1.0, None, 1, fake, fake,
                                  1, 1, 1, 1, 1, None) == binding.LRS_E_INVAL
    assert lib.lrs_context_create(0, None) == binding.LRS_E_INVAL
    assert lib.lrs_context_set_param(None, 1, 0) == binding.LRS_E_INVAL
    assert lib.lrs_context_check(None) == binding.LRS_E_INVAL
    lib.lrs_context_destroy(None)   # documented no-op


def test_context_create_without_gpu_is_unsupported(lib):
    import torch

    if torch.cuda.is_available():
        pytest.skip("a GPU is present; covered by the GPU tests")
    h = ctypes.c_void_p()
    assert lib.lrs_context_create(0, ctypes.byref(h)) == binding.LRS_E_UNSUPPORTED
    assert not h.value


def test_noalloc_entry_validates_before_any_hip_call(lib):
    """The allocation-free gated scan rejects bad arguments (LRS_E_INVAL) and
    shapes whose look-back words exceed its static scratch
    (LRS_E_UNSUPPORTED) on the host, before any HIP call: both paths run here
    without a GPU.  The pointers are never dereferenced."""
    P = ctypes.c_void_p
    fake = P(0x1000)
    f = lib.lrs_scan_gated_noalloc
    assert f(None, fake, None, fake, fake, 1, 1, 1, None) == binding.LRS_E_INVAL
    assert f(fake, fake, None, fake, fake, 0, 1, 1, None) == binding.LRS_E_INVAL
    gib = 1 << 36   # 64 GiB apart: the fake tensors below do not overlap
    a, u, s, fin = (P(gib * (i + 1)) for i in range(4))
    assert f(a, u, None, a, fin, 1, 64, 64, None) == binding.LRS_E_INVAL          # output aliases input
    assert f(a, P(gib + 2), None, s, fin, 1, 64, 64, None) == binding.LRS_E_INVAL  # misaligned u
    # 2^20 steps x 4096 channels: 8192 chunks x 64 channel tiles x 192 words
    # = 768 MiB of status words, beyond the 64 MiB scratch
    assert f(a, u, None, s, fin, 1, 1 << 20, 4096, None) == binding.LRS_E_UNSUPPORTED
    # the headline shape fits (48 MiB of words); not called here: it would launch
