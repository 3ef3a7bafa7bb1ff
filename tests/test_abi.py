"""CPU checks of the C-ABI library: it loads, exports every entry point that
include/tq.h declares, and its host-side logic (codebook solver, rotation
signs, slot arithmetic, argument validation) agrees with the oracle and the
pages.  No device compute is called here.
"""

import os
import re

import numpy as np
import pytest

from conftest import ROOT, load_golden
from oracle import codebook as cb
from oracle import layout, rotation
from packed_cache_decode_amd import _lib


def _header_functions(name="tq.h"):
    src = open(os.path.join(ROOT, "include", name)).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(tq_[a-z_0-9]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib(request):
    return _lib.load(request.config.getoption("--tq-lib"))


def test_exports_every_declared_symbol(lib):
    names = _header_functions()
    assert len(names) >= 12
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(_lib.EXPORTS) == names
    probes = _header_functions("tq_probe.h")
    for n in probes:
        assert hasattr(lib, n), n
    assert sorted(_lib.PROBE_EXPORTS) == probes
    headers = sorted(f for f in os.listdir(os.path.join(ROOT, "include")) if f.endswith(".h"))
    assert headers == ["tq.h", "tq_probe.h"]


def test_probe_argument_checks(lib):
    assert lib.tq_probe_sink_words(1000) == -1
    assert lib.tq_probe_sink_words(1 << 30) == 2048 * 256
    assert lib.tq_probe_read(0, None, 1 << 20, None, None) == -1
    assert lib.tq_probe_read(7, 16, 1 << 20, 16, None) == -1
    assert lib.tq_probe_read(0, 8, 1 << 20, 16, None) == -3


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
@pytest.mark.parametrize("d", [64, 128, 256])
def test_host_codebook_bit_identical_to_oracle(lib, d, bits):
    c, m = _lib.tq_host_codebook(d, bits, "exact")
    oc, om = cb.codebook(d, bits, "exact")
    assert np.array_equal(c.view(np.uint32), oc.view(np.uint32))
    assert np.array_equal(m.view(np.uint32), om.view(np.uint32))


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
@pytest.mark.parametrize("d", [64, 128, 256])
def test_host_beta_codebook_bit_identical_to_oracle(lib, d, bits):
    # the host solves with Gauss-Legendre quadrature, the oracle with the
    # incomplete Beta function and a closed-form first moment
    c, m = _lib.tq_host_codebook(d, bits, "beta")
    oc, om = cb.codebook(d, bits, "beta")
    assert np.array_equal(c.view(np.uint32), oc.view(np.uint32))
    assert np.array_equal(m.view(np.uint32), om.view(np.uint32))


@pytest.mark.parametrize("seed,d", [(0, 64), (7, 128), (2 ** 63 + 5, 256)])
def test_host_haar_matrix_matches_oracle(lib, seed, d):
    # the host's own Householder QR against the oracle's library QR of the same
    # Gaussian matrix: equal after float32 rounding, up to rare last-bit cases
    from oracle import haar
    q = _lib.tq_host_haar_matrix(seed, d)
    oq = haar.haar_matrix_f32(seed, d)
    ulps = np.abs(q.view(np.int32).astype(np.int64) - oq.view(np.int32).astype(np.int64))
    assert ulps.max() <= 1
    assert (ulps > 0).mean() < 1e-3


@pytest.mark.parametrize("bits", [3, 4])
def test_host_page_trapz_codebook_bit_identical_to_oracle(lib, bits):
    c, m = _lib.tq_host_codebook(128, bits, "page_trapz")
    oc, om = cb.codebook(128, bits, "page_trapz")
    assert np.array_equal(c.view(np.uint32), oc.view(np.uint32))
    assert np.array_equal(m.view(np.uint32), om.view(np.uint32))


@pytest.mark.parametrize("seed,flip", [(0, 1), (1234567, 1), (2 ** 64 - 1, 1), (5, 0)])
@pytest.mark.parametrize("d", [64, 128, 256])
def test_host_signs_match_oracle(lib, seed, flip, d):
    assert np.array_equal(_lib.tq_host_rotation_signs(seed, d, flip),
                          rotation.rotation_signs(seed, d, bool(flip)))


def test_host_slot_bytes(lib):
    g = load_golden("slot_sizes.json")
    for name in ("turboquant_k8v4", "turboquant_4bit_nc", "turboquant_k3v4_nc", "turboquant_3bit_nc"):
        assert _lib.tq_host_slot_bytes(name, 128) == g["presets"][name]["slot_aligned"]
        for d in (64, 256):
            assert _lib.tq_host_slot_bytes(name, d) == layout.slot_layout(name, d).slot_size_aligned
    assert _lib.tq_host_slot_bytes(1, 96) == -1
    assert _lib.tq_host_slot_bytes(7, 128) == -1


def test_host_argument_errors(lib):
    c = np.zeros(16, np.float32)
    assert lib.tq_host_codebook(96, 4, 0, c.ctypes.data, c.ctypes.data) == -2
    assert lib.tq_host_codebook(128, 5, 0, c.ctypes.data, c.ctypes.data) == -2
    assert lib.tq_host_codebook(128, 4, 9, c.ctypes.data, c.ctypes.data) == -1
    assert lib.tq_host_codebook(128, 4, 0, None, c.ctypes.data) == -1
    assert lib.tq_host_rotation_signs(1, 128, 1, None) == -1
    assert _lib.tq_status_str(-4) == "workspace too small"
    assert _lib.tq_status_str(0) == "ok"


def test_null_context_paths(lib):
    # argument checks run before any device work
    assert lib.tq_slot_bytes(None) == -1
    assert lib.tq_cache_bytes(None, 4) == -1
    assert lib.tq_destroy(None) == 0
    assert lib.tq_store(None, None, None, 0, None, 0, None, 0, None) == -1
    assert lib.tq_decode(None, None, None, 0, None, 0, None, 0, 1, 0, 0.0, None, 0, None, 0, None) == -1
    assert lib.tq_decode_workspace_bytes(None, 1, 1, 1) == 0


def test_init_rejects_bad_arguments_before_touching_a_device(lib):
    h = _lib._vp()
    import ctypes
    bad = [(9, 128, 8, 16, 0), (1, 96, 8, 16, 0), (1, 128, 0, 16, 0), (1, 128, 8, 24, 0),
           (1, 128, 8, 16, 5)]
    want = [-1, -2, -1, -2, -1]
    for (p, d, H, bs, mode), w in zip(bad, want):
        assert lib.tq_codebook_init(ctypes.byref(h), p, d, H, bs, 0, 1, mode, None) == w


def test_decode_option_calls_reject_a_null_context(lib):
    import ctypes
    o = _lib.DecodeOptions(0, 0, 0, 0)
    assert lib.tq_set_decode_options(None, ctypes.byref(o)) == -1
    assert lib.tq_get_decode_options(None, ctypes.byref(o)) == -1
    code = _lib._i32(0)
    assert lib.tq_get_device_error(None, ctypes.byref(code), 1, None) == -1


def test_library_reads_no_environment():
    # decode planning depends only on the call's arguments and the context's
    # options, never on the process environment
    csrc = os.path.join(ROOT, "packed_cache_decode_amd", "csrc")
    for name in os.listdir(csrc):
        src = open(os.path.join(csrc, name)).read()
        assert "getenv" not in src, name
