"""C-ABI boundary tests that need no GPU: the library loads, exports every
function include/libmuon.h declares, its defaults equal the page's locked
values, and host-side validation rejects bad batches with the documented
status codes (nothing is enqueued; no device is touched)."""
import ctypes
import json
import os
import re

import pytest

import muon_newton_schulz_update_amd as mu
from muon_newton_schulz_update_amd import MuonMatrix

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "libmuon.h")
PAGE = json.load(open(os.path.join(ROOT, "tests", "golden", "page_constants.json")))

OK, INVALID, DTYPE, SHAPE = 0, -1, -2, -3


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"\b([a-z_][a-z0-9_]*)\s*\([^;{]*\)\s*;", text)
    return sorted(set(n for n in names if n not in ("if", "sizeof")))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(mu.library_path()):
        pytest.skip("libmuon.so not built")
    return mu.load_library()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert {"ns_polar", "aurora_orthogonalize", "muon_update", "muon_create"} <= set(names)
    for n in names:
        assert hasattr(lib, n), f"libmuon.so does not export {n}"


def test_defaults_equal_page_values(lib):
    c = mu.default_config()
    assert c.ns_steps == PAGE["ns"]["steps"]
    assert (c.ns_a, c.ns_b, c.ns_c) == (PAGE["ns"]["a"], PAGE["ns"]["b"], PAGE["ns"]["c"])
    assert c.ns_eps == pytest.approx(PAGE["ns"]["norm_eps"], rel=1e-6)
    assert c.pp_iterations == PAGE["table"]["pp_iterations"]
    assert c.pp_beta == PAGE["table"]["pp_beta"]
    assert c.pp_eps == pytest.approx(PAGE["aurora_signature"]["eps"], rel=1e-6)
    assert c.mu == pytest.approx(PAGE["muon_update_signature"]["mu"], rel=1e-7)
    assert c.nesterov == 1
    assert c.power_steps == PAGE["power_steps"]
    assert c.contra == pytest.approx(PAGE["contra"], rel=1e-7)
    assert c.target_uw == pytest.approx(PAGE["target_uw"], rel=1e-7)
    assert c.lr == pytest.approx(PAGE["table"]["lr"], rel=1e-7)
    assert c.flags == 0


def test_status_strings(lib):
    for code, name in mu.STATUS.items():
        assert lib.muon_status_string(code).decode() == name
    assert lib.muon_version().decode().count(".") == 2


FAKE = 0x10000  # never dereferenced: validation is host-only
_fresh = [1 << 40]


def m(rows, cols, dtype=1, ld=None, ptr="fresh"):
    """A descriptor; by default at an address of its own, 64 GiB from any other."""
    if ptr == "fresh":
        ptr = _fresh[0]
        _fresh[0] += 1 << 36
    return MuonMatrix(ptr, rows, cols, cols if ld is None else ld, dtype)


def test_valid_batch_passes(lib):
    g = [m(4, 8), m(16, 3, 0), m(0, 5)]
    mom = [m(4, 8, 0), m(16, 3, 0), m(0, 5, 0)]
    rc, msg = mu.check_update_args(g, mom, [m(4, 8), MuonMatrix(None, 0, 0, 0, 0), m(0, 5)], None)
    assert rc == OK, msg
    assert mu.check_update_args([], [], None, None)[0] == OK


@pytest.mark.parametrize("case,code", [
    ("null_ptr", INVALID), ("ld_lt_cols", SHAPE), ("bad_dtype", DTYPE), ("mom_bf16", DTYPE),
    ("shape_mismatch", SHAPE), ("weight_mismatch", SHAPE), ("out_mismatch", SHAPE),
    ("negative", SHAPE), ("too_big", SHAPE), ("short_too_big", SHAPE), ("misaligned", INVALID),
    ("ld_too_big", SHAPE),
])
def test_update_validation(lib, case, code):
    g, mom, w, uo = [m(4, 8)], [m(4, 8, 0)], None, None
    if case == "null_ptr":
        g = [m(4, 8, ptr=None)]
    elif case == "ld_lt_cols":
        g = [m(4, 8, ld=7)]
    elif case == "bad_dtype":
        g = [m(4, 8, dtype=7)]
    elif case == "mom_bf16":
        mom = [m(4, 8, 1)]
    elif case == "shape_mismatch":
        mom = [m(4, 9, 0)]
    elif case == "weight_mismatch":
        w = [m(8, 4)]
    elif case == "out_mismatch":
        uo = [m(4, 7, 0)]
    elif case == "negative":
        g, mom = [m(-1, 8)], [m(-1, 8, 0)]
    elif case == "too_big":
        g, mom = [m(4, 70000)], [m(4, 70000, 0)]
    elif case == "short_too_big":
        g, mom = [m(20000, 20000)], [m(20000, 20000, 0)]
    elif case == "misaligned":
        g = [m(4, 8, ptr=FAKE + 1)]
    elif case == "ld_too_big":
        g = [m(4, 8, ld=(1 << 40) + 1)]
    rc, msg = mu.check_update_args(g, mom, w, uo)
    assert rc == code, (case, rc, msg)
    assert msg


@pytest.mark.parametrize("field,value", [
    ("ns_steps", 0), ("ns_steps", 65), ("pp_iterations", -1), ("pp_iterations", 9),
    ("mu", 1.5), ("mu", -0.1), ("nesterov", 2), ("power_steps", 0), ("pp_eps", 0.0),
    ("target_uw", -1.0), ("flags", 16), ("flags", 0x80000000), ("lr", float("nan")), ("ns_a", float("inf")),
])
def test_config_validation(lib, field, value):
    cfg = mu.default_config()
    setattr(cfg, field, value)
    rc, msg = mu.check_update_args([m(4, 8)], [m(4, 8, 0)], None, None, cfg)
    assert rc == INVALID, (field, value, rc, msg)


@pytest.mark.parametrize("rows,cols,code", [
    (16384, 65536, OK), (65536, 16384, OK), (1, 65536, OK), (65536, 1, OK),
    (16385, 65536, SHAPE), (16384, 65537, SHAPE), (65537, 1, SHAPE), (16385, 16385, SHAPE),
])
def test_size_limits_at_the_boundary(lib, rows, cols, code):
    rc, msg = mu.check_update_args([m(rows, cols)], [m(rows, cols, 0)], None, None)
    assert rc == code, (rows, cols, rc, msg)
    rc, msg = mu.check_polar_args([m(rows, cols)], [m(rows, cols)])
    assert rc == code, (rows, cols, rc, msg)


def test_polar_validation(lib):
    assert mu.check_polar_args([m(5, 3)], [m(5, 3, 0)])[0] == OK
    assert mu.check_polar_args([m(5, 3)], [m(3, 5)])[0] == SHAPE
    assert mu.check_polar_args([m(5, 3)], [m(5, 3, 9)])[0] == DTYPE
    assert mu.check_polar_args([m(5, 3, ptr=None)], [m(5, 3)])[0] == INVALID


BASE = 1 << 62   # far above every fresh address


def at(off, rows, cols, ld, dtype=0):
    """A descriptor at byte offset `off` of one parent allocation."""
    return MuonMatrix(BASE + off, rows, cols, ld, dtype)


@pytest.mark.parametrize("case,code", [
    ("grad_is_momentum", INVALID), ("weight_is_grad", INVALID), ("out_is_grad", INVALID),
    ("momentum_meets_other_weight", INVALID), ("out_meets_other_momentum", INVALID),
    ("column_slices", OK), ("column_slices_one_shared", INVALID),
    ("wraps_into_next_row", INVALID), ("ends_at_last_row", OK),
    ("strides_differ_interleaved", OK), ("strides_differ_meet", INVALID),
    ("grads_share", OK), ("bf16_out_inside_f32_gap", OK),
])
def test_update_buffer_overlap(lib, case, code):
    """Buffers the call writes must share no element with any other buffer;
    the check is exact per element, so slices of one parent are allowed."""
    g, mom, w, uo = [m(4, 8, 0), m(4, 8, 0)], [m(4, 8, 0), m(4, 8, 0)], None, None
    if case == "grad_is_momentum":
        mom[1] = g[1]
    elif case == "weight_is_grad":
        w = [m(4, 8, 0), g[0]]
    elif case == "out_is_grad":
        uo = [g[1], MuonMatrix(None, 0, 0, 0, 0)]
    elif case == "momentum_meets_other_weight":
        w = [m(4, 8, 0), mom[0]]
    elif case == "out_meets_other_momentum":
        # update_out[0] starts inside momentum[1]'s last row
        mom[1] = at(0, 4, 8, 8)
        uo = [at(3 * 32 + 28, 4, 8, 8), MuonMatrix(None, 0, 0, 0, 0)]
    elif case == "column_slices":
        # one 4 x 16 fp32 parent: momentum 0 = columns 0..7, momentum 1 = columns 8..15
        mom = [at(0, 4, 8, 16), at(32, 4, 8, 16)]
    elif case == "column_slices_one_shared":
        mom = [at(0, 4, 8, 16), at(28, 4, 8, 16)]
    elif case == "wraps_into_next_row":
        # momentum 1 starts 24 bytes into row 0 of momentum 0 (its columns end at
        # byte 16) and runs 16 bytes, into momentum 0's row 1 (bytes 32..47)
        g = [m(2, 4, 0), m(2, 4, 0)]
        mom = [at(0, 2, 4, 8), at(24, 2, 4, 8)]
    elif case == "ends_at_last_row":
        # the same, but momentum 0 has one row: the wrapped bytes are outside it
        g = [m(1, 4, 0), m(2, 4, 0)]
        mom = [at(0, 1, 4, 8), at(24, 2, 4, 8)]
    elif case == "strides_differ_interleaved":
        # momentum 0: rows of 16 bytes every 64; momentum 1: rows of 16 bytes every
        # 32, starting 16 bytes in: they alternate and never meet
        g = [m(4, 4, 0), m(8, 4, 0)]
        mom = [at(0, 4, 4, 16), at(16, 8, 4, 8)]
    elif case == "strides_differ_meet":
        g = [m(4, 4, 0), m(8, 4, 0)]
        mom = [at(0, 4, 4, 16), at(8, 8, 4, 8)]
    elif case == "grads_share":
        g = [at(0, 4, 8, 8), at(0, 4, 8, 8)]
    elif case == "bf16_out_inside_f32_gap":
        # fp32 momentum rows use bytes 0..31 of every 64; the bf16 output's rows use 32..47
        mom = [at(0, 4, 8, 16), m(4, 8, 0)]
        uo = [at(32, 4, 8, 32, 1), MuonMatrix(None, 0, 0, 0, 0)]
    rc, msg = mu.check_update_args(g, mom, w, uo)
    assert rc == code, (case, rc, msg)
    if code != OK:
        assert "share memory" in msg, msg


def test_polar_buffer_overlap(lib):
    x = at(0, 4, 8, 8)
    assert mu.check_polar_args([x], [x])[0] == OK                              # in place
    assert mu.check_polar_args([x, m(4, 8, 0)], [m(4, 8, 0), x])[0] == OK      # an output over another input
    shifted = at(4, 4, 8, 8)
    assert mu.check_polar_args([x], [shifted])[0] == OK                        # partly over its own input
    rc, msg = mu.check_polar_args([m(4, 8, 0), m(4, 8, 0)], [x, shifted])
    assert rc == INVALID and "out[0] and out[1]" in msg, msg
    assert mu.check_polar_args([m(4, 8, 0), m(4, 8, 0)], [at(0, 4, 8, 16), at(32, 4, 8, 16)])[0] == OK


def test_batch_count_limits(lib):
    buf = ctypes.create_string_buffer(64)
    assert lib.muon_check_polar_args(-1, None, None, None, buf, 64) == INVALID
    assert lib.muon_check_update_args(2, None, None, None, None, None, buf, 64) == INVALID


def test_null_handle_is_rejected(lib):
    assert lib.ns_polar(None, 0, None, None, None) == INVALID
    assert lib.muon_update(None, 0, None, None, None, None, None) == INVALID
    assert lib.muon_destroy(None) == OK


def test_classic_config_equals_page_values(lib):
    c = mu.classic_config()
    k, n = PAGE["classic_recipe"], PAGE["ns5_classic"]
    assert c.ns_steps == n["steps"]
    assert (c.ns_a, c.ns_b, c.ns_c) == pytest.approx((n["a"], n["b"], n["c"]), rel=1e-7)
    assert c.lr == pytest.approx(k["lr"], rel=1e-7)
    assert c.mu == pytest.approx(k["mu"], rel=1e-7)
    assert c.nesterov == 1
    assert (c.pp_iterations, c.contra, c.target_uw) == (0, 0.0, 0.0)
    # everything else keeps the default values
    d = mu.default_config()
    for f in ("ns_eps", "pp_beta", "pp_eps", "power_steps"):
        assert getattr(c, f) == getattr(d, f), f
    # the page's SGD momentum (and nothing else) among the flags
    assert k["momentum_form"] == "sgd" and c.flags == mu.MUON_FLAG_SGD_MOMENTUM
    assert mu.make_config("classic", lr=0.02).lr == pytest.approx(0.02)


def test_momentum_warmup_host_function(lib):
    w = PAGE["classic_recipe"]["warmup"]
    for s in (-3, 0, 1, 137, 250, 499, 500, 501, 10 ** 9):
        frac = min(max(s, 0) / w["steps"], 1.0)
        want = (1 - frac) * w["mu_start"] + frac * w["mu_end"]
        got = lib.muon_momentum_warmup(s, w["mu_start"], w["mu_end"], w["steps"])
        assert got == pytest.approx(want, abs=1e-7), s
    assert lib.muon_momentum_warmup(5, 0.85, 0.95, 0) == pytest.approx(0.95)


def test_overlapping_rows_are_rejected(lib):
    """A tensor whose rows overlap (an expanded row, stride(0) = 0, or an
    as_strided view with stride(0) < cols) keeps its stride in the
    descriptor, and the library rejects it as momentum, weight or output
    before anything is enqueued."""
    import torch
    ex = torch.zeros(1, 8).expand(4, 8)
    ov = torch.zeros(40).as_strided((4, 8), (5, 1))
    assert mu.row_stride(ex) == 0 and mu.row_stride(ov) == 5
    assert mu.row_stride(torch.zeros(1, 8)) == 8 and mu.row_stride(torch.zeros(6, 8)[:, 2:5]) == 8
    for ld in (mu.row_stride(ex), mu.row_stride(ov)):
        bad = m(4, 8, 0, ld=ld)
        rc, msg = mu.check_update_args([m(4, 8)], [bad], None, None)
        assert rc == -3 and "ld" in msg, (ld, rc, msg)
        rc, _ = mu.check_update_args([m(4, 8)], [m(4, 8, 0)], [bad], None)
        assert rc == -3
        rc, _ = mu.check_update_args([m(4, 8)], [m(4, 8, 0)], None, [bad])
        assert rc == -3
        rc, _ = mu.check_polar_args([m(4, 8)], [bad])
        assert rc == -3
