"""Host-side checks of the C ABI (no GPU needed): the library loads, exports every function the
header declares, and rejects bad arguments before anything is launched."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "aaac.h")
LIB = os.path.join(ROOT, "post_weight_quantization_06_amd", "libaaac.so")

OK, INVALID, SHAPE, WS_SMALL, HIP = 0, 1, 2, 3, 4
OP_IMPORTANCE, OP_INIT, OP_ASSIGN, OP_REFINE = 0, 1, 2, 3
# a fake, 256-byte aligned device address: only ever passed to calls that must fail validation
FAKE = ctypes.c_void_p(1 << 20)
i64 = ctypes.c_int64


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(aaac_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail("libaaac.so is not built (python -m post_weight_quantization_06_amd.build)")
    L = ctypes.CDLL(LIB)
    L.aaac_status_string.restype = ctypes.c_char_p
    L.aaac_last_error.restype = ctypes.c_char_p
    L.aaac_workspace_bytes.restype = ctypes.c_size_t
    L.aaac_workspace_bytes.argtypes = [ctypes.c_int, i64, i64, ctypes.c_int, ctypes.c_int,
                                       ctypes.c_int]
    L.aaac_batch_workspace_bytes.restype = ctypes.c_size_t
    return L


def test_header_declares_the_six_operations_and_the_batch_calls():
    names = declared_functions()
    for op in ("importance", "init_quantiles", "assign", "refine", "pack", "dequant",
               "init_quantiles_batch", "assign_batch", "refine_batch", "pack_batch",
               "dequant_batch"):
        assert "aaac_" + op in names


def test_every_declared_function_is_exported(lib):
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing


def test_status_strings(lib):
    for st in (OK, INVALID, SHAPE, WS_SMALL, HIP, 99):
        s = lib.aaac_status_string(st)
        assert s and len(s) > 0


def test_workspace_queries_are_host_only(lib):
    ws = lib.aaac_workspace_bytes
    # assign needs a workspace only for its error totals: counters and per-workgroup partials
    assert ws(OP_ASSIGN, 64, 1024, 128, 128, 16) > 256
    assert ws(OP_ASSIGN, 64, 1000, 128, 128, 16) == 0          # C not a multiple of g
    assert ws(OP_REFINE, 64, 1024, 128, 128, 16) > 0
    assert ws(OP_INIT, 64, 1024, 128, 0, 16) >= 64 * 1024 * 4  # one 32-bit key per weight
    assert ws(OP_REFINE, 64, 1000, 128, 128, 16) == 0          # C not a multiple of g
    assert ws(OP_REFINE, 64, 1024, 96, 32, 16) == 0            # g not a power of two
    assert ws(OP_REFINE, 64, 1024, 128, 256, 16) == 0          # S > g
    assert ws(OP_REFINE, 64, 1024, 128, 128, 17) == 0          # n > 16
    assert ws(OP_REFINE, 64, 1024, 128, 128, 1) == 0           # n < 2
    assert ws(42, 64, 1024, 128, 128, 16) == 0                 # unknown op


def test_batch_workspace_grows_with_count(lib):
    R1 = (i64 * 1)(64)
    C1 = (i64 * 1)(1024)
    R2 = (i64 * 2)(64, 128)
    C2 = (i64 * 2)(1024, 2048)
    a = lib.aaac_batch_workspace_bytes(OP_REFINE, 1, R1, C1, 128, 128, 16)
    b = lib.aaac_batch_workspace_bytes(OP_REFINE, 2, R2, C2, 128, 128, 16)
    assert 0 < a < b
    assert lib.aaac_batch_workspace_bytes(OP_REFINE, 9, R2, C2, 128, 128, 16) == 0


def _assign(lib, R, C, g, S, n, W=FAKE, I=FAKE, T=FAKE, codes=FAKE, sel=FAKE, err=None,
            err_total=None, ws=None, ws_bytes=0):
    return lib.aaac_assign(W, i64(R), i64(C), g, S, n, I, T, codes, sel, err, err_total, ws,
                           ctypes.c_size_t(ws_bytes), None)


def test_assign_rejects_bad_shapes_and_pointers_before_launch(lib):
    assert _assign(lib, 64, 1024, 96, 96, 16) == SHAPE
    assert _assign(lib, 64, 1024, 128, 256, 16) == SHAPE
    assert _assign(lib, 64, 1000, 128, 128, 16) == SHAPE
    assert _assign(lib, 0, 1024, 128, 128, 16) == SHAPE
    assert _assign(lib, -1, 1024, 128, 128, 16) == SHAPE               # negative R
    assert _assign(lib, 64, 0, 8, 8, 16) == SHAPE                      # empty rows
    assert _assign(lib, 64, 4, 8, 8, 16) == SHAPE                      # C < 8
    assert _assign(lib, 64, 1 << 31, 128, 128, 16) == SHAPE            # C >= 2^31
    assert _assign(lib, 64, 1024, 4, 4, 16) == SHAPE                   # g < 8
    assert _assign(lib, 64, 2048, 1024, 128, 16) == SHAPE              # g > 512
    assert _assign(lib, 64, 1024, 128, 4, 16) == SHAPE                 # S < 8
    assert _assign(lib, 64, 1024, 128, 128, 1) == SHAPE                # n < 2
    assert _assign(lib, 64, 1024, 128, 128, 17) == SHAPE
    assert _assign(lib, 1 << 21, 1 << 19, 128, 128, 16) == SHAPE   # R*C >= 2^40
    assert b"n=17" in lib.aaac_last_error() or b"2^40" in lib.aaac_last_error()
    assert _assign(lib, 64, 1024, 128, 128, 16, W=None) == INVALID
    assert _assign(lib, 64, 1024, 128, 128, 16, W=ctypes.c_void_p((1 << 20) + 2)) == INVALID
    assert _assign(lib, 64, 1024, 128, 128, 16, codes=None) == INVALID
    assert _assign(lib, 64, 1024, 128, 128, 16, err=ctypes.c_void_p((1 << 20) + 4)) == INVALID
    assert len(lib.aaac_last_error()) > 0


def test_assign_error_total_needs_its_workspace(lib):
    need = lib.aaac_workspace_bytes(OP_ASSIGN, 64, 1024, 128, 128, 16)
    assert _assign(lib, 64, 1024, 128, 128, 16, err_total=FAKE) == INVALID          # no ws
    assert b"err_total" in lib.aaac_last_error()
    assert _assign(lib, 64, 1024, 128, 128, 16, err_total=FAKE, ws=FAKE,
                   ws_bytes=need - 1) == WS_SMALL
    assert _assign(lib, 64, 1024, 128, 128, 16, err_total=ctypes.c_void_p((1 << 20) + 4), ws=FAKE,
                   ws_bytes=need) == INVALID                                         # misaligned
    assert _assign(lib, 64, 1024, 128, 128, 16, err_total=FAKE,
                   ws=ctypes.c_void_p((1 << 20) + 128), ws_bytes=need) == INVALID    # ws alignment
    R2 = (i64 * 2)(64, 128)
    C2 = (i64 * 2)(1024, 2048)
    two = lib.aaac_batch_workspace_bytes(OP_ASSIGN, 2, R2, C2, 128, 128, 16)
    assert two > need
    P = (ctypes.c_void_p * 2)(FAKE, FAKE)
    f = lib.aaac_assign_batch
    assert f(2, P, R2, C2, 128, 128, 16, P, P, P, P, FAKE, FAKE, ctypes.c_size_t(need),
             None) == WS_SMALL


def test_refine_rejects_small_workspace_and_unknown_flags(lib):
    need = lib.aaac_workspace_bytes(OP_REFINE, 64, 1024, 128, 128, 16)
    args = (FAKE, i64(64), i64(1024), 128, 128, 16, FAKE, FAKE, FAKE, FAKE, FAKE)
    n_ = ctypes.c_size_t(need)
    assert lib.aaac_refine(*args, 0, None, None, FAKE, ctypes.c_size_t(need - 1), None) == WS_SMALL
    assert b"workspace" in lib.aaac_last_error()
    assert lib.aaac_refine(*args, 4, None, None, FAKE, n_, None) == INVALID       # unknown flag
    assert lib.aaac_refine(*args, 0, None, None, None, n_, None) == INVALID
    assert lib.aaac_refine(*args, 0, None, None, ctypes.c_void_p((1 << 20) + 128), n_,
                           None) == INVALID
    # the optional error output: 8-byte aligned, with its w2 partner, and the W2-known flag only
    # with them
    assert lib.aaac_refine(*args, 0, ctypes.c_void_p((1 << 20) + 4), FAKE, FAKE, n_,
                           None) == INVALID
    assert lib.aaac_refine(*args, 0, FAKE, None, FAKE, n_, None) == INVALID
    assert lib.aaac_refine(*args, 2, None, None, FAKE, n_, None) == INVALID


def test_pack_and_dequant_bitmap_rule(lib):
    # S == g forbids a bitmap, S < g requires one
    assert lib.aaac_pack(FAKE, i64(64), i64(1024), 128, 128, 16, FAKE, FAKE, None, None, FAKE,
                         FAKE, FAKE, None) == INVALID
    assert lib.aaac_pack(FAKE, i64(64), i64(1024), 128, 16, 16, FAKE, FAKE, None, None, FAKE,
                         None, FAKE, None) == INVALID
    # codes one per byte: codes_u8 and codes_out together, aligned
    assert lib.aaac_pack(FAKE, i64(64), i64(1024), 128, 128, 16, FAKE, FAKE, FAKE, None, FAKE,
                         None, FAKE, None) == INVALID
    assert lib.aaac_pack(FAKE, i64(64), i64(1024), 128, 128, 16, FAKE, FAKE, None, FAKE, FAKE,
                         None, FAKE, None) == INVALID
    assert lib.aaac_pack(FAKE, i64(64), i64(1024), 128, 128, 16, FAKE, FAKE,
                         ctypes.c_void_p((1 << 20) + 4), FAKE, FAKE, None, FAKE, None) == INVALID
    assert b"codes_u8" in lib.aaac_last_error()
    assert lib.aaac_dequant(FAKE, FAKE, FAKE, FAKE, i64(64), i64(1024), 128, 128, 16, FAKE,
                            None) == INVALID
    assert lib.aaac_dequant(FAKE, FAKE, None, FAKE, i64(64), i64(1024), 128, 16, 16, FAKE,
                            None) == INVALID


def test_init_and_importance_reject_bad_arguments(lib):
    assert lib.aaac_init_quantiles(FAKE, i64(64), i64(1024), 100, 16, FAKE, FAKE,
                                   ctypes.c_size_t(1 << 30), None) == SHAPE
    assert lib.aaac_init_quantiles(FAKE, i64(64), i64(1024), 128, 16, FAKE, FAKE,
                                   ctypes.c_size_t(16), None) == WS_SMALL
    assert lib.aaac_importance(FAKE, i64(16), i64(64), i64(32), FAKE, FAKE, FAKE,
                               ctypes.c_size_t(1 << 30), None) == SHAPE   # ldx < K
    assert lib.aaac_importance(None, i64(16), i64(64), i64(64), FAKE, FAKE, FAKE,
                               ctypes.c_size_t(1 << 30), None) == INVALID


def test_batch_calls_reject_bad_counts(lib):
    P = (ctypes.c_void_p * 1)(FAKE)
    R = (i64 * 1)(64)
    C = (i64 * 1)(1024)
    z = ctypes.c_size_t(0)
    assert lib.aaac_assign_batch(0, P, R, C, 128, 128, 16, P, P, P, P, None, None, z,
                                 None) == INVALID
    assert lib.aaac_assign_batch(9, P, R, C, 128, 128, 16, P, P, P, P, None, None, z,
                                 None) == INVALID
    assert lib.aaac_refine_batch(1, P, R, C, 128, 128, 16, P, P, P, P, 0, None, None, FAKE,
                                 ctypes.c_size_t(16), None) == WS_SMALL


def test_awq_prescale_rejects_bad_arguments(lib):
    f = lib.aaac_awq_prescale
    assert f(FAKE, i64(4), i64(12), FAKE, FAKE, FAKE, FAKE, None) == SHAPE      # C % 8
    assert f(FAKE, i64(0), i64(16), FAKE, FAKE, FAKE, FAKE, None) == SHAPE      # R < 1
    assert f(FAKE, i64(1 << 21), i64(1 << 19), FAKE, None, FAKE, None, None) == SHAPE
    assert f(None, i64(4), i64(16), FAKE, FAKE, FAKE, FAKE, None) == INVALID
    assert f(FAKE, i64(4), i64(16), ctypes.c_void_p((1 << 20) + 4), None, FAKE, None,
             None) == INVALID                                                  # a misaligned
    assert f(FAKE, i64(4), i64(16), FAKE, FAKE, FAKE, None, None) == INVALID    # I without I_scaled
    assert b"I_scaled" in lib.aaac_last_error()


def test_assign_refine_batch_rejects_bad_arguments(lib):
    P = (ctypes.c_void_p * 1)(FAKE)
    R = (i64 * 1)(64)
    C = (i64 * 1)(1024)
    f = lib.aaac_assign_refine_batch
    need = lib.aaac_batch_workspace_bytes(OP_REFINE, 1, R, C, 128, 128, 16)
    N = ctypes.c_size_t(need)
    assert f(0, P, R, C, 128, 128, 16, P, P, P, P, 0, None, None, FAKE, N, None) == INVALID
    assert f(1, P, R, C, 128, 128, 16, P, P, P, P, 4, None, None, FAKE, N, None) == INVALID
    assert f(1, P, R, C, 128, 128, 16, P, P, P, P, 0, None, None, FAKE, ctypes.c_size_t(16),
             None) == WS_SMALL
    assert f(1, P, R, C, 100, 100, 16, P, P, P, P, 0, None, None, FAKE, N, None) == SHAPE
    # error outputs: err and w2 together, 8-byte aligned; the W2-known flag needs them
    assert f(1, P, R, C, 128, 128, 16, P, P, P, P, 0, FAKE, None, FAKE, N, None) == INVALID
    assert f(1, P, R, C, 128, 128, 16, P, P, P, P, 0, ctypes.c_void_p((1 << 20) + 4), FAKE, FAKE,
             N, None) == INVALID
    assert f(1, P, R, C, 128, 128, 16, P, P, P, P, 2, None, None, FAKE, N, None) == INVALID
    assert b"W2_KNOWN" in lib.aaac_last_error()


def test_init_batch_workspace_and_arguments(lib):
    R1 = (i64 * 1)(64)
    C1 = (i64 * 1)(1024)
    R2 = (i64 * 2)(64, 128)
    C2 = (i64 * 2)(1024, 2048)
    one = lib.aaac_batch_workspace_bytes(OP_INIT, 1, R1, C1, 128, 8, 16)
    two = lib.aaac_batch_workspace_bytes(OP_INIT, 2, R2, C2, 128, 8, 16)
    # the single call and a batch of one need the same workspace; keys add 4 bytes per weight
    assert one == lib.aaac_workspace_bytes(OP_INIT, 64, 1024, 128, 0, 16)
    assert two - one >= 128 * 2048 * 4
    assert lib.aaac_batch_workspace_bytes(OP_INIT, 1, R1, (i64 * 1)(1000), 128, 8, 16) == 0
    f = lib.aaac_init_quantiles_batch
    P = (ctypes.c_void_p * 1)(FAKE)
    assert f(0, P, R1, C1, 128, 16, P, FAKE, ctypes.c_size_t(one), None) == INVALID
    assert f(9, P, R1, C1, 128, 16, P, FAKE, ctypes.c_size_t(one), None) == INVALID
    assert f(1, None, R1, C1, 128, 16, P, FAKE, ctypes.c_size_t(one), None) == INVALID
    assert f(1, P, R1, C1, 128, 16, P, FAKE, ctypes.c_size_t(one - 1), None) == WS_SMALL
    assert f(1, P, R1, (i64 * 1)(1000), 128, 16, P, FAKE, ctypes.c_size_t(one), None) == SHAPE
    assert f(1, P, R1, C1, 128, 17, P, FAKE, ctypes.c_size_t(one), None) == SHAPE
    bad = (ctypes.c_void_p * 1)((1 << 20) + 2)
    assert f(1, bad, R1, C1, 128, 16, P, FAKE, ctypes.c_size_t(one), None) == INVALID


def test_pack_and_dequant_batches_reject_bad_arguments(lib):
    """Argument checks of the batched pack and dequant run on the host: nothing is launched."""
    R1 = (i64 * 1)(64)
    C1 = (i64 * 1)(1024)
    P = (ctypes.c_void_p * 1)(FAKE)
    bad = (ctypes.c_void_p * 1)((1 << 20) + 2)
    pk = lib.aaac_pack_batch
    assert pk(0, P, R1, C1, 128, 128, 16, P, P, P, None, P, None) == INVALID      # count 0
    assert pk(9, P, R1, C1, 128, 128, 16, P, P, P, None, P, None) == INVALID      # count > 8
    assert pk(1, None, R1, C1, 128, 128, 16, P, P, P, None, P, None) == INVALID   # null array
    assert pk(1, P, R1, C1, 128, 128, 16, P, P, P, P, P, None) == INVALID         # bitmap, S == g
    assert pk(1, P, R1, C1, 128, 16, 16, P, P, P, None, P, None) == INVALID       # none, S < g
    assert pk(1, bad, R1, C1, 128, 128, 16, P, P, P, None, P, None) == INVALID    # misaligned W
    assert pk(1, P, R1, (i64 * 1)(1000), 128, 128, 16, P, P, P, None, P, None) == SHAPE
    dq = lib.aaac_dequant_batch
    assert dq(0, P, P, None, P, R1, C1, 128, 128, 16, P, None) == INVALID
    assert dq(1, P, P, None, None, R1, C1, 128, 128, 16, P, None) == INVALID     # null tables
    assert dq(1, P, P, None, P, R1, C1, 128, 16, 16, P, None) == INVALID         # S < g, no bitmap
    assert dq(1, P, P, None, P, R1, C1, 128, 128, 16, bad, None) == INVALID      # misaligned out
    assert dq(1, P, P, None, P, R1, C1, 128, 128, 17, P, None) == SHAPE


def test_refine_noalloc_rejects_bad_arguments_before_touching_the_device(lib):
    """The allocation-free refine checks every argument on the host before it looks up its device
    scratch or launches anything."""
    P = (ctypes.c_void_p * 1)(FAKE)
    R = (i64 * 1)(64)
    C = (i64 * 1)(1024)
    f = lib.aaac_refine_batch_noalloc
    assert f(0, P, R, C, 128, 128, 16, P, P, P, P, 0, None, None, None) == INVALID   # count
    assert f(9, P, R, C, 128, 128, 16, P, P, P, P, 0, None, None, None) == INVALID
    assert f(1, P, R, C, 100, 100, 16, P, P, P, P, 0, None, None, None) == SHAPE     # g
    assert f(1, P, R, C, 128, 128, 16, P, P, P, P, 8, None, None, None) == INVALID   # flags
    assert f(1, P, R, C, 128, 128, 16, P, P, P, P, 2, None, None, None) == INVALID   # W2 known
    assert f(1, P, R, C, 128, 128, 16, P, P, P, None, 0, None, None, None) == INVALID
    assert b"noalloc" in lib.aaac_last_error()
