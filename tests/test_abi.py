"""Host-side checks of the C ABI: the library loads, exports every function the
header declares, and rejects bad arguments before touching the device.

No test here launches a kernel: every call either fails validation or is a
zero-size no-op, both of which return before any HIP call.  (The addresses are
fake, so a call that passed validation would launch on a garbage pointer; the
adjacency case of the overlap check is covered on the GPU with real buffers.)
"""
import ctypes
import os
import re

import pytest

from linear_recurrence_scan_row_amd import rlca as binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rlca.h")

OK, NULLP, SIZE, VALUE, ALIAS, MISAL, HIP = range(7)
A = 0x10000000          # fake, 256-byte aligned "device" addresses: never dereferenced
B = 0x20000000
C = 0x30000000
D = 0x40000000
E = 0x50000000
F = 0x60000000
G = 0x70000000
H = 0x80000000


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:rlca_status|const char \*)\s*(rlca_\w+)\s*\(",
                                 text, re.M)))


@pytest.fixture(scope="module")
def lib():
    return binding.lib()


def test_header_declares_the_seven_estimators():
    names = declared_functions()
    for n in ("rlca_gae", "rlca_td_lambda", "rlca_discounted_returns", "rlca_vtrace",
              "rlca_retrace", "rlca_eligibility_traces", "rlca_episodic_prefix_sum",
              "rlca_status_string"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    # and the binding's signature table covers every compute entry point
    compute = [n for n in declared_functions() if n != "rlca_status_string"]
    assert sorted(binding.SIGNATURES) == sorted(compute)


def test_status_strings(lib):
    for s in range(7):
        assert lib.rlca_status_string(s)
    assert lib.rlca_status_string(99) == b"unknown status"


def gae(lib, r=A, v=B, term=C, trunc=None, tv=None, boot=None, gamma=0.99, lam=0.95, n=4,
        t=8, adv=D, ret=E):
    return lib.rlca_gae(r, v, term, trunc, tv, boot, gamma, lam, n, t, adv, ret, None)


def test_zero_size_is_a_no_op(lib):
    assert gae(lib, n=0) == OK
    assert gae(lib, t=0) == OK
    assert gae(lib, r=None, v=None, term=None, adv=None, ret=None, n=0) == OK
    assert lib.rlca_episodic_prefix_sum(None, 0, None, 0, 0, 5, None, None) == OK


def test_size_errors(lib):
    assert gae(lib, n=-1) == SIZE
    assert gae(lib, t=-3) == SIZE
    assert gae(lib, t=(1 << 30) + 1) == SIZE
    assert gae(lib, n=(1 << 31) + 1) == SIZE
    assert lib.rlca_discounted_returns(A, C, None, None, None, 0.9, 1 << 31, 1 << 30, D,
                                       None) == SIZE


def test_value_errors(lib):
    for g in (-0.1, 1.5, float("nan"), float("inf")):
        assert gae(lib, gamma=g) == VALUE
        assert gae(lib, lam=g) == VALUE
    assert lib.rlca_vtrace(A, B, C, D, E, None, None, None, 0.99, 1.0, 0.0, 1.0, 4, 8, F, G,
                           None) == VALUE
    assert lib.rlca_vtrace(A, B, C, D, E, None, None, None, 0.99, 1.0, 1.0, float("nan"), 4,
                           8, F, G, None) == VALUE
    assert lib.rlca_retrace(A, B, C, D, E, F, None, None, None, 0.99, 0.95, -1.0, 4, 8, G,
                            None) == VALUE
    assert lib.rlca_eligibility_traces(A, B, 7, 0.9, 0.9, 4, 8, C, None) == VALUE
    assert lib.rlca_episodic_prefix_sum(A, 5, B, 0, 4, 8, C, None) == VALUE
    assert lib.rlca_affine_scan(A, B, None, 2, 4, 8, C, None) == VALUE


def test_null_pointer_errors(lib):
    assert gae(lib, r=None) == NULLP
    assert gae(lib, v=None) == NULLP
    assert gae(lib, term=None) == NULLP
    assert gae(lib, adv=None) == NULLP
    assert gae(lib, trunc=F, tv=None) == NULLP
    assert lib.rlca_td_lambda(A, B, C, None, None, None, 0.9, 0.9, 4, 8, None, None) == NULLP
    assert lib.rlca_retrace(A, B, None, D, E, F, None, None, None, 0.9, 0.9, 1.0, 4, 8, G,
                            None) == NULLP
    assert lib.rlca_eligibility_traces(A, None, 0, 0.9, 0.9, 4, 8, C, None) == NULLP
    assert lib.rlca_episodic_prefix_sum(A, 1, B, 0, 4, 8, None, None) == NULLP
    assert lib.rlca_affine_scan(A, None, None, 0, 4, 8, C, None) == NULLP
    assert lib.rlca_affine_scan(A, B, None, 1, 4, 8, None, None) == NULLP


def test_alignment_errors(lib):
    assert gae(lib, r=A + 2) == MISAL
    assert gae(lib, adv=D + 1) == MISAL
    assert gae(lib, boot=F + 2) == MISAL
    # flags are bytes: any address is fine; 4-byte but not 16-byte alignment is fine
    assert gae(lib, term=C + 1, r=A + 4, n=0) == OK


def test_aliasing_errors(lib):
    n, t = 4, 8
    nbytes = n * t * 4
    assert gae(lib, adv=A) == ALIAS                         # in-place on rewards
    assert gae(lib, adv=B + nbytes - 4) == ALIAS            # overlaps the tail of values
    assert gae(lib, adv=D, ret=D + 4) == ALIAS              # outputs overlap each other
    assert gae(lib, adv=C) == ALIAS                         # over the flags
    assert lib.rlca_episodic_prefix_sum(A, 0, B, 0, n, t, A + 4, None) == ALIAS
    assert lib.rlca_affine_scan(A, B, C, 0, n, t, C - 8, None) == ALIAS     # over the carry
    assert lib.rlca_affine_scan(A, B, None, 1, n, t, B + 4, None) == ALIAS
    assert lib.rlca_affine_scan(A + 2, B, None, 1, n, t, C, None) == MISAL
