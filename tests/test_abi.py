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
    return sorted(set(re.findall(r"^\s*(?:rlca_status|const char \*|size_t)\s*(rlca_\w+)\s*\(",
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
    assert sorted(list(binding.SIGNATURES) + list(binding.SIZE_QUERIES)) == sorted(compute)


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
    # 2^31 rows longer than one 2048-step tile would need 2^31 workgroups
    # (fake arrays 2^45 bytes apart, so that none of them overlaps)
    far = [k << 45 for k in range(1, 6)]
    assert gae(lib, r=far[0], v=far[1], term=far[2], adv=far[3], ret=far[4], n=1 << 31,
               t=2049) == SIZE
    assert lib.rlca_eligibility_traces(far[0], far[1], 0, 0.9, 0.9, 1 << 31, 2049, far[2],
                                       None) == SIZE
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
    # trace clips above 1 would make the recurrence expansive: refused
    for c_bar in (1.0001, 3.0, float("inf")):
        assert lib.rlca_vtrace(A, B, C, D, E, None, None, None, 0.99, 1.0, 1.0, c_bar, 4, 8, F,
                               G, None) == VALUE
        assert lib.rlca_retrace(A, B, C, D, E, F, None, None, None, 0.99, 0.95, c_bar, 4, 8, G,
                                None) == VALUE
        assert run_batch(lib, call(op=binding.OP_VTRACE, rewards=A, values=B, behaviour_logp=C,
                                   target_logp=D, terminated=E, out0=F, c_bar=c_bar)) == VALUE
    # rho_bar above 1 only scales alpha: accepted (nothing to enqueue at n = 0)
    assert lib.rlca_vtrace(A, B, C, D, E, None, None, None, 0.99, 1.0, 1e3, 1.0, 0, 8, F, G,
                           None) == OK
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


def call(op=0, n=4, t=8, **fields):
    c = binding.RlcaCall(op=op, num_envs=n, T=t, gamma=0.99, lambda_=0.95, rho_bar=1.0,
                         c_bar=1.0)
    if op in (binding.OP_GAE, binding.OP_TD_LAMBDA):
        c.rewards, c.values, c.terminated, c.out0 = A, B, C, D
    for k, v in fields.items():
        setattr(c, k, v)
    return c


def run_batch(lib, *calls, count=None):
    arr = (binding.RlcaCall * max(len(calls), 1))(*calls)
    return lib.rlca_run_batch(arr, len(calls) if count is None else count, None)


def test_batch_struct_matches_header():
    # rlca_call: int op; two int64; nine pointers; four floats; three ints; two pointers
    assert ctypes.sizeof(binding.RlcaCall) == 144
    assert binding.RlcaCall.out0.offset == 128 and binding.RlcaCall.gamma.offset == 96
    text = open(HEADER).read()
    assert re.search(r"#define\s+RLCA_MAX_BATCH\s+64\b", text)
    assert binding.MAX_BATCH == 64


def test_batch_count_and_null(lib):
    assert lib.rlca_run_batch(None, 0, None) == OK
    assert lib.rlca_run_batch(None, 1, None) == NULLP
    assert run_batch(lib, call(), count=-1) == SIZE
    assert run_batch(lib, *[call(n=0)] * 65) == SIZE
    assert run_batch(lib, *[call(n=0)] * 64) == OK          # all empty: nothing launched


def test_batch_rejects_before_launching_anything(lib):
    # the first call is valid on its own; the batch fails on a later one, and
    # since every call is checked before the first launch nothing runs
    assert run_batch(lib, call(), call(op=99)) == VALUE
    assert run_batch(lib, call(), call(gamma=1.5, rewards=E, values=F, terminated=G,
                                       out0=H)) == VALUE
    assert run_batch(lib, call(), call(t=-1)) == SIZE
    assert run_batch(lib, call(), call(values=None)) == NULLP
    assert run_batch(lib, call(), call(rewards=A + 2)) == MISAL
    assert run_batch(lib, call(), call(out0=A)) == ALIAS    # aliasing within the call
    affine = call(op=binding.OP_AFFINE, rewards=A, values=B, direction=3, out0=C)
    assert run_batch(lib, affine) == VALUE
    prefix = call(op=binding.OP_PREFIX_SUM, rewards=A, terminated=B, dtype=7, out0=C)
    assert run_batch(lib, prefix) == VALUE


def test_batch_cross_call_aliasing(lib):
    n, t = 4, 8
    first = call(out0=D, out1=E)
    # a second call reading the first call's output
    assert run_batch(lib, first, call(op=1, rewards=E + 4, values=F, terminated=G,
                                      out0=H)) == ALIAS
    # ... or writing the first call's input
    assert run_batch(lib, first, call(op=1, rewards=F, values=G, terminated=H,
                                      out0=C)) == ALIAS
    # ... or both writing one buffer, in either order
    assert run_batch(lib, call(op=1, rewards=F, values=G, terminated=H, out0=D + n * t * 4 - 4),
                     first) == ALIAS
    # an empty call is exempt
    assert run_batch(lib, call(n=0, out0=A), call(n=0, rewards=D)) == OK


def test_batch_dtype_validation(lib):
    bf16, f16, i32 = 2, 3, 1
    assert run_batch(lib, call(dtype=9)) == VALUE
    assert run_batch(lib, call(dtype=i32)) == VALUE          # int32 only for the prefix sum
    affine = dict(op=binding.OP_AFFINE, rewards=A, values=B, out0=C)
    assert run_batch(lib, call(dtype=i32, **affine)) == VALUE
    # 16-bit storage: 2-byte alignment suffices, odd addresses do not
    assert run_batch(lib, call(dtype=bf16, rewards=A + 1)) == MISAL
    assert run_batch(lib, call(dtype=f16, out0=D + 3)) == MISAL
    assert run_batch(lib, call(dtype=bf16, rewards=A + 2, n=0)) == OK
    assert run_batch(lib, call(dtype=0, rewards=A + 2)) == MISAL          # fp32 needs 4 bytes
    # byte ranges use the storage size: with bf16 the values span n*T*2 bytes
    n, t = 4, 8
    assert run_batch(lib, call(dtype=bf16, out0=B + n * t * 2 - 2)) == ALIAS
    assert run_batch(lib, call(dtype=bf16, out0=B + n * t * 4 - 4, t=-1)) == SIZE
    prefix = dict(op=binding.OP_PREFIX_SUM, rewards=A + 1, terminated=B, out0=C)
    assert run_batch(lib, call(dtype=f16, **prefix)) == MISAL
    assert lib.rlca_episodic_prefix_sum(A + 1, bf16, B, 0, 4, 8, C, None) == MISAL
    assert lib.rlca_episodic_prefix_sum(A, 7, B, 0, 4, 8, C, None) == VALUE


def test_workspace_size_queries(lib):
    assert lib.rlca_gae_stats_workspace_size(0, 128) == 0
    assert lib.rlca_gae_stats_workspace_size(-1, 128) == 0
    assert lib.rlca_ppo_clip_loss_workspace_size(4, 0) == 0
    # ticket counters (33 words, 128 bytes apart), then one (sum, sum of squares) pair of doubles
    # per workgroup: 4096 x 128 packs 16 rows per 8-wave workgroup; the
    # unaligned path packs 8 per 4-wave one
    assert lib.rlca_gae_stats_workspace_size(4096, 128) == 4224 + 16 * 512
    # chunked: 2048-step chunks (49 per row) for aligned arrays, 2040-step
    # chunks (50 per row, the last in scan order 4..2043 steps) for T % 4 != 0
    # or inputs off phase 0; the size covers whichever the pointers select
    assert lib.rlca_gae_stats_workspace_size(3, 100000) == 4224 + 16 * 3 * 50
    assert lib.rlca_gae_stats_workspace_size(3, 100001) == 4224 + 16 * 3 * 50
    # the chunked path's bounds for backward scans: rows of 16384 steps or
    # more, fewer than 128 of them (one pair per chunk: 9 chunks of 16388 or
    # 16384 steps, 17 of 32768 at 2040 steps each); otherwise one row per
    # workgroup (rows longer than a tile), or several short rows
    assert lib.rlca_gae_stats_workspace_size(127, 16388) == 4224 + 16 * 127 * 9
    assert lib.rlca_gae_stats_workspace_size(128, 16388) == 4224 + 16 * 128
    assert lib.rlca_gae_stats_workspace_size(127, 32768) == 4224 + 16 * 127 * 17
    assert lib.rlca_gae_stats_workspace_size(128, 32768) == 4224 + 16 * 128
    assert lib.rlca_gae_stats_workspace_size(1, 16384) == 4224 + 16 * 9
    assert lib.rlca_gae_stats_workspace_size(1, 16383) == 4224 + 16 * 1
    assert lib.rlca_ppo_clip_loss_workspace_size(4096, 128) == 4224 + 8 * 512
    assert lib.rlca_ppo_clip_loss_workspace_size(1 << 20, 512) == 4224 + 8 * 2048


def gae_stats(lib, stats=F, ws=G, nbytes=1 << 20, **kw):
    a = dict(r=A, v=B, term=C, adv=D, ret=E, n=4, t=8, gamma=0.99, lam=0.95)
    a.update(kw)
    return lib.rlca_gae_stats(a["r"], a["v"], a["term"], None, None, None, a["gamma"],
                              a["lam"], a["n"], a["t"], a["adv"], a["ret"], stats, ws, nbytes,
                              None)


def ppo(lib, adv=A, stats=None, new=B, old=C, clip=0.2, eps=1e-8, n=4, t=8, grad=D, loss=E,
        ws=F, nbytes=1 << 20):
    return lib.rlca_ppo_clip_loss(adv, stats, new, old, clip, eps, n, t, grad, loss, ws, nbytes,
                                  None)


def test_gae_stats_validation(lib):
    assert gae_stats(lib, n=0) == OK
    assert gae_stats(lib, stats=None) == NULLP
    assert gae_stats(lib, ws=None) == NULLP
    assert gae_stats(lib, stats=F + 4) == MISAL
    assert gae_stats(lib, ws=G + 4) == MISAL
    assert gae_stats(lib, nbytes=15) == SIZE                 # one pair needs 16 bytes
    assert gae_stats(lib, gamma=2.0) == VALUE
    assert gae_stats(lib, stats=D + 8) == ALIAS              # stats inside the advantages
    assert gae_stats(lib, ws=B) == ALIAS                     # workspace over the values
    assert gae_stats(lib, ws=F + 8) == ALIAS                 # workspace over the stats


def test_gae_stats_noalloc_validation(lib):
    """Checks that run before the entry point touches the GPU (the scratch
    buffer's address is looked up only after them)."""
    def call(stats=F, gamma=0.99, n=4, r=A):
        return lib.rlca_gae_stats_noalloc(r, B, C, None, None, None, gamma, 0.95, n, 8, D, E,
                                          stats, None)
    assert call(n=0) == OK
    assert call(stats=None) == NULLP
    assert call(r=None) == NULLP
    assert call(stats=F + 4) == MISAL
    assert call(gamma=1.5) == VALUE
    assert call(stats=D) == ALIAS            # stats over the advantages
    text = open(HEADER).read()
    assert re.search(r"#define\s+RLCA_GAE_STATS_SCRATCH_BYTES\s+69760\b", text)


def test_ppo_clip_loss_validation(lib):
    assert ppo(lib, n=0) == OK
    for clip in (-0.1, 1.0, float("nan")):
        assert ppo(lib, clip=clip) == VALUE
    assert ppo(lib, eps=-1.0) == VALUE
    assert ppo(lib, eps=float("inf")) == VALUE
    assert ppo(lib, adv=None) == NULLP
    assert ppo(lib, loss=None) == NULLP
    assert ppo(lib, ws=None) == NULLP
    assert ppo(lib, new=B + 2) == MISAL
    assert ppo(lib, loss=E + 4) == MISAL
    assert ppo(lib, stats=G + 4) == MISAL
    assert ppo(lib, nbytes=7) == SIZE
    assert ppo(lib, grad=B) == ALIAS                         # gradient over logp_new
    assert ppo(lib, loss=A + 8) == ALIAS                     # loss inside the advantages
    assert ppo(lib, ws=E) == ALIAS                           # workspace over the loss
    assert ppo(lib, stats=G, ws=G + 8) == ALIAS              # workspace over the stats


def test_missing_library_fails_loudly():
    """Without librlca.so the binding raises; there is no CPU fallback."""
    import subprocess
    import sys
    code = ("import linear_recurrence_scan_row_amd.rlca as r\n"
            "r.LIB_PATH = '/nonexistent/librlca.so'\n"
            "r._lib = None\n"
            "try:\n"
            "    r.lib()\n"
            "except ImportError as e:\n"
            "    print('raised', e)\n"
            "else:\n"
            "    raise SystemExit('lib() returned without the library')\n")
    out = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True,
                         timeout=120)
    assert out.returncode == 0 and "raised" in out.stdout, out.stdout + out.stderr


def test_product_package_never_imports_the_oracle():
    """The oracle is test infrastructure: importing the package (and its
    binding, build and workload modules) must not load it."""
    import subprocess
    import sys
    code = ("import sys\n"
            "import linear_recurrence_scan_row_amd as rl\n"
            "from linear_recurrence_scan_row_amd import rlca, build, workloads\n"
            "rl.lib()\n"
            "bad = [m for m in sys.modules if m == 'oracle' or m.startswith('oracle.')]\n"
            "raise SystemExit(f'oracle imported: {bad}' if bad else 0)\n")
    out = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True,
                         timeout=120)
    assert out.returncode == 0, out.stdout + out.stderr
    pkg = os.path.join(ROOT, "linear_recurrence_scan_row_amd")
    for dirpath, _, files in os.walk(pkg):
        for name in files:
            if name.endswith((".py", ".hip", ".hpp", ".h", ".c")):
                text = open(os.path.join(dirpath, name)).read()
                assert not re.search(r"^\s*(import|from)\s+oracle\b", text, re.M), name
                assert "liboracle" not in text, name


def test_binding_refuses_host_tensors():
    """No CPU fallback: every op of the binding, batched or not, raises on
    host tensors before anything reaches the library."""
    import torch

    import linear_recurrence_scan_row_amd as rl

    n, t = 4, 8
    r, v = torch.zeros(n, t), torch.zeros(n, t)
    f = torch.zeros(n, t, dtype=torch.uint8)
    calls = {
        "gae": lambda m: m.gae(r, v, f),
        "td_lambda": lambda m: m.td_lambda(r, v, f),
        "discounted_returns": lambda m: m.discounted_returns(r, f),
        "vtrace": lambda m: m.vtrace(r, v, r, v, f),
        "retrace": lambda m: m.retrace(r, v, v, r, v, f),
        "eligibility_traces": lambda m: m.eligibility_traces(r, f, rl.RESET_ON_START, 0.9, 0.9),
        "episodic_prefix_sum": lambda m: m.episodic_prefix_sum(r, f, rl.RESET_ON_START),
        "affine_scan": lambda m: m.affine_scan(r, v),
    }
    for name, call in calls.items():
        with pytest.raises(ValueError, match="GPU"):
            call(rl)
        with pytest.raises(ValueError, match="GPU"):
            call(rl.Batch())
    with pytest.raises(ValueError, match="GPU"):
        rl.gae_stats(r, v, f)
    with pytest.raises(ValueError, match="GPU"):
        rl.ppo_clip_loss(r, v, r)
