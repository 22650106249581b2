"""Host-side tests of the C-ABI library (no GPU needed).

The library must load, export every function include/cp_attn.h declares, and
reject bad arguments with the documented status before touching the GPU.
Only argument paths that fail validation are called here; device pointers are
fake (never dereferenced).
"""
import ctypes
import os
import subprocess

import pytest

import oracle
from long_sequence_causal_cp_amd import binding as cb

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
ALIGNED = 0x7F0000000000        # fake, 256-byte aligned device addresses
MB = 1 << 20


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(cb.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    return cb.load_library()


def fake(i):
    return ctypes.c_void_p(ALIGNED + i * 1024 * MB)


def test_every_header_function_is_exported(lib):
    names = cb.header_functions()
    assert "cp_ring_attn_fwd" in names and "cp_attn_step_fwd" in names and "cp_attn_merge" in names
    out = subprocess.run(["nm", "-D", "--defined-only", cb.LIB_PATH], capture_output=True, text=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for n in names:
        assert n in exported, n
        assert getattr(lib, n) is not None


def test_version(lib):
    assert cb.cp_version() >= 100


def test_zigzag_matches_pages_worked_example(lib):
    with open(os.path.join(GOLDEN, "zigzag_cp4.txt")) as f:
        rows = [tuple(map(int, l.split())) for l in f if l.strip() and not l.startswith("#")]
    for r, a, b in rows:
        q, kv = cb.cp_zigzag_chunks(4, r, 10, 0)
        assert q.n_chunks == 2 and q.chunk_len == 10
        assert q.starts() == [10 * a, 10 * b]
        assert kv.starts() == q.starts()


@pytest.mark.parametrize("cp", [1, 2, 4, 8, 16])
def test_zigzag_ring_matches_oracle_index_maths(lib, cp):
    L = 64
    S = 2 * cp * L
    for r in range(cp):
        for j in range(cp):
            q, kv = cb.cp_zigzag_chunks(cp, r, L, j)
            qpos = [s + i for s in q.starts() for i in range(L)]
            kpos = [s + i for s in kv.starts() for i in range(L)]
            assert qpos == list(oracle.local_positions(S, cp, r))
            assert kpos == list(oracle.ring_kv_positions(S, cp, r, j))


@pytest.mark.parametrize("args", [(0, 0, 64, 0), (2, 2, 64, 0), (2, -1, 64, 0), (2, 0, 64, 2), (2, 0, 0, 0)])
def test_zigzag_rejects_bad_arguments(lib, args):
    with pytest.raises(cb.CpError) as e:
        cb.cp_zigzag_chunks(*args)
    assert e.value.status == cb.CP_ERR_INVALID
    assert cb.cp_last_error()


def test_workspace_bytes(lib):
    B, H, Skv, D, Sq = 1, 32, 4096, 128, 4096
    kv = B * H * Skv * D * 2
    # 2 slots x 4 steps x (K, V), the fp32 running O, and the key-split partials (O and LSE of two
    # halves for at most 512 * 128 rows) with 512 counters
    R = min(512 * 128, B * H * Sq)
    split = 2 * R * D * 4 + 2 * R * 4 + 512 * 4
    assert cb.cp_ring_attn_workspace_bytes(B, H, Skv, D, Sq) == 16 * kv + B * H * Sq * D * 4 + split
    assert cb.cp_ring_attn_workspace_bytes(1, 1, 64, 64, 64) % 256 == 0
    assert cb.cp_ring_attn_workspace_bytes(0, 1, 64, 64, 64) == 0


def _step(lib, D=128, qt=None, kvt=None, scale=0.088, mode=0, q=None, o=None, lse=None, out=None, B=1, H=2):
    qt = qt or cb.CpChunks.make([0, 192], 64)
    kvt = kvt or cb.CpChunks.make([0, 192], 64)
    return lib.cp_attn_step_fwd(q or fake(0), fake(1), fake(2), o or fake(3), lse or fake(4), out,
                                B, H, D, ctypes.byref(qt), ctypes.byref(kvt), scale, mode, None)


@pytest.mark.parametrize("kw,status", [
    (dict(D=96), cb.CP_ERR_UNSUPPORTED),
    (dict(D=32), cb.CP_ERR_UNSUPPORTED),
    (dict(B=0), cb.CP_ERR_INVALID),
    (dict(scale=float("nan")), cb.CP_ERR_INVALID),
    (dict(scale=0.0), cb.CP_ERR_INVALID),
    (dict(scale=float("inf")), cb.CP_ERR_INVALID),
    (dict(mode=7), cb.CP_ERR_INVALID),
    (dict(qt=cb.CpChunks.make([0, 192], 48)), cb.CP_ERR_INVALID),        # chunk_len not multiple of 64
    (dict(qt=cb.CpChunks.make([0, 32], 64)), cb.CP_ERR_INVALID),         # overlapping chunks
    (dict(kvt=cb.CpChunks.make([-64], 64)), cb.CP_ERR_INVALID),          # negative start
    (dict(kvt=cb.CpChunks.make([2**31 - 64], 128)), cb.CP_ERR_INVALID),  # positions overflow int32
    (dict(qt=cb.CpChunks.make([], 64)), cb.CP_ERR_INVALID),              # no chunks
    (dict(q=ctypes.c_void_p(ALIGNED + 8)), cb.CP_ERR_INVALID),           # misaligned
    (dict(o=fake(0)), cb.CP_ERR_INVALID),                                # o aliases q
    (dict(out=fake(3)), cb.CP_ERR_INVALID),                              # out aliases o
])
def test_step_fwd_validation(lib, kw, status):
    assert _step(lib, **kw) == status
    assert cb.cp_last_error()


def test_step_fwd_too_many_chunks(lib):
    t = cb.CpChunks()
    t.n_chunks = 9
    t.chunk_len = 64
    assert lib.cp_attn_step_fwd(fake(0), fake(1), fake(2), fake(3), fake(4), None, 1, 1, 128,
                                ctypes.byref(t), ctypes.byref(t), 0.1, 0, None) == cb.CP_ERR_INVALID


@pytest.mark.parametrize("kw,status", [
    (dict(D=6), cb.CP_ERR_INVALID),
    (dict(B=0), cb.CP_ERR_INVALID),
    (dict(o_part=fake(0)), cb.CP_ERR_INVALID),
    (dict(o_acc=ctypes.c_void_p(ALIGNED + 4)), cb.CP_ERR_INVALID),
])
def test_merge_validation(lib, kw, status):
    a = dict(o_acc=fake(0), lse_acc=fake(1), o_part=fake(2), lse_part=fake(3), B=1, H=1, Sq=64, D=128)
    a.update(kw)
    assert lib.cp_attn_merge(a["o_acc"], a["lse_acc"], a["o_part"], a["lse_part"], a["B"], a["H"],
                             a["Sq"], a["D"], None, None) == status


def _ring(lib, n_steps=2, ws_bytes=None, copy_stream=ctypes.c_void_p(0x1234), kv_override=None,
          workspace=None, stream=None, out=None):
    L = 64
    qt = cb.CpChunks.make([0, 192], L)
    tabs = [cb.cp_zigzag_chunks(2, 0, L, j % 2)[1] for j in range(max(n_steps, 1))]
    if kv_override is not None:
        tabs[1] = kv_override
    T = cb.CpChunks * len(tabs)
    ks = (ctypes.c_void_p * len(tabs))(*[ALIGNED + (10 + j) * 1024 * MB for j in range(len(tabs))])
    vs = (ctypes.c_void_p * len(tabs))(*[ALIGNED + (40 + j) * 1024 * MB for j in range(len(tabs))])
    need = cb.cp_ring_attn_workspace_bytes(1, 2, 128, 128, 128)
    return lib.cp_ring_attn_fwd(fake(0), ctypes.byref(qt), ks, vs, T(*tabs), n_steps, out or fake(1), fake(2),
                                1, 2, 128, 0.088, workspace or fake(3), need if ws_bytes is None else ws_bytes,
                                stream, copy_stream)


def test_ring_validation(lib):
    assert _ring(lib, n_steps=0) == cb.CP_ERR_INVALID
    assert _ring(lib, n_steps=65) == cb.CP_ERR_INVALID
    assert _ring(lib, ws_bytes=1000) == cb.CP_ERR_WORKSPACE
    assert "needed" in cb.cp_last_error()
    assert _ring(lib, copy_stream=None, stream=ctypes.c_void_p(0x99)) == cb.CP_ERR_INVALID  # NULL beside a stream
    assert _ring(lib, kv_override=cb.CpChunks.make([0, 128, 192], 64)) == cb.CP_ERR_INVALID
    assert _ring(lib, workspace=ctypes.c_void_p(ALIGNED + 128)) == cb.CP_ERR_INVALID   # misaligned
    assert _ring(lib, workspace=fake(1)) == cb.CP_ERR_INVALID                           # overlaps out
    assert _ring(lib, out=fake(10)) == cb.CP_ERR_INVALID                                # out overlaps K


def _bwd(lib, D=128, mode=0, scale=0.088, B=1, H=2, qt=None, kvt=None, **ptrs):
    qt = qt or cb.CpChunks.make([0, 192], 64)
    kvt = kvt or cb.CpChunks.make([0, 192], 64)
    p = dict(q=fake(0), k=fake(1), v=fake(2), d_out=fake(3), lse=fake(4), delta=fake(5), dq=fake(6), dk=fake(7),
             dv=fake(8))
    p.update(ptrs)
    return lib.cp_attn_step_bwd(p["q"], p["k"], p["v"], p["d_out"], p["lse"], p["delta"], p["dq"], p["dk"],
                                p["dv"], B, H, D, ctypes.byref(qt), ctypes.byref(kvt), scale, mode, None)


@pytest.mark.parametrize("kw,status", [
    (dict(D=96), cb.CP_ERR_UNSUPPORTED),
    (dict(B=0), cb.CP_ERR_INVALID),
    (dict(scale=float("nan")), cb.CP_ERR_INVALID),
    (dict(mode=4), cb.CP_ERR_INVALID),
    (dict(mode=-1), cb.CP_ERR_INVALID),
    (dict(qt=cb.CpChunks.make([0, 192], 96)), cb.CP_ERR_INVALID),
    (dict(kvt=cb.CpChunks.make([0, 32], 64)), cb.CP_ERR_INVALID),
    (dict(dq=None), cb.CP_ERR_INVALID),
    (dict(delta=None), cb.CP_ERR_INVALID),
    (dict(dk=ctypes.c_void_p(ALIGNED + 7 * 1024 * MB + 8)), cb.CP_ERR_INVALID),    # misaligned
    (dict(lse=ctypes.c_void_p(ALIGNED + 4 * 1024 * MB + 2)), cb.CP_ERR_INVALID),   # misaligned
    (dict(dq=fake(0)), cb.CP_ERR_INVALID),                                         # dq aliases q
    (dict(dv=fake(4)), cb.CP_ERR_INVALID),                                         # dv aliases lse
    (dict(dv=fake(7)), cb.CP_ERR_INVALID),                                         # dv overlaps dk
])
def test_step_bwd_validation(lib, kw, status):
    assert _bwd(lib, **kw) == status
    assert cb.cp_last_error()


@pytest.mark.parametrize("args,status", [
    ((1, 1, 64, 96), cb.CP_ERR_UNSUPPORTED),
    ((0, 1, 64, 128), cb.CP_ERR_INVALID),
    ((1, 1, -1, 128), cb.CP_ERR_INVALID),
])
def test_bwd_delta_validation(lib, args, status):
    B, H, Sq, D = args
    assert lib.cp_attn_bwd_delta(fake(0), fake(1), fake(2), B, H, Sq, D, None) == status
    assert lib.cp_attn_bwd_delta(fake(0), fake(1), None, 1, 1, 64, 128, None) == cb.CP_ERR_INVALID
    assert lib.cp_attn_bwd_delta(fake(0), fake(1), fake(0), 1, 1, 64, 128, None) == cb.CP_ERR_INVALID  # overlap


def test_ring_bwd_workspace_bytes(lib):
    B, H, Skv, D, Sq = 1, 32, 4096, 128, 4096
    kv = B * H * Skv * D * 2
    assert cb.cp_ring_attn_bwd_workspace_bytes(B, H, Skv, D, Sq) == B * H * Sq * 4 + 2 * (2 * kv + 4 * kv)
    assert cb.cp_ring_attn_bwd_workspace_bytes(1, 1, 64, 64, 64) % 256 == 0
    assert cb.cp_ring_attn_bwd_workspace_bytes(1, 0, 64, 64, 64) == 0


def _ring_bwd(lib, n_steps=2, ws_bytes=None, copy_stream=ctypes.c_void_p(0x1234), stream=None, dq=None,
              dk_override=None, workspace=None, D=128, acc=None):
    L = 64
    qt = cb.CpChunks.make([0, 192], L)
    m = max(n_steps, 1)
    tabs = [cb.cp_zigzag_chunks(2, 0, L, j % 2)[1] for j in range(m)]
    T = cb.CpChunks * m
    arr = lambda base: (ctypes.c_void_p * m)(*[ALIGNED + (base + j) * 1024 * MB for j in range(m)])
    ks, vs, dks, dvs = arr(10), arr(40), arr(70), arr(100)
    if dk_override is not None:
        dks[1] = dk_override
    need = cb.cp_ring_attn_bwd_workspace_bytes(1, 2, 128, 128, 128)
    accp = None if acc is None else (ctypes.c_int * m)(*acc)
    return lib.cp_ring_attn_bwd(fake(0), ctypes.byref(qt), fake(1), fake(2), fake(3), ks, vs, T(*tabs), n_steps,
                                dks, dvs, accp, dq or fake(4), 1, 2, D, 0.088, workspace or fake(5),
                                need if ws_bytes is None else ws_bytes, stream, copy_stream)


def test_ring_bwd_validation(lib):
    assert _ring_bwd(lib, n_steps=0) == cb.CP_ERR_INVALID
    assert _ring_bwd(lib, n_steps=65) == cb.CP_ERR_INVALID
    assert _ring_bwd(lib, D=96) == cb.CP_ERR_UNSUPPORTED
    assert _ring_bwd(lib, ws_bytes=1000) == cb.CP_ERR_WORKSPACE
    assert "needed" in cb.cp_last_error()
    assert _ring_bwd(lib, copy_stream=None, stream=ctypes.c_void_p(0x99)) == cb.CP_ERR_INVALID
    assert _ring_bwd(lib, workspace=ctypes.c_void_p(ALIGNED + 128)) == cb.CP_ERR_INVALID      # misaligned
    assert _ring_bwd(lib, workspace=fake(4)) == cb.CP_ERR_INVALID                              # overlaps dq
    assert _ring_bwd(lib, dq=fake(0)) == cb.CP_ERR_INVALID                                     # dq aliases q
    assert _ring_bwd(lib, dk_override=ALIGNED + 70 * 1024 * MB) == cb.CP_ERR_INVALID           # two steps share dK
    assert _ring_bwd(lib, dk_override=ALIGNED + 10 * 1024 * MB) == cb.CP_ERR_INVALID           # dK aliases K
    assert _ring_bwd(lib, dk_override=ALIGNED + 70 * 1024 * MB + 8) == cb.CP_ERR_INVALID       # misaligned
    assert cb.cp_last_error()


def test_empty_merge_and_delta_need_no_pointers(lib):
    # zero rows: nothing to do, NULL pointers accepted, no device call made
    assert lib.cp_attn_merge(None, None, None, None, 1, 1, 0, 128, None, None) == cb.CP_OK
    assert lib.cp_attn_bwd_delta(None, None, None, 1, 1, 0, 128, None) == cb.CP_OK


@pytest.mark.parametrize("kw,status", [
    (dict(D=64), cb.CP_ERR_UNSUPPORTED),
    (dict(qt=cb.CpChunks.make([0, 192], 64)), cb.CP_ERR_UNSUPPORTED),      # q chunks not a multiple of 128
    (dict(vs=0.0), cb.CP_ERR_INVALID),
    (dict(qs=float("nan")), cb.CP_ERR_INVALID),
    (dict(mode=3), cb.CP_ERR_INVALID),
    (dict(o=fake(0)), cb.CP_ERR_INVALID),                                   # o aliases q
])
def test_step_fwd_fp8_validation(lib, kw, status):
    a = dict(D=128, qt=cb.CpChunks.make([0, 768], 256), kvt=cb.CpChunks.make([0, 768], 256), qs=0.5, ks=0.5,
             vs=0.5, mode=0, o=None)
    a.update(kw)
    assert lib.cp_attn_step_fwd_fp8(fake(0), fake(1), fake(2), a["o"] or fake(3), fake(4), None, 1, 2, a["D"],
                                    ctypes.byref(a["qt"]), ctypes.byref(a["kvt"]), 0.088, a["qs"], a["ks"],
                                    a["vs"], a["mode"], None) == status
    assert cb.cp_last_error()


def test_ring_fwd_fp8_validation(lib):
    L = 256
    qt = cb.CpChunks.make([0, 3 * L], L)
    tabs = [cb.cp_zigzag_chunks(2, 0, L, j)[1] for j in range(2)]
    T = cb.CpChunks * 2
    ks = (ctypes.c_void_p * 2)(*[ALIGNED + (10 + j) * 1024 * MB for j in range(2)])
    vs = (ctypes.c_void_p * 2)(*[ALIGNED + (40 + j) * 1024 * MB for j in range(2)])
    need = cb.cp_ring_attn_fwd_fp8_workspace_bytes(1, 2, 2 * L, 128, 2 * L)
    assert need == 16 * 2 * 2 * L * 128 + 2 * 2 * L * 128 * 4

    def call(D=128, ws=need, q_tab=qt, vscale=0.5):
        return lib.cp_ring_attn_fwd_fp8(fake(0), ctypes.byref(q_tab), ks, vs, T(*tabs), 2, fake(1), fake(2), 1, 2, D,
                                        0.088, 0.5, 0.5, vscale, fake(3), ws, None, ctypes.c_void_p(0x1234))
    assert call(D=64) == cb.CP_ERR_UNSUPPORTED
    assert call(q_tab=cb.CpChunks.make([0, 192], 64)) == cb.CP_ERR_UNSUPPORTED
    assert call(ws=need - 1) == cb.CP_ERR_WORKSPACE
    assert call(vscale=-1.0) == cb.CP_ERR_INVALID
    assert cb.cp_last_error()


def test_test_delay_hook_validation(lib):
    for bad in ((-1, 0), (0, -1), (100001, 0), (0, 10 ** 6)):
        assert lib.cp_test_set_delays(*bad) == cb.CP_ERR_INVALID
        assert cb.cp_last_error()
    assert lib.cp_test_set_delays(0, 0) == cb.CP_OK


def test_zigzag_rejects_sequences_past_int32(lib):
    # chunk tables hold positions below 2^31 - 1 (start + chunk_len <= 2^31 - 1)
    for n, L in ((1 << 16, 1 << 15), (1 << 14, 1 << 16)):      # 2^32 and 2^31 positions
        with pytest.raises(cb.CpError):
            cb.cp_zigzag_chunks(n, 0, L, 0)
    n, L = 1 << 14, (1 << 16) - 1                               # 2^31 - 2^15 positions
    q, _ = cb.cp_zigzag_chunks(n, n - 1, L, 0)
    assert q.starts() == [(n - 1) * L, n * L]


def test_profile_read_named_when_empty(lib):
    assert cb.cp_profile_read_named() == []


def test_ring_plan_query(lib):
    """The published plan of the 32K cp=8 share, rank 0: step 0 alone, then steps 1-3 and 4-7; chunk 0
    (positions 0..2047) sees only its own block and finishes at step 0; chunk 15 is written at step 0,
    merged in both groups and finalised by the last."""
    q, _ = cb.cp_zigzag_chunks(8, 0, 2048, 0)
    kv = [cb.cp_zigzag_chunks(8, 0, 2048, j)[1] for j in range(8)]
    A, M, W, F = cb.CP_PLAN_ACTIVE, cb.CP_PLAN_MERGE, cb.CP_PLAN_WRITE_O, cb.CP_PLAN_FINALIZE
    assert cb.cp_ring_attn_fwd_plan(q, kv) == [(0, 1, {0: A | F, 1: A | W}), (1, 3, {1: A | M | W}),
                                               (4, 4, {1: A | M | F})]
    with pytest.raises(cb.CpError):
        cb.cp_ring_attn_fwd_plan(q, [])
