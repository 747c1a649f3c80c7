"""CPU tests of libqgemm.so's C ABI: exported symbols, argument validation,
planning, the dispatch cache's export/import and the tuning sequence.

No call here reaches a kernel launch: every qg_run request is rejected during
validation (fake device addresses are never dereferenced), and plans come from
qg_plan, which never touches the device."""
import ctypes
import os
import re

import pytest

import quantized_gemm_bf16_amd as qg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 1 << 20  # aligned, never dereferenced


def header_functions():
    text = open(os.path.join(ROOT, "include", "qgemm.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qg_[a-z_]+)\s*\(", text)))


def test_every_declared_function_is_exported():
    names = header_functions()
    assert len(names) >= 14
    lib = ctypes.CDLL(qg.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(qg.EXPORTS)


def test_measurement_library_exports_its_header():
    from quantized_gemm_bf16_amd import ceiling
    text = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "qgceil.h")).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(qgc_[a-z_]+)\s*\(", text)))
    lib = ctypes.CDLL(ceiling.CEIL_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(ceiling.EXPORTS)


def test_measurement_library_rejects_bad_arguments():
    # every rejection happens before a launch
    from quantized_gemm_bf16_amd import ceiling
    L = ceiling.lib
    assert L.qgc_mfma_loop(0, 1, FAKE, FAKE, None) == qg.ERR_INVALID_ARG
    assert L.qgc_mfma_loop(1, 0, FAKE, FAKE, None) == qg.ERR_INVALID_ARG
    assert L.qgc_mfma_loop(1, 1, None, FAKE, None) == qg.ERR_INVALID_ARG
    assert L.qgc_stream_read(FAKE, 15, 1, FAKE, None) == qg.ERR_INVALID_ARG
    assert L.qgc_stream_read(FAKE + 4, 16, 1, FAKE, None) == qg.ERR_INVALID_ARG
    assert L.qgc_stream_read(FAKE, 1 << 31, 1, FAKE, None) == qg.ERR_INVALID_ARG
    assert L.qgc_stream_read(FAKE, 16, 65536, FAKE, None) == qg.ERR_INVALID_ARG
    for mode, kind, grid, iters in ((0, 0, 1, 1), (4, 0, 1, 1), (2, 3, 1, 1), (2, -1, 1, 1), (1, 0, 0, 1),
                                    (1, 0, 65536, 1), (1, 0, 1, 0), (1, 0, 1, (1 << 20) + 1)):
        assert L.qgc_issue_mix(mode, kind, grid, iters, FAKE, FAKE, None) == qg.ERR_INVALID_ARG
    assert L.qgc_issue_mix(1, 0, 1, 1, None, FAKE, None) == qg.ERR_INVALID_ARG
    assert L.qgc_issue_mix(1, 0, 1, 1, FAKE, None, None) == qg.ERR_INVALID_ARG
    out = ctypes.c_double()
    assert L.qgc_host_us_per_empty(0, 0, None, ctypes.byref(out)) == qg.ERR_INVALID_ARG
    assert L.qgc_host_us_per_empty(1, 8, None, ctypes.byref(out)) == qg.ERR_INVALID_ARG
    assert L.qgc_host_us_per_call(None, 1, None, None, 0.0, None, None, None, None, None, None, None, None, 0.0,
                                  None, None, None, None, None, None, ctypes.byref(out)) == qg.ERR_INVALID_ARG


def test_constants_and_strings():
    assert qg.barriers_size() == 1 << 20
    assert qg.partials_size() == 32 << 20
    assert qg.version().startswith("qgemm")
    assert qg.status_str(0) == "ok"
    assert "workspace" in qg.status_str(qg.ERR_WORKSPACE)
    names = qg.kernel_names()
    assert len(names) == qg.lib.qg_kernel_count() and len(set(names)) == len(names)
    assert qg.lib.qg_kernel_name(-1) is None and qg.lib.qg_kernel_name(len(names)) is None


@pytest.fixture(scope="module")
def g():
    return qg.Gemm()


def ws_desc(b=1 << 20, p=32 << 20):
    return qg.Workspace(FAKE, b, FAKE, p)


def dense(M, N, K, t="bf16", out="bf16"):
    return qg.layout(t, M, K), qg.layout(t, N, K), qg.layout(out, M, N)


def run(g, op=None, alpha=1.0, A=FAKE, Ad=None, B=FAKE, Bd=None, beta=0.0, C=None, Cd=None, D=FAKE, Dd=None,
        U=None, Ud=None, V=None, Vd=None, ws=None):
    return g.run_raw(op or qg.operation(), alpha, A, Ad, U, Ud, B, Bd, V, Vd, beta, C, Cd, D, Dd, ws, stream=None)


def test_invalid_arguments(g):
    Ad, Bd, Dd = dense(64, 64, 64)
    assert run(g, Ad=None, Bd=Bd, Dd=Dd) == qg.ERR_INVALID_ARG
    assert run(g, Ad=Ad, Bd=Bd, Dd=Dd, A=None) == qg.ERR_INVALID_ARG
    assert run(g, Ad=Ad, Bd=Bd, Dd=Dd, D=None) == qg.ERR_INVALID_ARG
    # shape mismatch
    assert run(g, Ad=Ad, Bd=qg.layout("bf16", 64, 32), Dd=Dd) == qg.ERR_INVALID_ARG
    assert run(g, Ad=Ad, Bd=Bd, Dd=qg.layout("bf16", 64, 65)) == qg.ERR_INVALID_ARG
    # ld smaller than the row
    assert run(g, Ad=qg.layout("bf16", 64, 64, ld=32), Bd=Bd, Dd=Dd) == qg.ERR_INVALID_ARG
    # beta != 0 without C
    assert run(g, Ad=Ad, Bd=Bd, Dd=Dd, beta=1.0) == qg.ERR_INVALID_ARG
    # non-finite scalars
    assert run(g, Ad=Ad, Bd=Bd, Dd=Dd, alpha=float("nan")) == qg.ERR_INVALID_ARG
    # a bad policy
    assert run(g, op=qg.operation(policy=9), Ad=Ad, Bd=Bd, Dd=Dd) == qg.ERR_INVALID_ARG
    assert qg.lib.qg_run(None, None, 1.0, None, None, None, None, None, None, None, None, 0.0, None, None, None,
                         None, None, None) == qg.ERR_INVALID_ARG


def test_alignment(g):
    Ad, Bd, Dd = dense(64, 64, 64)
    assert run(g, Ad=Ad, Bd=Bd, Dd=Dd, A=FAKE + 2) == qg.ERR_ALIGNMENT
    assert run(g, Ad=Ad, Bd=Bd, Dd=Dd, D=FAKE + 8) == qg.ERR_ALIGNMENT
    # rows not a multiple of 16 bytes
    assert run(g, Ad=qg.layout("bf16", 64, 60), Bd=qg.layout("bf16", 64, 60), Dd=Dd) == qg.ERR_ALIGNMENT
    assert run(g, Ad=qg.layout("bf16", 64, 64, ld=68), Bd=Bd, Dd=Dd) == qg.ERR_ALIGNMENT


@pytest.mark.parametrize("t, K, ld", [("bf16", 100, 104), ("f16", 6, 8), ("i8", 40, 48), ("i8", 1, 16)])
def test_k_need_not_fill_16_byte_chunks(g, t, K, ld):
    # only pointers and row pitches must be 16-byte aligned: a K whose last
    # chunk is partial is planned like any other (its bytes past K are zeroed
    # on chip)
    out = "i32" if t == "i8" else "bf16"
    Ad, Bd, Dd = qg.layout(t, 64, K, ld=ld), qg.layout(t, 96, K, ld=ld), qg.layout(out, 64, 96, ld=96)
    assert "kernel=" in g.plan(qg.operation(), Ad, None, Bd, None, None, Dd, 1.0, 0.0, ws_desc())
    # ...but the pitch still has to be
    with pytest.raises(RuntimeError):
        g.plan(qg.operation(), qg.layout(t, 64, K, ld=K), None, qg.layout(t, 96, K, ld=K), None, None, Dd, 1.0,
               0.0, ws_desc())


def test_unsupported(g):
    Ad, Bd, Dd = dense(64, 64, 64)
    assert run(g, Ad=qg.layout("bf16", 64, 64, order=qg.COL_MAJOR), Bd=Bd, Dd=Dd) == qg.ERR_UNSUPPORTED
    assert run(g, Ad=Ad, Bd=qg.layout("f16", 64, 64), Dd=Dd) == qg.ERR_UNSUPPORTED
    assert run(g, Ad=Ad, Bd=Bd, Dd=qg.layout("i32", 64, 64)) == qg.ERR_UNSUPPORTED
    i8 = dense(64, 64, 64, "i8", "i32")
    assert run(g, Ad=i8[0], Bd=i8[1], Dd=i8[2], alpha=2.0) == qg.ERR_UNSUPPORTED
    Cd = qg.layout("i32", 64, 64)
    assert run(g, Ad=i8[0], Bd=i8[1], Dd=i8[2], beta=0.5, C=FAKE, Cd=Cd) == qg.ERR_UNSUPPORTED
    assert run(g, Ad=i8[0], Bd=i8[1], Dd=qg.layout("f32", 64, 64)) == qg.ERR_UNSUPPORTED
    assert run(g, op=qg.operation(quant_a=(qg.QUANT_INT4_ZP, 128, 1, 8)), Ad=Ad, Bd=Bd, Dd=Dd) == qg.ERR_UNSUPPORTED


def test_workspace_checks(g):
    Ad, Bd, Dd = dense(16, 4096, 14336)
    op = qg.operation(policy=qg.POLICY_FORCE, schedule=qg.SCHED_SPLITK, split_k=8)
    assert run(g, op=op, Ad=Ad, Bd=Bd, Dd=Dd, ws=None) == qg.ERR_WORKSPACE
    assert run(g, op=op, Ad=Ad, Bd=Bd, Dd=Dd, ws=ws_desc(p=1024)) == qg.ERR_WORKSPACE
    assert run(g, op=op, Ad=Ad, Bd=Bd, Dd=Dd, ws=ws_desc(b=16)) == qg.ERR_WORKSPACE
    # DEFAULT policy without a workspace falls back to a data-parallel plan
    desc = g.plan(qg.operation(), Ad, None, Bd, None, None, Dd, 1.0, 0.0, None)
    assert "schedule=dp" in desc


def test_run_timed_argument_checks(g):
    # qg_run_timed: split-K and data-parallel plans, a stamps buffer of
    # 8 x 8 bytes per unit; the unit count comes back even when the buffer is
    # short
    Ad, Bd, Dd = dense(16, 4096, 14336)
    op = qg.operation(policy=qg.POLICY_FORCE, schedule=qg.SCHED_SPLITK, split_k=8)

    def timed(op, stamps, cap, ws=ws_desc()):
        return g.run_timed_raw(op, 1.0, FAKE, Ad, None, None, FAKE, Bd, None, None, 0.0, None, None, FAKE, Dd, ws,
                               stamps, cap)
    d = dict(kv.split("=") for kv in g.plan(op, Ad, None, Bd, None, None, Dd, 1.0, 0.0, ws_desc()).split())
    units = int(d["tiles"]) * 8
    assert timed(op, FAKE, units - 1) == (qg.ERR_INVALID_ARG, units)
    assert timed(op, None, units) == (qg.ERR_INVALID_ARG, units)
    assert timed(op, FAKE + 4, units) == (qg.ERR_INVALID_ARG, units)
    # a valid request: without a GPU the handle is offline
    st, n = timed(op, FAKE, units)
    assert n == units and st in (qg.ERR_HIP, qg.OK)
    # data-parallel: one unit per tile
    dp = qg.operation(policy=qg.POLICY_FORCE, schedule=qg.SCHED_DP)
    tiles = int(dict(kv.split("=") for kv in g.plan(dp, Ad, None, Bd, None, None, Dd, 1.0, 0.0,
                                                     ws_desc()).split())["tiles"])
    assert timed(dp, FAKE, tiles - 1) == (qg.ERR_INVALID_ARG, tiles)
    st, n = timed(dp, FAKE, tiles)
    assert n == tiles and st in (qg.ERR_HIP, qg.OK)
    # stream-K, measuring, or nothing to launch
    sk = qg.operation(policy=qg.POLICY_FORCE, schedule=qg.SCHED_STREAMK, programs=64)
    assert timed(sk, FAKE, 1 << 20)[0] == qg.ERR_UNSUPPORTED
    assert timed(qg.operation(policy=qg.POLICY_MEASURE), FAKE, 1 << 20)[0] == qg.ERR_UNSUPPORTED
    Ad0, Bd0, Dd0 = dense(0, 4096, 14336)
    assert g.run_timed_raw(op, 1.0, FAKE, Ad0, None, None, FAKE, Bd0, None, None, 0.0, None, None, FAKE, Dd0,
                           ws_desc(), FAKE, 1 << 20)[0] == qg.ERR_UNSUPPORTED
    # the request itself is validated first
    assert timed(op, FAKE, units, ws=ws_desc(p=1024))[0] == qg.ERR_WORKSPACE


def test_plan_decode_split8(g):
    Ad, Bd, Dd = dense(16, 4096, 14336)
    op = qg.operation(policy=qg.POLICY_FORCE, schedule=qg.SCHED_SPLITK, split_k=8)
    d = dict(kv.split("=") for kv in g.plan(op, Ad, None, Bd, None, None, Dd, 1.0, 0.0, ws_desc()).split())
    assert d["schedule"] == "splitk" and d["split"] == "8"
    assert int(d["grid"]) == int(d["tiles"]) * 8
    assert int(d["partials"]) <= 32 << 20 and int(d["barriers"]) <= 1 << 20


def test_plan_streamk_matches_planner(g):
    M, N, K = 16, 4096, 14336
    Ad, Bd, Dd = dense(M, N, K)
    op = qg.operation(policy=qg.POLICY_FORCE, schedule=qg.SCHED_STREAMK, programs=256)
    d = dict(kv.split("=") for kv in g.plan(op, Ad, None, Bd, None, None, Dd, 1.0, 0.0, ws_desc()).split())
    assert d["schedule"] == "streamk" and d["programs"] == "256" and d["grid"] == "256"
    bm, bn, bk = int(d["bm"]), int(d["bn"]), int(d["bk"])
    assert int(d["tiles"]) == -(-M // bm) * -(-N // bn)
    assert int(d["partials"]) == 2 * 256 * bm * bn * 4
    assert int(d["barriers"]) == int(d["tiles"]) * 4


# ---------------------------------------------------------------- stream-K division
# (tiles, iters, programs): fewer tiles than programs, a multiple of the
# program count, ragged waves, one iteration per tile, more programs than
# iterations, and the decode / 4096^3 shapes
SK_SHAPES = [(32, 112, 256), (512, 16, 256), (300, 7, 256), (100, 9, 7), (1, 1, 256), (13, 1, 5),
             (3, 2, 8), (25, 64, 13), (256, 64, 256), (1024, 64, 256), (37, 11, 37), (1000, 3, 64)]


@pytest.mark.parametrize("shape", SK_SHAPES)
def test_streamk_covers_every_iteration_once(shape):
    T, I, P = shape
    units = qg.streamk_units(T, I, P)
    seen = {}
    for (p, t, kb, ke, slot) in units:
        assert 0 <= p < P and 0 <= t < T and 0 <= kb < ke <= I
        for k in range(kb, ke):
            assert (t, k) not in seen, f"iteration {(t, k)} owned twice"
            seen[(t, k)] = p
    assert len(seen) == T * I


@pytest.mark.parametrize("shape", SK_SHAPES)
def test_streamk_balance_and_slots(shape):
    T, I, P = shape
    units = qg.streamk_units(T, I, P)
    per_prog = {}
    whole = {}
    slots = set()
    for (p, t, kb, ke, slot) in units:
        per_prog[p] = per_prog.get(p, 0) + (ke - kb)
        if slot < 0:
            assert kb == 0 and ke == I
            whole[p] = whole.get(p, 0) + 1
        else:
            assert not (kb == 0 and ke == I), "a whole tile must be stored directly"
            assert slot in (2 * p, 2 * p + 1) and slot not in slots
            slots.add(slot)
    work = [per_prog.get(p, 0) for p in range(P)]
    # every program gets the same whole-tile count before the shared region and
    # a balanced share of it, so total work differs by at most one iteration
    assert max(work) - min(work) <= 1
    if T % P == 0:
        assert all(s < 0 for (*_, s) in units)
    # each program's units come out in execution order: whole tiles, then its
    # shared range in increasing iteration order
    for p in range(P):
        mine = [(t, kb, ke) for (q, t, kb, ke, _) in units if q == p]
        flat = [t * I + kb for (t, kb, ke) in mine]
        assert flat == sorted(flat)


@pytest.mark.parametrize("shape", SK_SHAPES)
def test_streamk_fixup_order_matches_pieces(shape):
    # the completing workgroup sums a shared tile's pieces in k order; the
    # slots it reads must be exactly the slots its pieces were written to
    T, I, P = shape
    units = qg.streamk_units(T, I, P)
    pieces = {}
    for (p, t, kb, ke, slot) in units:
        if slot >= 0:
            pieces.setdefault(t, []).append((kb, ke, slot))
    for t, lst in pieces.items():
        lst.sort()
        assert lst[0][0] == 0 and lst[-1][1] == I
        assert all(a[1] == b[0] for a, b in zip(lst, lst[1:]))
        assert qg.streamk_fixup(T, I, P, t) == [s for (_, _, s) in lst]


def test_streamk_decode_shape_all_shared():
    # 32 tiles of 112 iterations over 256 programs: 14 iterations each, every
    # tile shared by 8 programs
    units = qg.streamk_units(32, 112, 256)
    assert len(units) == 256 and all(ke - kb == 14 and s >= 0 for (_, _, kb, ke, s) in units)
    assert all(len(qg.streamk_fixup(32, 112, 256, t)) == 8 for t in range(32))


def test_streamk_units_argument_checks():
    n = ctypes.c_int()
    assert qg.lib.qg_streamk_units(4, 0, 2, None, 0, ctypes.byref(n)) == qg.ERR_INVALID_ARG
    assert qg.lib.qg_streamk_units(4, 3, 2, None, 0, None) == qg.ERR_INVALID_ARG
    assert qg.lib.qg_streamk_units(4, 3, 3, None, 0, ctypes.byref(n)) == qg.ERR_BUFFER_SMALL and n.value > 0
    assert qg.lib.qg_streamk_fixup(4, 3, 3, 4, None, 0, ctypes.byref(n)) == qg.ERR_INVALID_ARG


def test_plan_square_uses_one_wave_of_big_tiles(g):
    Ad, Bd, Dd = dense(4096, 4096, 4096)
    d = dict(kv.split("=") for kv in g.plan(qg.operation(), Ad, None, Bd, None, None, Dd, 1.0, 0.0, ws_desc()).split())
    assert d["schedule"] == "dp" and d["kernel"].startswith("tile_BF16_256x256")
    assert d["tiles"] == "256"


def test_plan_zero_sized(g):
    Ad, Bd, Dd = dense(0, 64, 64)
    assert "grid=0" in g.plan(qg.operation(), Ad, None, Bd, None, None, Dd, 1.0, 0.0, None)
    assert run(g, Ad=Ad, Bd=Bd, Dd=Dd) == qg.OK  # nothing to do, nothing launched


def test_tuning_sequence(g):
    seq = g.tuning_seq()
    assert seq[0] == 1 and seq == sorted(seq) and 16 in seq and 4096 in seq and len(seq) == len(set(seq))


CACHE = """qgemm-cache 2 arch=gfx950 entries=2
16|bf16.bf16.-.bf16.q00.e0.x0.n4096.k14336 kernel=tile_BF16_32x64x128b_w1x2_s6 schedule=splitk split=4 programs=0 us=20.5
4096|bf16.bf16.-.bf16.q00.e0.x0.n4096.k4096 kernel=tile_BF16_128x128x128b_w2x2_s4 schedule=dp split=1 programs=0 us=90
"""


def test_cache_import_export_roundtrip_and_lookup():
    g = qg.Gemm()
    assert g.cache_size() == 0
    assert g.import_(CACHE) == qg.OK
    assert g.cache_size() == 2
    out = g.export()
    assert out.splitlines()[0] == "qgemm-cache 2 arch=gfx950 entries=2"
    assert sorted(out.splitlines()[1:]) == sorted(CACHE.splitlines()[1:])
    g2 = qg.Gemm()
    assert g2.import_(out) == qg.OK and g2.export() == out
    # the DEFAULT policy uses the cached choice, also for an M that maps to the same bucket
    Ad, Bd, Dd = dense(16, 4096, 14336)
    assert "kernel=tile_BF16_32x64x128b_w1x2_s6 schedule=splitk split=4" in g.plan(qg.operation(), Ad, None, Bd, None, None, Dd, 1.0, 0.0, ws_desc())
    Ad, Bd, Dd = dense(11, 4096, 14336)
    assert "kernel=tile_BF16_32x64x128b_w1x2_s6" in g.plan(qg.operation(), Ad, None, Bd, None, None, Dd, 1.0, 0.0, ws_desc())
    # REUSE misses where nothing is cached
    Ad, Bd, Dd = dense(16, 2048, 2048)
    with pytest.raises(qg.QGemmError) as e:
        g.plan(qg.operation(policy=qg.POLICY_REUSE), Ad, None, Bd, None, None, Dd, 1.0, 0.0, ws_desc())
    assert e.value.status == qg.ERR_NO_KERNEL


@pytest.mark.parametrize("bad", [
    "",
    "nonsense\n",
    "qgemm-cache 1 arch=gfx950 entries=0\n",
    "qgemm-cache 2 arch=gfx942 entries=0\n",
    CACHE.replace("entries=2", "entries=3"),
    CACHE.replace("kernel=tile_BF16_32x64x128b_w1x2_s6", "kernel=no_such_kernel"),
    CACHE.replace("schedule=dp", "schedule=zigzag"),
    CACHE.replace("split=4", "split=x"),
    CACHE.replace("us=90", "us=90 extra"),
    CACHE.replace("us=90", "us=-90"),
    CACHE.replace("us=90", "us=nan"),
    CACHE.replace("us=90", "us=inf"),
    CACHE[: len(CACHE) // 2],
])
def test_cache_import_is_all_or_nothing(bad):
    g = qg.Gemm()
    assert g.import_(CACHE) == qg.OK
    before = g.export()
    assert g.import_(bad) == qg.ERR_FORMAT
    assert g.export() == before


def test_export_buffer_too_small():
    g = qg.Gemm()
    assert g.import_(CACHE) == qg.OK
    n = ctypes.c_size_t()
    assert qg.lib.qg_export(g.h, None, 0, ctypes.byref(n)) == qg.OK
    buf = ctypes.create_string_buffer(4)
    assert qg.lib.qg_export(g.h, buf, 4, ctypes.byref(n)) == qg.ERR_BUFFER_SMALL
    assert n.value == len(g.export()) + 1


def test_w4a16_validation(g):
    M, N, K = 64, 512, 1024
    Ad = qg.layout("bf16", M, K)
    Bd = qg.layout("u4", N, K)  # ld = K/8 words
    Dd = qg.layout("bf16", M, N)
    Vd = qg.layout("f16", N, K // 128)
    q = qg.operation(quant_b=(qg.QUANT_INT4_ZP, 128, 1, 8))
    # missing scales
    assert run(g, op=q, Ad=Ad, Bd=Bd, Dd=Dd) == qg.ERR_INVALID_ARG
    # wrong group size / K not a multiple of the group
    q64 = qg.operation(quant_b=(qg.QUANT_INT4_ZP, 64, 1, 8))
    assert run(g, op=q64, Ad=Ad, Bd=Bd, Dd=Dd, V=FAKE, Vd=qg.layout("f16", N, K // 64)) == qg.ERR_UNSUPPORTED
    # scale shape mismatch, misaligned scale rows
    assert run(g, op=q, Ad=Ad, Bd=Bd, Dd=Dd, V=FAKE, Vd=qg.layout("f16", N, K // 128 + 1)) == qg.ERR_INVALID_ARG
    assert run(g, op=q, Ad=Ad, Bd=Bd, Dd=Dd, V=FAKE, Vd=qg.layout("f16", N, 8, ld=12)) == qg.ERR_ALIGNMENT
    # u4 without the quant descriptor, fp16 A
    assert run(g, Ad=Ad, Bd=Bd, Dd=Dd, V=FAKE, Vd=Vd) == qg.ERR_UNSUPPORTED
    assert run(g, op=q, Ad=qg.layout("f16", M, K), Bd=Bd, Dd=Dd, V=FAKE, Vd=Vd) == qg.ERR_UNSUPPORTED
    # a valid request plans onto the int4 kernel with split-K
    d = dict(kv.split("=") for kv in g.plan(q, Ad, None, Bd, Vd, None, Dd, 1.0, 0.0, ws_desc()).split())
    assert d["kernel"].startswith("w4_BF16_") and d["bk"] == "256"


def test_fp8_block_scaled_validation(g):
    M, N, K = 96, 384, 640
    Ad = qg.layout("e4m3", M, K)
    Bd = qg.layout("e4m3", N, K)
    Dd = qg.layout("bf16", M, N)
    Ud = qg.layout("f32", M, K // 128, ld=8)
    Vd = qg.layout("f32", N // 128, K // 128, ld=8)
    q = qg.operation(quant_a=(qg.QUANT_BLOCK_F32, 128, 1, 0), quant_b=(qg.QUANT_BLOCK_F32, 128, 128, 0))
    ok = dict(Ad=Ad, Bd=Bd, Dd=Dd, U=FAKE, Ud=Ud, V=FAKE, Vd=Vd)
    # missing scales, or quant descriptors that are not 1x128 / 128x128 blocks
    assert run(g, op=q, Ad=Ad, Bd=Bd, Dd=Dd) == qg.ERR_INVALID_ARG
    assert run(g, **ok) == qg.ERR_UNSUPPORTED
    q_bad = qg.operation(quant_a=(qg.QUANT_BLOCK_F32, 128, 128, 0), quant_b=(qg.QUANT_BLOCK_F32, 128, 128, 0))
    assert run(g, op=q_bad, **ok) == qg.ERR_UNSUPPORTED
    q_bad = qg.operation(quant_a=(qg.QUANT_BLOCK_F32, 64, 1, 0), quant_b=(qg.QUANT_BLOCK_F32, 64, 128, 0))
    assert run(g, op=q_bad, **ok) == qg.ERR_UNSUPPORTED
    # scale shapes: U rows = M, V rows = ceil(N / 128), both ceil(K / 128) columns
    assert run(g, op=q, **{**ok, "Ud": qg.layout("f32", M - 1, K // 128, ld=8)}) == qg.ERR_INVALID_ARG
    assert run(g, op=q, **{**ok, "Vd": qg.layout("f32", N // 128 + 1, K // 128, ld=8)}) == qg.ERR_INVALID_ARG
    assert run(g, op=q, **{**ok, "Ud": qg.layout("f16", M, K // 128, ld=8)}) == qg.ERR_UNSUPPORTED
    # scale row pitch must be 16-byte aligned
    assert run(g, op=q, **{**ok, "Ud": qg.layout("f32", M, K // 128, ld=5)}) == qg.ERR_ALIGNMENT
    # e4m3 A with a bf16 B
    assert run(g, op=q, **{**ok, "Bd": qg.layout("bf16", N, K)}) == qg.ERR_UNSUPPORTED
    # a valid request plans onto a block-scaled fp8 kernel with 128-deep k-tiles
    d = dict(kv.split("=") for kv in g.plan(q, Ad, Ud, Bd, Vd, None, Dd, 1.0, 0.0, ws_desc()).split())
    assert d["kernel"].startswith("f8_E4M3_") and d["bk"] == "128"
    # grouped: V carries one scale matrix per expert
    off = FAKE
    Ag = qg.layout("e4m3", M, K, num=4, offsets=off)
    Bg = qg.layout("e4m3", N, K, num=4, stride=N * K)
    Dg = qg.layout("bf16", M, N, num=4, offsets=off)
    Ug = qg.layout("f32", M, K // 128, ld=8, num=4, offsets=off)
    Vg = qg.layout("f32", N // 128, K // 128, ld=8, num=4, stride=3 * 8)
    d = dict(kv.split("=") for kv in g.plan(q, Ag, Ug, Bg, Vg, None, Dg, 1.0, 0.0, ws_desc()).split())
    assert d["kernel"].startswith("f8_E4M3_") and d["schedule"] == "grouped"
    Vshort = qg.layout("f32", N // 128, K // 128, ld=8, num=4, stride=3 * 8 - 4)
    with pytest.raises(qg.QGemmError) as e:
        g.plan(q, Ag, Ug, Bg, Vshort, None, Dg, 1.0, 0.0, ws_desc())
    assert e.value.status == qg.ERR_INVALID_ARG


def test_batched_validation_and_plan(g):
    E, M, N, K = 4, 100, 256, 512
    Ad = qg.layout("bf16", M, K, num=E, stride=M * K)
    Bd = qg.layout("bf16", N, K, num=E, stride=N * K)
    Dd = qg.layout("bf16", M, N, num=E, stride=M * N)
    d = dict(kv.split("=") for kv in g.plan(qg.operation(), Ad, None, Bd, None, None, Dd, 1.0, 0.0, ws_desc()).split())
    assert d["schedule"] == "batched" and int(d["tiles"]) > 0
    # one shared B (stride 0) is accepted
    g.plan(qg.operation(), Ad, None, qg.layout("bf16", N, K, num=E, stride=0), None, None, Dd, 1.0, 0.0, ws_desc())
    # batch counts must agree; A/C/D batches must be back to back
    assert run(g, Ad=Ad, Bd=qg.layout("bf16", N, K, num=E - 1, stride=N * K), Dd=Dd) == qg.ERR_INVALID_ARG
    assert run(g, Ad=Ad, Bd=Bd, Dd=qg.layout("bf16", M, N, num=E - 1, stride=M * N)) == qg.ERR_INVALID_ARG
    assert run(g, Ad=qg.layout("bf16", M, K, num=E, stride=M * K + 8), Bd=Bd, Dd=Dd) == qg.ERR_UNSUPPORTED
    assert run(g, Ad=Ad, Bd=Bd, Dd=Dd, beta=1.0, C=FAKE, Cd=qg.layout("bf16", M, N, num=E, stride=M * N + 8)) == \
        qg.ERR_UNSUPPORTED
    # B stride shorter than one B
    assert run(g, Ad=Ad, Bd=qg.layout("bf16", N, K, num=E, stride=N * K - 8), Dd=Dd) == qg.ERR_INVALID_ARG
    # the int4 path is not batched
    q = qg.operation(quant_b=(qg.QUANT_INT4_ZP, 128, 1, 8))
    assert run(g, op=q, Ad=Ad, Bd=qg.layout("u4", N, K, num=E, stride=N * K // 8), Dd=Dd, V=FAKE,
               Vd=qg.layout("f16", N, K // 128, num=E, stride=N * K // 128)) == qg.ERR_UNSUPPORTED


def test_struct_layouts_match_the_header(tmp_path):
    # compile a probe against include/qgemm.h and compare sizes and offsets with the ctypes mirrors
    src = tmp_path / "layout.c"
    src.write_text("""
#include <stdio.h>
#include <stddef.h>
#include "qgemm.h"
int main(void) {
  printf("layout %zu %zu %zu %zu\\n", sizeof(qg_layout), offsetof(qg_layout, num), offsetof(qg_layout, offsets),
         offsetof(qg_layout, stride));
  printf("quant %zu\\n", sizeof(qg_quant));
  printf("epi %zu %zu %zu\\n", sizeof(qg_epilogue_args), offsetof(qg_epilogue_args, row_scale),
         offsetof(qg_epilogue_args, zero_point));
  printf("op %zu %zu %zu %zu\\n", sizeof(qg_operation), offsetof(qg_operation, schedule),
         offsetof(qg_operation, kernel), offsetof(qg_operation, epi));
  printf("ws %zu %zu\\n", sizeof(qg_workspace), offsetof(qg_workspace, partials));
  return 0;
}
""")
    import subprocess
    exe = tmp_path / "layout"
    subprocess.check_call(["gcc", "-std=c11", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)])
    got = dict((l.split()[0], [int(x) for x in l.split()[1:]]) for l in subprocess.check_output([str(exe)]).decode().splitlines())
    C = ctypes
    assert got["layout"] == [C.sizeof(qg.Layout), qg.Layout.num.offset, qg.Layout.offsets.offset, qg.Layout.stride.offset]
    assert got["quant"] == [C.sizeof(qg.Quant)]
    assert got["epi"] == [C.sizeof(qg.EpilogueArgs), qg.EpilogueArgs.row_scale.offset, qg.EpilogueArgs.zero_point.offset]
    assert got["op"] == [C.sizeof(qg.Operation), qg.Operation.schedule.offset, qg.Operation.kernel.offset,
                         qg.Operation.epi.offset]
    assert got["ws"] == [C.sizeof(qg.Workspace), qg.Workspace.partials.offset]


def test_epilogue_validation(g):
    Ad, Bd, Dd = dense(64, 64, 64)
    E = qg
    assert run(g, op=qg.operation(epilogue=E.EPI_RELU | E.EPI_GELU), Ad=Ad, Bd=Bd, Dd=Dd) == qg.ERR_INVALID_ARG
    assert run(g, op=qg.operation(epilogue=E.EPI_BIAS), Ad=Ad, Bd=Bd, Dd=Dd) == qg.ERR_INVALID_ARG
    assert run(g, op=qg.operation(epilogue=E.EPI_BIAS, bias=FAKE + 4), Ad=Ad, Bd=Bd, Dd=Dd) == qg.ERR_ALIGNMENT
    assert run(g, op=qg.operation(epilogue=E.EPI_BIAS, bias=FAKE, bias_type="i32"), Ad=Ad, Bd=Bd, Dd=Dd) == \
        qg.ERR_UNSUPPORTED
    q = qg.operation(epilogue=E.EPI_QUANT_I8, row_scale=FAKE)
    assert run(g, op=q, Ad=Ad, Bd=Bd, Dd=Dd) == qg.ERR_UNSUPPORTED                 # D must be int8
    assert run(g, Ad=Ad, Bd=Bd, Dd=qg.layout("i8", 64, 64)) == qg.ERR_UNSUPPORTED  # int8 D needs QUANT_I8
    d = g.plan(q, Ad, None, Bd, None, None, qg.layout("i8", 64, 64), 1.0, 0.0, ws_desc())
    assert d.startswith("kernel=")
    i8 = dense(64, 64, 64, "i8", "i32")
    assert run(g, op=qg.operation(epilogue=E.EPI_RELU), Ad=i8[0], Bd=i8[1], Dd=i8[2]) == qg.ERR_UNSUPPORTED


def test_w8a8_validation(g):
    M, N, K = 64, 128, 256
    Ad, Bd = qg.layout("i8", M, K), qg.layout("i8", N, K)
    Dd = qg.layout("bf16", M, N)
    Ud, Vd = qg.layout("f32", M, 1, ld=1), qg.layout("f32", N, 1, ld=1)
    q = qg.operation(quant_a=(qg.QUANT_BLOCK_F32, 0, 1, 0), quant_b=(qg.QUANT_BLOCK_F32, 0, 1, 0))
    ok = dict(Ad=Ad, Bd=Bd, Dd=Dd, U=FAKE, Ud=Ud, V=FAKE, Vd=Vd)
    d = dict(kv.split("=") for kv in g.plan(q, Ad, Ud, Bd, Vd, None, Dd, 1.0, 0.0, ws_desc()).split())
    assert d["kernel"].startswith(("tile_I8_", "skinny_I8_"))
    # scales shorter than a whole row of K, or per block of rows, are not this path
    q_bad = qg.operation(quant_a=(qg.QUANT_BLOCK_F32, 128, 1, 0), quant_b=(qg.QUANT_BLOCK_F32, 0, 1, 0))
    assert run(g, op=q_bad, **ok) == qg.ERR_UNSUPPORTED
    q_bad = qg.operation(quant_a=(qg.QUANT_BLOCK_F32, 0, 4, 0), quant_b=(qg.QUANT_BLOCK_F32, 0, 1, 0))
    assert run(g, op=q_bad, **ok) == qg.ERR_UNSUPPORTED
    # missing / misshaped / misaligned scales
    assert run(g, op=q, Ad=Ad, Bd=Bd, Dd=Dd) == qg.ERR_INVALID_ARG
    assert run(g, op=q, **{**ok, "Ud": qg.layout("f32", M - 1, 1, ld=1)}) == qg.ERR_INVALID_ARG
    assert run(g, op=q, **{**ok, "V": FAKE + 2}) == qg.ERR_ALIGNMENT
    # an int32 D belongs to the exact path, not to scaled sums
    assert run(g, op=q, **{**ok, "Dd": qg.layout("i32", M, N)}) == qg.ERR_UNSUPPORTED


def test_w4a16_asymmetric_zero_point_validation(g):
    M, N, K = 64, 512, 1024
    Ad, Bd, Dd = qg.layout("bf16", M, K), qg.layout("u4", N, K), qg.layout("bf16", M, N)
    Vd = qg.layout("f16", N, K // 128)
    q = qg.operation(quant_b=(qg.QUANT_INT4_ZP, 128, 1, 8))
    base = dict(op=q, Ad=Ad, Bd=Bd, Dd=Dd, V=FAKE, Vd=Vd)
    Ud = qg.layout("i8", N, K // 128, ld=16)
    assert g.plan(q, Ad, Ud, Bd, Vd, None, Dd, 1.0, 0.0, ws_desc()).startswith("kernel=w4_")
    assert run(g, **base, U=FAKE) == qg.ERR_INVALID_ARG                            # U without its layout
    assert run(g, **base, U=FAKE, Ud=qg.layout("f16", N, K // 128, ld=16)) == qg.ERR_UNSUPPORTED
    assert run(g, **base, U=FAKE, Ud=qg.layout("i8", N, K // 128 + 1, ld=16)) == qg.ERR_INVALID_ARG
    assert run(g, **base, U=FAKE, Ud=qg.layout("i8", N, K // 128, ld=8)) == qg.ERR_ALIGNMENT
