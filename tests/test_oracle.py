"""Pins for the CPU oracle: each check ties it to something other than itself
(library decoders, closed forms, exact rational arithmetic, numpy's fp64 / int64
matmul, invariants), so that a dropped term, a wrong sign or index, or a
transposed operand in `oracle.c` fails at least one of them."""
from fractions import Fraction
import itertools

import numpy as np
import pytest
import torch

import oracle
import synth


def _dense(M, N, K, A, B, in_dtype="bf16", C=None, c_dtype=None, alpha=1.0, beta=0.0, out="f32"):
    return dict(kind="dense", M=M, N=N, K=K, in_dtype=in_dtype, out_dtype=out, c_dtype=c_dtype,
                alpha=alpha, beta=beta, A=A, B=B, C=C)


def _bf16_to_f64(bits):
    return torch.from_numpy(np.asarray(bits, dtype=np.uint16).view(np.int16)).view(torch.bfloat16).double().numpy()


def _f16_to_f64(bits):
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


# ---------------------------------------------------------------- decoders
def test_dec_bf16_all_codes_vs_torch():
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    lib = _bf16_to_f64(codes)
    mine = np.array([oracle.dec_bf16(c) for c in codes])
    nan = np.isnan(lib)
    assert np.array_equal(np.isnan(mine), nan)
    assert np.array_equal(mine[~nan], lib[~nan])


def test_dec_f16_all_codes_vs_numpy():
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    lib = _f16_to_f64(codes)
    mine = np.array([oracle.dec_f16(c) for c in codes])
    nan = np.isnan(lib)
    assert np.array_equal(np.isnan(mine), nan)
    assert np.array_equal(mine[~nan], lib[~nan])


def test_dec_e4m3_all_codes_vs_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    lib = codes.view(torch.float8_e4m3fn).double().numpy()
    mine = np.array([oracle.dec_e4m3(c) for c in range(256)])
    nan = np.isnan(lib)
    assert nan.sum() == 2  # S.1111.111 only
    assert np.array_equal(np.isnan(mine), nan)
    assert np.array_equal(mine[~nan], lib[~nan])


def test_dec_e4m3_format_facts():
    # OCP E4M3: largest finite 448, smallest normal 2^-6, smallest subnormal 2^-9, 1.0 = 0x38
    assert oracle.dec_e4m3(0x7E) == 448.0
    assert oracle.dec_e4m3(0xFE) == -448.0
    assert oracle.dec_e4m3(0x08) == 2.0 ** -6
    assert oracle.dec_e4m3(0x01) == 2.0 ** -9
    assert oracle.dec_e4m3(0x38) == 1.0
    assert oracle.dec_e4m3(0x80) == 0.0


# ---------------------------------------------------------------- closed forms
@pytest.mark.parametrize("in_dtype", ["bf16", "f16"])
def test_identity_b(in_dtype):
    M, K = 37, 24
    a = synth.uniform((M, K), -1, 1, 1)
    A = synth.to_storage(a, in_dtype)
    B = synth.to_storage(np.eye(K, dtype=np.float32), in_dtype)
    C = synth.uniform((M, K), -1, 1, 2)
    ref, _ = oracle.gemm(_dense(M, K, K, A, B, in_dtype, C, "f32", alpha=1.5, beta=0.5))
    dec = _bf16_to_f64 if in_dtype == "bf16" else _f16_to_f64
    assert np.array_equal(ref, 1.5 * dec(A) + 0.5 * C.astype(np.float64))


def test_permutation_b():
    M, K = 19, 32
    A = synth.to_bf16_bits(synth.uniform((M, K), -1, 1, 3))
    perm = synth.rng(7).permutation(K)
    P = np.zeros((K, K), dtype=np.float32)
    P[np.arange(K), perm] = 1.0  # B[j, perm[j]] = 1  ->  D[:, j] = A[:, perm[j]]
    C = synth.to_bf16_bits(synth.uniform((M, K), -1, 1, 4))
    ref, _ = oracle.gemm(_dense(M, K, K, A, synth.to_bf16_bits(P), "bf16", C, "bf16", alpha=2.0, beta=-0.25))
    a, c = _bf16_to_f64(A), _bf16_to_f64(C)
    assert np.array_equal(ref, 2.0 * a[:, perm] + (-0.25) * c)


def test_alpha_beta_linearity():
    M, N, K = 13, 21, 40
    p = synth.dense_problem(M, N, K, "bf16", "f32", c_dtype="f32", dist="uniform", seed=11)
    r10, _ = oracle.gemm(p, alpha=1.0, beta=0.0)
    c = p["C"].astype(np.float64)
    for al, be in [(2.0, 0.5), (-0.5, 4.0), (0.25, -1.0)]:
        r, _ = oracle.gemm(p, alpha=al, beta=be)
        assert np.array_equal(r, al * r10 + be * c)


def test_beta_only_passthrough():
    M, N, K = 9, 17, 16
    for cdt in ["f32", "bf16", "f16"]:
        p = synth.dense_problem(M, N, K, "bf16", cdt, c_dtype=cdt, dist="uniform", seed=5)
        ref, absdot = oracle.gemm(p, alpha=0.0, beta=1.0)
        dec = {"f32": lambda x: x.astype(np.float64), "bf16": _bf16_to_f64, "f16": _f16_to_f64}[cdt]
        assert np.array_equal(ref, dec(p["C"]))


def test_beta_zero_ignores_c_nan():
    M, N, K = 4, 5, 8
    p = synth.dense_problem(M, N, K, "bf16", "f32", c_dtype="f32", dist="uniform", seed=6)
    p["C"] = np.full((M, N), np.nan, dtype=np.float32)
    ref, _ = oracle.gemm(p, alpha=1.0, beta=0.0)
    assert np.isfinite(ref).all()


def test_nonnegative_inputs_absdot_equals_acc():
    M, N, K = 7, 9, 64
    a = np.abs(synth.uniform((M, K), -1, 1, 8))
    b = np.abs(synth.uniform((N, K), -1, 1, 9))
    p = _dense(M, N, K, synth.to_bf16_bits(a), synth.to_bf16_bits(b))
    ref, absdot = oracle.gemm(p)
    assert np.array_equal(ref, absdot)


# ---------------------------------------------------------------- brute force, exact arithmetic
def _frac_bf16(bits):
    return [Fraction(float(v)) for v in _bf16_to_f64(bits).ravel()]


def test_bruteforce_tiny_shapes_exact_rationals():
    dims = [1, 2, 3, 5, 8, 17]
    for M, N, K in itertools.product(dims, dims, dims):
        seed = 100 + M * 1000 + N * 31 + K
        A = synth.to_bf16_bits(synth.uniform((M, K), -1, 1, seed))
        B = synth.to_bf16_bits(synth.uniform((N, K), -1, 1, seed + 1))
        C = synth.uniform((M, N), -1, 1, seed + 2)
        ref, absdot = oracle.gemm(_dense(M, N, K, A, B, "bf16", C, "f32", alpha=1.5, beta=0.5))
        fa = np.array(_frac_bf16(A), dtype=object).reshape(M, K)
        fb = np.array(_frac_bf16(B), dtype=object).reshape(N, K)
        for i in range(M):
            for j in range(N):
                exact = sum((fa[i, k] * fb[j, k] for k in range(K)), Fraction(0))
                eabs = sum((abs(fa[i, k] * fb[j, k]) for k in range(K)), Fraction(0))
                want = Fraction(3, 2) * exact + Fraction(1, 2) * Fraction(float(C[i, j]))
                assert abs(Fraction(ref[i, j]) - want) <= Fraction(2) ** -50 * (eabs + abs(want)), (M, N, K, i, j)
                assert abs(Fraction(absdot[i, j]) - eabs) <= Fraction(2) ** -50 * eabs


def test_agrees_with_numpy_fp64_matmul():
    for (M, N, K), dt in [((64, 48, 200), "bf16"), ((33, 70, 129), "f16")]:
        p = synth.dense_problem(M, N, K, dt, "f32", c_dtype="f32", alpha=0.75, beta=-2.0, dist="uniform", seed=21)
        ref, absdot = oracle.gemm(p)
        dec = _bf16_to_f64 if dt == "bf16" else _f16_to_f64
        a, b = dec(p["A"]), dec(p["B"])
        want = 0.75 * (a @ b.T) + (-2.0) * p["C"].astype(np.float64)
        assert np.all(np.abs(ref - want) <= 1e-12 * (np.abs(a) @ np.abs(b).T + 1.0))
        assert np.allclose(absdot, np.abs(a) @ np.abs(b).T, rtol=1e-12, atol=0)


def test_int8_exact_vs_numpy_int64():
    M, N, K = 40, 33, 256
    p = synth.dense_problem(M, N, K, "i8", "i32", c_dtype="i32", alpha=1.0, beta=1.0, seed=31)
    ref, _ = oracle.gemm(p)
    want = p["A"].astype(np.int64) @ p["B"].astype(np.int64).T + p["C"].astype(np.int64)
    assert np.array_equal(ref, want.astype(np.float64))


# ---------------------------------------------------------------- split invariance
def test_split_invariance_integer_valued_bitexact():
    M, N, K = 16, 24, 300
    a = synth.rng(41).integers(-8, 8, size=(M, K)).astype(np.float32)
    b = synth.rng(42).integers(-8, 8, size=(N, K)).astype(np.float32)
    p = _dense(M, N, K, synth.to_bf16_bits(a), synth.to_bf16_bits(b))
    r1, d1 = oracle.gemm(p, splits=1)
    for s in (2, 3, 7, 8, 300, 301):
        rs, ds = oracle.gemm(p, splits=s)
        assert np.array_equal(r1, rs) and np.array_equal(d1, ds)


def test_split_invariance_random_few_ulps():
    p = synth.dense_problem(8, 8, 4096, "bf16", "f32", dist="normal", seed=44)
    r1, d1 = oracle.gemm(p, splits=1)
    r8, _ = oracle.gemm(p, splits=8)
    assert np.all(np.abs(r1 - r8) <= 4096 * 2.0 ** -52 * d1)


# ---------------------------------------------------------------- int4 weight-only
def _w4(M, N, K, A_bits, words, scales_f16, group=128, zp=8, C=None, beta=0.0):
    return dict(kind="w4a16", M=M, N=N, K=K, in_dtype="bf16", out_dtype="bf16", c_dtype="f32" if C is not None else None,
                alpha=1.0, beta=beta, group=group, zero_point=zp, A=A_bits, B=words, V=scales_f16, C=C)


def test_int4_single_nibble_probes():
    # One nonzero nibble per probe: word w, nibble i -> k = 8w + i. A = one-hot rows.
    N, K = 3, 256
    M = K
    A = synth.to_bf16_bits(np.eye(K, dtype=np.float32))  # D[i, j] = b(j, i)
    s = synth.to_f16_bits(np.full((N, K // 128), 1.0, dtype=np.float32))
    for (j, w, i) in [(0, 0, 0), (1, 0, 7), (2, 5, 3), (0, 31, 7), (1, 16, 0)]:
        words = np.full((N, K // 8), 0x88888888, dtype=np.uint32)  # all nibbles = zero point
        words[j, w] = (0x88888888 & ~(0xF << (4 * i))) | (0xB << (4 * i))  # q = 11 -> value 3
        ref, _ = oracle.gemm(_w4(M, N, K, A, words, s))
        k = 8 * w + i
        expect = np.zeros((M, N))
        expect[k, j] = 3.0
        assert np.array_equal(ref, expect), (j, w, i)


def test_int4_group_scale_indexing():
    # scale of group g for row j = 2^(j + g); a single nibble at k selects group k // 128
    N, K = 2, 512
    A = synth.to_bf16_bits(np.ones((1, K), dtype=np.float32))
    s = np.array([[2.0 ** (j + g) for g in range(K // 128)] for j in range(N)], dtype=np.float32)
    for k in (0, 127, 128, 300, 511):
        words = np.full((N, K // 8), 0x88888888, dtype=np.uint32)
        for j in range(N):
            words[j, k // 8] = (0x88888888 & ~(0xF << (4 * (k % 8)))) | (0x9 << (4 * (k % 8)))  # q = 9 -> 1
        ref, _ = oracle.gemm(_w4(1, N, K, A, words, synth.to_f16_bits(s)))
        assert np.array_equal(ref[0], [2.0 ** (j + k // 128) for j in range(N)]), k


def test_int4_all_zero_point_gives_beta_c():
    M, N, K = 5, 6, 256
    A = synth.to_bf16_bits(synth.uniform((M, K), -1, 1, 51))
    words = np.full((N, K // 8), 0x88888888, dtype=np.uint32)
    s = synth.to_f16_bits(synth.uniform((N, 2), 0.005, 0.02, 52))
    C = synth.uniform((M, N), -1, 1, 53)
    ref, _ = oracle.gemm(_w4(M, N, K, A, words, s, C=C, beta=0.5))
    assert np.array_equal(ref, 0.5 * C.astype(np.float64))


def test_int4_ones_gives_rowsum():
    M, N, K = 4, 3, 384
    a = synth.uniform((M, K), -1, 1, 54)
    A = synth.to_bf16_bits(a)
    words = np.full((N, K // 8), 0x99999999, dtype=np.uint32)  # q = 9 everywhere
    s = synth.to_f16_bits(np.ones((N, 3), dtype=np.float32))
    ref, _ = oracle.gemm(_w4(M, N, K, A, words, s))
    rows = _bf16_to_f64(A).sum(axis=1)
    assert np.allclose(ref, np.repeat(rows[:, None], N, axis=1), rtol=0, atol=1e-12)


def test_int4_matches_unpacked_numpy():
    p = synth.w4a16_problem(8, 16, 512, seed=61)
    ref, absdot = oracle.gemm(p)
    words = p["B"]
    q = np.zeros((16, 512), dtype=np.int64)
    for k in range(512):
        q[:, k] = (words[:, k // 8] >> np.uint32(4 * (k % 8))) & np.uint32(15)
    s = _f16_to_f64(p["V"])
    b = (q - 8) * np.repeat(s, 128, axis=1)
    a = _bf16_to_f64(p["A"])
    assert np.allclose(ref, a @ b.T, rtol=0, atol=1e-12 * (np.abs(a) @ np.abs(b).T).max())


# ---------------------------------------------------------------- fp8 block scales
def test_fp8_block_scale_indexing():
    # U[i, g] = 2^i * 3^g style distinct scales; a single pair of codes picks exactly one U and one V
    E, N, K = 1, 256, 256
    M = 2
    A = np.zeros((M, K), dtype=np.uint8)
    B = np.zeros((E, N, K), dtype=np.uint8)
    U = np.array([[2.0 ** (i + 4 * g) for g in range(2)] for i in range(M)], dtype=np.float32)
    V = np.array([[[2.0 ** (-(nb + 2 * g)) for g in range(2)] for nb in range(2)]], dtype=np.float32)
    for (i, j, k) in [(0, 0, 0), (1, 255, 255), (0, 130, 129), (1, 7, 200)]:
        A[:] = 0
        B[:] = 0
        A[i, k] = 0x40  # 2.0
        B[0, j, k] = 0xC4  # -3.0
        p = dict(kind="grouped", M=M, N=N, K=K, E=1, offsets=np.array([0, M], dtype=np.int32),
                 counts=np.array([M]), in_dtype="e4m3", out_dtype="bf16", c_dtype=None, alpha=1.0, beta=0.0,
                 A=A, B=B, U=U, V=V, group_k=128, group_n=128)
        ref, _ = oracle.gemm(p)
        want = np.zeros((M, N))
        want[i, j] = 2.0 * -3.0 * U[i, k // 128] * V[0, j // 128, k // 128]
        assert np.array_equal(ref, want), (i, j, k)


def test_fp8_quantized_matches_numpy():
    counts = np.array([3, 0, 5], dtype=np.int32)
    p = synth.grouped_problem(counts, 256, 384, fp8=True, seed=71)
    ref, _ = oracle.gemm(p)
    dec = torch.from_numpy(np.arange(256, dtype=np.uint8)).view(torch.float8_e4m3fn).double().numpy()
    a = dec[p["A"]] * np.repeat(p["U"].astype(np.float64), 128, axis=1)
    off = p["offsets"]
    for e in range(3):
        b = dec[p["B"][e]] * np.repeat(np.repeat(p["V"][e].astype(np.float64), 128, axis=0), 128, axis=1)
        want = a[off[e]:off[e + 1]] @ b.T
        assert np.allclose(ref[off[e]:off[e + 1]], want, rtol=1e-12, atol=1e-12)


def test_fp8_dense_ragged_matches_numpy():
    # N and K not multiples of the 128 block: the last block of V and U is partial
    p = synth.dense_fp8_problem(7, 300, 400, c_dtype="f32", alpha=0.5, beta=2.0, seed=3)
    ref, _ = oracle.gemm(p)
    dec = torch.from_numpy(np.arange(256, dtype=np.uint8)).view(torch.float8_e4m3fn).double().numpy()
    K, N = 400, 300
    a = dec[p["A"]] * np.repeat(p["U"].astype(np.float64), 128, axis=1)[:, :K]
    vb = np.repeat(np.repeat(p["V"].astype(np.float64), 128, axis=0), 128, axis=1)[:N, :K]
    want = 0.5 * (a @ (dec[p["B"]] * vb).T) + 2.0 * p["C"].astype(np.float64)
    assert p["U"].shape == (7, 4) and p["V"].shape == (3, 4)
    assert np.allclose(ref, want, rtol=1e-12, atol=1e-12)


def test_fp8_dense_equals_grouped_single_expert():
    p = synth.dense_fp8_problem(9, 256, 384, seed=4)
    ref, absdot = oracle.gemm(p)
    q = dict(p, kind="grouped", E=1, offsets=np.array([0, 9], dtype=np.int32), counts=np.array([9]),
             B=p["B"][None], V=p["V"][None])
    ref_g, absdot_g = oracle.gemm(q)
    assert np.array_equal(ref, ref_g) and np.array_equal(absdot, absdot_g)


# ---------------------------------------------------------------- grouped
def test_grouped_equals_per_expert_numpy():
    counts = np.array([5, 0, 17, 1, 0, 9], dtype=np.int32)
    N, K = 40, 96
    p = synth.grouped_problem(counts, N, K, seed=81)
    ref, absdot = oracle.gemm(p)
    a = _bf16_to_f64(p["A"])
    off = p["offsets"]
    for e in range(len(counts)):
        b = _bf16_to_f64(p["B"][e])
        want = a[off[e]:off[e + 1]] @ b.T
        assert np.allclose(ref[off[e]:off[e + 1]], want, rtol=0, atol=1e-12 * max(1.0, np.abs(want).max(initial=0)))


def test_grouped_expert_permutation():
    counts = np.array([4, 7, 0, 3], dtype=np.int32)
    N, K = 16, 64
    p = synth.grouped_problem(counts, N, K, seed=82)
    ref, _ = oracle.gemm(p)
    perm = [2, 3, 0, 1]
    off = p["offsets"]
    A2 = np.concatenate([p["A"][off[e]:off[e + 1]] for e in perm])
    q = dict(p, counts=counts[perm], offsets=synth.offsets_from_counts(counts[perm]), A=A2, B=p["B"][perm])
    ref2, _ = oracle.gemm(q)
    want = np.concatenate([ref[off[e]:off[e + 1]] for e in perm])
    assert np.array_equal(ref2, want)


def test_row_sampling_matches_full():
    p = synth.dense_problem(30, 20, 64, "bf16", "bf16", c_dtype="bf16", alpha=1.0, beta=1.0, seed=91)
    full, fa = oracle.gemm(p)
    rows = [0, 29, 7, 7, 13]
    part, pa = oracle.gemm(p, rows=rows)
    assert np.array_equal(part, full[rows]) and np.array_equal(pa, fa[rows])


# ---------------------------------------------------------------- generator
def test_zipf_counts_properties():
    c = synth.zipf_counts()
    assert c.sum() == 65536 and c.max() <= 8192 and c.min() >= 0 and len(c) == 64
    assert np.array_equal(c, synth.zipf_counts())


def test_pack_int4_layout_literal():
    q = np.array([[1, 2, 3, 4, 5, 6, 7, 8, 15, 0, 0, 0, 0, 0, 0, 9]], dtype=np.int64)
    assert synth.pack_int4(q).tolist() == [[0x87654321, 0x9000000F]]


def test_batched_problem_matches_numpy_per_batch():
    # the batched generator goes through the oracle's grouped definition
    p = synth.batched_problem(3, 5, 40, 48, c_dtype="f32", alpha=0.5, beta=2.0, seed=21, share_b=True)
    ref, _ = oracle.gemm(p)
    a = _bf16_to_f64(p["A"])
    b = _bf16_to_f64(p["B"][0])
    c = p["C"].astype(np.float64)
    for e in range(3):
        rows = slice(5 * e, 5 * e + 5)
        want = 0.5 * (a[rows] @ b.T) + 2.0 * c[rows]
        assert np.allclose(ref[rows], want, rtol=1e-12, atol=1e-12)
    assert np.array_equal(p["B"][1], p["B"][0]) and np.array_equal(p["B"][2], p["B"][0])


# ---------------------------------------------------------------- fused epilogue
def _epi_problem(flags, bias=None, bias_type="f32", row_scale=None, zero_point=0.0, seed=31, M=6, N=40, K=32):
    p = synth.dense_problem(M, N, K, "bf16", "f32", c_dtype="f32", alpha=0.75, beta=0.5, dist="uniform", seed=seed)
    p["epilogue"] = dict(flags=flags, bias=bias, bias_type=bias_type, row_scale=row_scale, zero_point=zero_point)
    return p


def test_epilogue_bias_adds_per_column():
    bias = synth.uniform((40,), -2, 2, 5).astype(np.float32)
    p = _epi_problem(1, bias=bias)
    q = dict(p, epilogue=None)
    ref, _ = oracle.gemm(p)
    ref0, _ = oracle.gemm(q)
    assert np.array_equal(ref, ref0 + bias.astype(np.float64)[None, :])
    # a bf16 bias decodes like any bf16 operand
    bb = synth.to_bf16_bits(bias)
    refb, _ = oracle.gemm(_epi_problem(1, bias=bb, bias_type="bf16"))
    assert np.array_equal(refb, ref0 + _bf16_to_f64(bb)[None, :])


def test_epilogue_relu_and_gelu():
    bias = synth.uniform((40,), -2, 2, 6).astype(np.float32)
    x, _ = oracle.gemm(_epi_problem(1, bias=bias))
    relu, _ = oracle.gemm(_epi_problem(1 | 2, bias=bias))
    assert np.array_equal(relu, np.maximum(x, 0.0))
    gelu, _ = oracle.gemm(_epi_problem(1 | 4, bias=bias))
    from scipy.special import erf
    assert np.allclose(gelu, 0.5 * x * (1 + erf(x / np.sqrt(2))), rtol=1e-14, atol=1e-15)
    # closed forms: gelu(x) - gelu(-x) = x; gelu(0) = 0; gelu(x) -> x for large x, -> 0 for very negative x
    neg = _epi_problem(1 | 4, bias=-bias)
    neg["alpha"], neg["beta"] = -0.75, -0.5
    gneg, _ = oracle.gemm(neg)
    assert np.allclose(gelu - gneg, x, rtol=0, atol=1e-13)


def test_quantisation_rounding_and_saturation():
    # ref values chosen directly: ties go to even, values past the int8 range saturate
    M, N = 2, 8
    p = _epi_problem(8, row_scale=np.array([1.0, 0.5], dtype=np.float32), zero_point=0.0, M=M, N=N)
    ref = np.array([[0.5, 1.5, 2.5, -0.5, -1.5, 200.0, -300.0, 126.6],
                    [5.0, 3.0, -5.0, 1.0, 253.0, 256.0, -257.0, -258.0]])
    pre, code = oracle.quant_codes(p, ref)
    assert np.array_equal(code[0], [0, 2, 2, 0, -2, 127, -128, 127])
    assert np.array_equal(code[1], [2, 2, -2, 0, 126, 127, -128, -128])
    assert np.array_equal(pre[1], ref[1] * 0.5)
    # the zero point is added before rounding
    p["epilogue"]["zero_point"] = 3.0
    _, code3 = oracle.quant_codes(p, ref)
    assert np.array_equal(code3[0], [4, 4, 6, 2, 2, 127, -128, 127])


def test_w8a8_matches_int_sums_times_scales():
    p = synth.w8a8_problem(9, 33, 80, out_dtype="f32", c_dtype="f32", alpha=2.0, beta=0.5, seed=17)
    ref, absdot = oracle.gemm(p)
    s = p["A"].astype(np.int64) @ p["B"].astype(np.int64).T  # exact integer sums
    u = p["U"][:, 0].astype(np.float64)
    v = p["V"][:, 0].astype(np.float64)
    want = 2.0 * s * u[:, None] * v[None, :] + 0.5 * p["C"].astype(np.float64)
    assert np.allclose(ref, want, rtol=1e-13, atol=1e-13)
    assert np.allclose(absdot, (np.abs(p["A"].astype(np.int64)) @ np.abs(p["B"].astype(np.int64)).T)
                       * u[:, None] * v[None, :], rtol=1e-13)


def test_int4_asymmetric_zero_points():
    # per-group zero points: numpy dequant with Z in place of the constant
    p = synth.w4a16_problem(3, 16, 256, seed=23, asym=True)
    ref, _ = oracle.gemm(p)
    N, K = 16, 256
    words = p["B"].astype(np.uint64)
    q = np.stack([(words >> np.uint64(4 * i)) & np.uint64(15) for i in range(8)], axis=2).reshape(N, K).astype(np.int64)
    z = np.repeat(p["Z"].astype(np.int64), 128, axis=1)
    s = np.repeat(p["V"].view(np.float16).astype(np.float64), 128, axis=1)
    want = _bf16_to_f64(p["A"]) @ ((q - z) * s).T
    assert np.allclose(ref, want, rtol=1e-12, atol=1e-12)
    # a zero point equal to every nibble of its group zeroes that group's contribution
    p2 = dict(p, Z=np.zeros_like(p["Z"]))
    p2["B"] = synth.pack_int4(np.zeros((N, K), dtype=np.int64))
    ref2, _ = oracle.gemm(p2)
    assert np.array_equal(ref2, np.zeros_like(ref2))
