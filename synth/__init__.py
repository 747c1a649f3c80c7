"""Seeded synthetic inputs for the GEMM engine and for the CPU oracle.

This module draws the random operands, encodes them into the storage formats
the engine reads (bf16 / fp16 bit patterns, OCP fp8 E4M3 codes with fp32
block scales, int4 nibbles packed eight to a uint32 word, int8, expert row
offsets) and holds none of the GEMM's arithmetic. Both the GPU path and the
oracle consume exactly the arrays built here.

Conventions (the pages leave them open; the plainest readings are taken):
  * "N(0, x)" means standard deviation x.
  * numpy PCG64 generators; values are sampled in fp32 and rounded to
    nearest-even into the storage type.
  * default seeds: A = 42, B = 43, C = 44, scales = 45, expert counts = 46.
  * B is always stored N x K, K-contiguous.
  * int4 packing: element k = 8*w + i of a row lives in bits [4i, 4i+4) of
    that row's uint32 word w; a row holds K/8 words.
  * fp8 quantisation: scale s = amax / 448 over the block (s = 1 when the
    block is all zero), code = RNE(x / s) saturated to +-448.
"""
from __future__ import annotations

import numpy as np
import torch

SEED_A, SEED_B, SEED_C, SEED_S, SEED_COUNTS = 42, 43, 44, 45, 46

# dtype names shared with the engine's enumeration (by name, not by code)
F32, F16, BF16, E4M3, I8, I32, U4 = "f32", "f16", "bf16", "e4m3", "i8", "i32", "u4"


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


# ---------------------------------------------------------------------------
# encoders: fp32 samples -> storage bit patterns (round to nearest even)
# ---------------------------------------------------------------------------
def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def to_f16_bits(x: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).view(np.uint16).copy()


def to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == BF16:
        return to_bf16_bits(x)
    if dtype == F16:
        return to_f16_bits(x)
    if dtype == F32:
        return np.ascontiguousarray(x, dtype=np.float32)
    raise ValueError(dtype)


def e4m3_codes(x: np.ndarray) -> np.ndarray:
    """RNE encode into OCP E4M3 (fn) codes, saturating at +-448."""
    xs = np.clip(np.asarray(x, dtype=np.float32), -448.0, 448.0)
    t = torch.from_numpy(np.ascontiguousarray(xs)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy().copy()


def _block_scales(x: np.ndarray, gm: int, gk: int) -> np.ndarray:
    """amax/448 over (gm x gk) blocks of a 2-D array (ragged edges allowed)."""
    R, K = x.shape
    nr, nk = -(-R // gm), -(-K // gk)
    s = np.ones((nr, nk), dtype=np.float32)
    for bi in range(nr):
        blk_rows = np.abs(x[bi * gm:(bi + 1) * gm])
        for bk in range(nk):
            amax = float(blk_rows[:, bk * gk:(bk + 1) * gk].max(initial=0.0))
            if amax > 0.0:
                s[bi, bk] = np.float32(amax) / np.float32(448.0)
    return s


def quantize_e4m3(x: np.ndarray, gm: int, gk: int):
    """Quantise a 2-D fp32 array into e4m3 codes with one fp32 scale per
    (gm x gk) block. Returns (codes uint8 [R, K], scales fp32 [ceil(R/gm), ceil(K/gk)])."""
    x = np.asarray(x, dtype=np.float32)
    s = _block_scales(x, gm, gk)
    full = np.repeat(np.repeat(s, gm, axis=0)[: x.shape[0]], gk, axis=1)[:, : x.shape[1]]
    return e4m3_codes(x / full), s


def pack_int4(q: np.ndarray) -> np.ndarray:
    """Pack nibbles q[N, K] (0..15, K % 8 == 0) into uint32 words [N, K/8]."""
    q = np.asarray(q, dtype=np.uint32)
    N, K = q.shape
    assert K % 8 == 0
    q = q.reshape(N, K // 8, 8)
    w = np.zeros((N, K // 8), dtype=np.uint32)
    for i in range(8):
        w |= (q[:, :, i] & np.uint32(0xF)) << np.uint32(4 * i)
    return w


# ---------------------------------------------------------------------------
# distributions
# ---------------------------------------------------------------------------
def uniform(shape, lo, hi, seed) -> np.ndarray:
    return rng(seed).uniform(lo, hi, size=shape).astype(np.float32)


def normal(shape, std, seed) -> np.ndarray:
    return (rng(seed).standard_normal(size=shape, dtype=np.float32) * np.float32(std)).astype(np.float32)


def int8_uniform(shape, seed) -> np.ndarray:
    return rng(seed).integers(-128, 128, size=shape, dtype=np.int64).astype(np.int8)


def zipf_counts(E=64, total=65536, s=1.1, cap=8192, seed=SEED_COUNTS) -> np.ndarray:
    """Per-expert row counts: multinomial(total, p_i ~ i^-s) assigned to experts by
    a seeded permutation, then capped at `cap` (top-k routing of `cap` tokens can
    give an expert at most `cap` rows) with the excess handed to uncapped experts
    in proportion to their Zipf weight. Sum stays `total`."""
    g = rng(seed)
    ranks = np.arange(1, E + 1, dtype=np.float64)
    p = ranks ** (-s)
    p /= p.sum()
    c = g.multinomial(total, p).astype(np.int64)
    perm = g.permutation(E)
    w = np.empty(E)
    counts = np.empty(E, dtype=np.int64)
    counts[perm] = c
    w[perm] = p
    while counts.max() > cap:
        excess = int(np.clip(counts - cap, 0, None).sum())
        counts = np.minimum(counts, cap)
        free = counts < cap
        share = w * free
        share /= share.sum()
        add = np.floor(share * excess).astype(np.int64)
        rem = excess - int(add.sum())
        order = np.argsort(-share, kind="stable")
        for i in order[:rem]:
            add[i] += 1
        counts = counts + add
    assert counts.sum() == total
    return counts.astype(np.int32)


def offsets_from_counts(counts: np.ndarray) -> np.ndarray:
    off = np.zeros(len(counts) + 1, dtype=np.int32)
    off[1:] = np.cumsum(counts)
    return off


# ---------------------------------------------------------------------------
# problems: dict of storage arrays + metadata understood by tests and bench
# ---------------------------------------------------------------------------
def dense_problem(M, N, K, in_dtype=BF16, out_dtype=BF16, c_dtype=None, alpha=1.0, beta=0.0,
                  dist="normal", a_std=None, b_std=None, c_std=1.0, seed=SEED_A):
    """A [M,K], B [N,K] in `in_dtype`; C [M,N] in `c_dtype` (None: no C).
    dist 'normal': A ~ N(0,a_std), B ~ N(0,b_std) (default 1/sqrt(K)), C ~ N(0,c_std).
    dist 'uniform': A, B, C ~ U[-1, 1]. dist 'int8': U{-128..127} int8, C int32."""
    sa, sb, sc = seed, seed + (SEED_B - SEED_A), seed + (SEED_C - SEED_A)
    p = dict(kind="dense", M=M, N=N, K=K, in_dtype=in_dtype, out_dtype=out_dtype,
             c_dtype=c_dtype, alpha=float(alpha), beta=float(beta))
    if dist == "int8" or in_dtype == I8:
        p["A"] = int8_uniform((M, K), sa)
        p["B"] = int8_uniform((N, K), sb)
        if c_dtype is not None:
            p["C"] = rng(sc).integers(-(1 << 20), 1 << 20, size=(M, N), dtype=np.int64).astype(np.int32)
        return p
    if dist == "uniform":
        a, b = uniform((M, K), -1, 1, sa), uniform((N, K), -1, 1, sb)
        c = uniform((M, N), -1, 1, sc) if c_dtype else None
    else:
        std = 1.0 / np.sqrt(K) if K > 0 else 1.0
        a = normal((M, K), a_std if a_std is not None else std, sa)
        b = normal((N, K), b_std if b_std is not None else std, sb)
        c = normal((M, N), c_std, sc) if c_dtype else None
    p["A"] = to_storage(a, in_dtype)
    p["B"] = to_storage(b, in_dtype)
    if c_dtype is not None:
        p["C"] = to_storage(c, c_dtype)
    return p


def dense_fp8_problem(M, N, K, out_dtype=BF16, c_dtype=None, alpha=1.0, beta=0.0, seed=SEED_A,
                      a_std=1.0, b_std=0.02, c_std=1.0, gk=128, gn_b=128):
    """Block-scaled fp8 GEMM: A ~ N(0,a_std) quantised per (row, 128-k) group -> U [M, K/128];
    B ~ N(0,b_std) per 128x128 block -> V [N/128, K/128]; codes e4m3. C [M,N] ~ N(0,c_std)."""
    a = normal((M, K), a_std, seed)
    b = normal((N, K), b_std, seed + (SEED_B - SEED_A))
    qa, su = quantize_e4m3(a, 1, gk)
    qb, sv = quantize_e4m3(b, gn_b, gk)
    p = dict(kind="dense", M=M, N=N, K=K, in_dtype=E4M3, out_dtype=out_dtype, c_dtype=c_dtype,
             alpha=float(alpha), beta=float(beta), A=qa, B=qb, U=su, V=sv, group_k=gk, group_n=gn_b)
    if c_dtype is not None:
        p["C"] = to_storage(normal((M, N), c_std, seed + (SEED_C - SEED_A)), c_dtype)
    return p


def w8a8_problem(M, N, K, out_dtype=BF16, c_dtype=None, alpha=1.0, beta=0.0, seed=SEED_A, s_lo=0.001, s_hi=0.01):
    """int8 A [M,K], B [N,K] uniform over [-128, 127] with fp32 scales per row of
    A (U [M, 1]) and per row of B (V [N, 1]) ~ U[s_lo, s_hi]; C ~ N(0, 1)."""
    p = dict(kind="dense", M=M, N=N, K=K, in_dtype=I8, out_dtype=out_dtype, c_dtype=c_dtype,
             alpha=float(alpha), beta=float(beta), w8a8=True,
             A=int8_uniform((M, K), seed), B=int8_uniform((N, K), seed + 1),
             U=uniform((M, 1), s_lo, s_hi, seed + 3), V=uniform((N, 1), s_lo, s_hi, seed + 4))
    if c_dtype is not None:
        p["C"] = to_storage(normal((M, N), 1.0, seed + 2), c_dtype)
    return p


def w4a16_problem(M, N, K, group=128, seed=SEED_A, out_dtype=BF16, a_std=1.0,
                  s_lo=0.005, s_hi=0.02, zero_point=8, asym=False, zp_cols=(), zp_groups=()):
    """A bf16 [M,K] ~ N(0,a_std); B int4 nibbles uniform 0..15 packed [N, K/8];
    V fp16 scales [N, K/group] ~ U[s_lo, s_hi]; asym: per-group zero points
    Z int8 [N, K/group] uniform 0..15 instead of the constant zero_point.
    zp_cols / zp_groups (column, group): nibbles set equal to the column's
    zero point over the whole column / one group (weights that dequantise to
    zero, as in pruned output channels)."""
    a = normal((M, K), a_std, seed)
    q = rng(seed + 1).integers(0, 16, size=(N, K), dtype=np.int64)
    G = -(-K // group)
    s = uniform((N, G), s_lo, s_hi, seed + 3)
    z = rng(seed + 5).integers(0, 16, size=(N, G), dtype=np.int64) if asym else np.full((N, G), zero_point)
    for n in zp_cols:
        for g in range(G):
            q[n, g * group:(g + 1) * group] = z[n, g]
    for (n, g) in zp_groups:
        q[n, g * group:(g + 1) * group] = z[n, g]
    p = dict(kind="w4a16", M=M, N=N, K=K, in_dtype=BF16, out_dtype=out_dtype, c_dtype=None,
             alpha=1.0, beta=0.0, group=group, zero_point=zero_point,
             A=to_bf16_bits(a), B=pack_int4(q), V=to_f16_bits(s))
    if asym:
        p["Z"] = z.astype(np.int8)
    return p


def grouped_problem(counts, N, K, in_dtype=BF16, out_dtype=BF16, seed=SEED_A, a_std=1.0, b_std=0.02,
                    fp8=False, gk=128, gn_b=128):
    """MoE grouped GEMM: A [sum(counts), K], B [E, N, K], offsets [E+1].
    fp8=True: A quantised per (row, 128-k) group -> U [rows, K/128]; B per 128x128 block
    -> V [E, N/128, K/128]; codes in e4m3."""
    counts = np.asarray(counts, dtype=np.int32)
    E, rows = len(counts), int(counts.sum())
    off = offsets_from_counts(counts)
    a = normal((rows, K), a_std, seed)
    b = normal((E, N, K), b_std, seed + 1)
    p = dict(kind="grouped", M=rows, N=N, K=K, E=E, counts=counts, offsets=off,
             in_dtype=E4M3 if fp8 else in_dtype, out_dtype=out_dtype, c_dtype=None,
             alpha=1.0, beta=0.0)
    if fp8:
        qa, su = quantize_e4m3(a, 1, gk)
        qb = np.empty((E, N, K), dtype=np.uint8)
        sv = np.empty((E, -(-N // gn_b), -(-K // gk)), dtype=np.float32)
        for e in range(E):
            qb[e], sv[e] = quantize_e4m3(b[e], gn_b, gk)
        p.update(A=qa, B=qb, U=su, V=sv, group_k=gk, group_n=gn_b)
    else:
        p.update(A=to_storage(a, in_dtype), B=to_storage(b.reshape(E * N, K), in_dtype).reshape(E, N, K))
    return p


def batched_problem(batch, M, N, K, in_dtype=BF16, out_dtype=BF16, c_dtype=None, alpha=1.0, beta=0.0,
                    seed=SEED_A, share_b=False, fp8=False, a_std=1.0, b_std=0.02):
    """Batched GEMM: `batch` products of the same M x N x K shape. Stored as a
    grouped problem with `batch` groups of M rows (A [batch*M, K], B [batch, N, K],
    C/D [batch*M, N]) and flagged `batched`; share_b: every batch uses B[0]."""
    counts = np.full(batch, M, dtype=np.int32)
    if in_dtype == I8:
        p = dict(kind="grouped", M=batch * M, N=N, K=K, E=batch, counts=counts,
                 offsets=offsets_from_counts(counts), in_dtype=I8, out_dtype=I32, c_dtype=None,
                 alpha=1.0, beta=0.0, A=int8_uniform((batch * M, K), seed),
                 B=int8_uniform((batch, N, K), seed + 1))
        if c_dtype is not None:
            p["C"] = rng(seed + 2).integers(-(1 << 20), 1 << 20, size=(batch * M, N), dtype=np.int64).astype(np.int32)
            p.update(c_dtype=I32, beta=float(beta))
    else:
        p = grouped_problem(counts, N, K, in_dtype=in_dtype, out_dtype=out_dtype, seed=seed, a_std=a_std,
                            b_std=b_std, fp8=fp8)
        p.update(alpha=float(alpha), beta=float(beta))
        if c_dtype is not None:
            p["C"] = to_storage(normal((batch * M, N), 1.0, seed + 2), c_dtype)
            p["c_dtype"] = c_dtype
    if share_b:
        p["B"] = np.ascontiguousarray(np.broadcast_to(p["B"][:1], p["B"].shape))
        if fp8:
            p["V"] = np.ascontiguousarray(np.broadcast_to(p["V"][:1], p["V"].shape))
    p.update(batched=True, share_b=share_b, batch_M=M)
    return p


# ---------------------------------------------------------------------------
# the five workloads the engine is measured and checked on
# ---------------------------------------------------------------------------
def config_tiny():
    """256^3 bf16, uniform[-1,1], C fp32, alpha 1.5, beta 0.5, fp32 out."""
    return dense_problem(256, 256, 256, BF16, F32, c_dtype=F32, alpha=1.5, beta=0.5, dist="uniform")


def config_square(dtype=BF16, n=4096):
    """n^3, A,B ~ N(0, 1/sqrt(K)), alpha 1, beta 0, out in the input type."""
    return dense_problem(n, n, n, dtype, dtype, c_dtype=None, alpha=1.0, beta=0.0)


def config_decode(M=16, N=4096, K=14336):
    """skinny decode GEMM: A,B ~ N(0,0.02), C bf16 ~ N(0,1), alpha = beta = 1, bf16 out."""
    return dense_problem(M, N, K, BF16, BF16, c_dtype=BF16, alpha=1.0, beta=1.0,
                         a_std=0.02, b_std=0.02, c_std=1.0)


def config_w4a16(M=64, N=8192, K=8192):
    return w4a16_problem(M, N, K)


def config_moe(fp8=False, E=64, N=2048, K=7168, total=65536, cap=8192):
    return grouped_problem(zipf_counts(E, total, 1.1, cap), N, K, fp8=fp8)
