"""Helpers for GPU parity tests: upload seeded inputs, call the engine through
the C ABI binding, read results back, compare with the fp64 oracle. `Run` is
also what bench.py drives; it does not touch the oracle (only
check_against_oracle imports it)."""
import numpy as np
import torch

import quantized_gemm_bf16_amd as qg

_TORCH_OUT = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16, "i32": torch.int32,
              "i8": torch.int8}


def dev(arr):
    """numpy array (any bit pattern) -> contiguous device tensor holding the same bytes."""
    a = np.ascontiguousarray(arr)
    if not a.flags.writeable:  # e.g. a broadcast view; torch wants a writable buffer
        a = a.copy()
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    elif a.dtype == np.uint32:
        a = a.view(np.int32)
    return torch.from_numpy(a).to("cuda")


def host_f64(t):
    return t.detach().to("cpu").to(torch.float64).numpy() if t.dtype != torch.int32 else t.cpu().numpy().astype(np.float64)


def decode_c(p):
    if p.get("C") is None:
        return None
    c = p["C"]
    if p["c_dtype"] == "bf16":
        return torch.from_numpy(c.view(np.int16)).view(torch.bfloat16).double().numpy()
    if p["c_dtype"] == "f16":
        return c.view(np.float16).astype(np.float64)
    return c.astype(np.float64)


def kind_of(p):
    return p["kind"]


# What the row padding past K holds when a test stores A and B with ld > K:
# NaN codes for the float formats (a NaN that reached an MFMA would poison the
# output), and for int8 extreme values of opposite sign in A and B (a product
# of two unmasked padding bytes adds -16256 to the sum).
_PAD_A = {"bf16": 0x7FC0, "f16": 0x7E00, "e4m3": 0x7F, "i8": 127}
_PAD_B = {"bf16": 0x7FC0, "f16": 0x7E00, "e4m3": 0x7F, "i8": -128}


def pad_k(x, ldk, fill):
    """Copy of x (last axis K) with rows of ldk elements; elements K..ldk-1 hold `fill`."""
    out = np.full(x.shape[:-1] + (ldk,), fill, dtype=x.dtype)
    out[..., :x.shape[-1]] = x
    return out


class Run:
    """Uploads a problem once; `run(op)` launches and returns D on the host."""

    def __init__(self, gemm, p, ws=None, out_dtype=None, ldk=None):
        """ldk: row pitch of A and B in elements (dense and grouped problems),
        with the padding past K filled with NaN codes / extreme int8 values."""
        self.g, self.p = gemm, p
        self.ws = ws
        self.out = out_dtype or p["out_dtype"]
        M, N, K = p["M"], p["N"], p["K"]
        self.ldk = ldk or K
        if ldk:
            assert p["kind"] in ("dense", "grouped") and not p.get("batched") and ldk >= K
            self.A = dev(pad_k(p["A"], ldk, _PAD_A[p["in_dtype"]]))
            self.B = dev(pad_k(p["B"], ldk, _PAD_B[p["in_dtype"]]))
        else:
            self.A = dev(p["A"])
            self.B = dev(p["B"])
        # C and D rows are padded to a 16-byte row pitch (8 elements; 16 for int8 D)
        self.ldn = -(-N // 16) * 16 if self.out == "i8" else -(-N // 8) * 8
        self.C = None
        if p.get("C") is not None:
            cp = np.zeros((M, self.ldn), dtype=p["C"].dtype)
            cp[:, :N] = p["C"]
            self.C = dev(cp)
        # scale rows padded to a 16-byte pitch
        self.U = None
        if p.get("U") is not None:
            U = p["U"]
            self.ldu = -(-U.shape[1] // 4) * 4
            Up = np.zeros((U.shape[0], self.ldu), dtype=U.dtype)
            Up[:, :U.shape[1]] = U
            self.U = dev(Up)
        self.V = None
        if p.get("V") is not None:
            V = p["V"]
            per = 8 if V.dtype == np.uint16 else 4
            self.ldv = -(-V.shape[-1] // per) * per
            Vp = np.zeros(V.shape[:-1] + (self.ldv,), dtype=V.dtype)
            Vp[..., :V.shape[-1]] = V
            self.V = dev(Vp)
        self.D = torch.full((M, self.ldn), float("nan"), dtype=_TORCH_OUT[self.out], device="cuda") \
            if self.out not in ("i32", "i8") else torch.full((M, self.ldn), -7, dtype=_TORCH_OUT[self.out], device="cuda")
        kind = p["kind"]
        if p.get("batched"):
            # batched: every descriptor gives ONE batch; A/C/D batches back to back
            E, Mb = p["E"], p["batch_M"]
            nb = 1 if p.get("share_b") else E
            if p.get("share_b"):
                self.B = dev(p["B"][0])
            self.Ad = qg.layout(p["in_dtype"], Mb, K, num=E, stride=Mb * K)
            self.Bd = qg.layout(p["in_dtype"], N, K, num=E, stride=0 if nb == 1 else N * K)
            self.Dd = qg.layout(self.out, Mb, N, ld=self.ldn, num=E, stride=Mb * self.ldn)
        elif kind == "grouped":
            E = p["E"]
            self.off = dev(np.asarray(p["offsets"], dtype=np.int32))
            self.Ad = qg.layout(p["in_dtype"], M, K, ld=self.ldk, num=E, offsets=self.off.data_ptr())
            self.Bd = qg.layout(p["in_dtype"], N, K, ld=self.ldk, num=E, stride=N * self.ldk)
            self.Dd = qg.layout(self.out, M, N, ld=self.ldn, num=E, offsets=self.off.data_ptr())
        else:
            bt = "u4" if kind == "w4a16" else p["in_dtype"]
            self.Ad = qg.layout(p["in_dtype"], M, K, ld=self.ldk)
            self.Bd = qg.layout(bt, N, K, ld=self.ldk if bt != "u4" else None)
            self.Dd = qg.layout(self.out, M, N, ld=self.ldn)
        self.Cd = qg.layout(p["c_dtype"], M, N, ld=self.ldn) if self.C is not None else None
        if p.get("batched") and self.C is not None:
            self.Cd = qg.layout(p["c_dtype"], p["batch_M"], N, ld=self.ldn, num=p["E"], stride=p["batch_M"] * self.ldn)
        self.Ud = self.Vd = None
        if kind == "w4a16":
            self.Vd = qg.layout("f16", N, p["V"].shape[1], ld=self.ldv)
            if p.get("Z") is not None:  # per-group zero points, rows padded to 16 bytes
                Z = p["Z"]
                ldz = -(-Z.shape[1] // 16) * 16
                Zp = np.zeros((Z.shape[0], ldz), dtype=np.int8)
                Zp[:, :Z.shape[1]] = Z
                self.U = dev(Zp)
                self.Ud = qg.layout("i8", N, Z.shape[1], ld=ldz)
        if p.get("U") is not None and p.get("batched"):
            nb, kg = p["V"].shape[1], p["V"].shape[2]
            Mb = p["batch_M"]
            if p.get("share_b"):
                self.V = self.V[:1].contiguous()
            self.Ud = qg.layout("f32", Mb, p["U"].shape[1], ld=self.ldu, num=p["E"], stride=Mb * self.ldu)
            self.Vd = qg.layout("f32", nb, kg, ld=self.ldv, num=p["E"], stride=0 if p.get("share_b") else nb * self.ldv)
        elif p.get("U") is not None and kind == "grouped":
            nb, kg = p["V"].shape[1], p["V"].shape[2]
            self.Ud = qg.layout("f32", M, p["U"].shape[1], ld=self.ldu, num=p["E"], offsets=self.off.data_ptr())
            self.Vd = qg.layout("f32", nb, kg, ld=self.ldv, num=p["E"], stride=nb * self.ldv)
        elif p.get("w8a8"):
            # per-row scale vectors, unpadded (ld 1)
            self.U, self.V = dev(p["U"]), dev(p["V"])
            self.Ud = qg.layout("f32", M, 1, ld=1)
            self.Vd = qg.layout("f32", N, 1, ld=1)
        elif p.get("U") is not None:
            self.Ud = qg.layout("f32", M, p["U"].shape[1], ld=self.ldu)
            self.Vd = qg.layout("f32", p["V"].shape[0], p["V"].shape[1], ld=self.ldv)

    def op(self, **kw):
        if self.p["kind"] == "w4a16":
            kw.setdefault("quant_b", (qg.QUANT_INT4_ZP, self.p["group"], 1, self.p["zero_point"]))
        if self.p.get("w8a8"):
            kw.setdefault("quant_a", (qg.QUANT_BLOCK_F32, 0, 1, 0))
            kw.setdefault("quant_b", (qg.QUANT_BLOCK_F32, 0, 1, 0))
        if self.p["in_dtype"] == "e4m3":
            kw.setdefault("quant_a", (qg.QUANT_BLOCK_F32, self.p["group_k"], 1, 0))
            kw.setdefault("quant_b", (qg.QUANT_BLOCK_F32, self.p["group_k"], self.p["group_n"], 0))
        return qg.operation(**kw)

    def launch(self, op=None, alpha=None, beta=None):
        p = self.p
        op = op or self.op()
        st = self.g.run_raw(op, p["alpha"] if alpha is None else alpha, self.A, self.Ad, self.U, self.Ud, self.B,
                            self.Bd, self.V, self.Vd, p["beta"] if beta is None else beta, self.C, self.Cd, self.D,
                            self.Dd, self.ws.desc if self.ws is not None else None)
        return st

    def launch_timed(self, op, stamps):
        """qg_run_timed with this problem's operands; stamps: device int64
        tensor of 8 * units entries. Returns (status, units)."""
        p = self.p
        return self.g.run_timed_raw(op, p["alpha"], self.A, self.Ad, self.U, self.Ud, self.B, self.Bd, self.V,
                                    self.Vd, p["beta"], self.C, self.Cd, self.D, self.Dd,
                                    self.ws.desc if self.ws is not None else None, stamps,
                                    stamps.numel() // 8 if stamps is not None else 0)

    def run(self, op=None, **kw):
        # poison the partials workspace: a split-K / stream-K fixup that read
        # a slot before (or without) it being written would pick up NaNs
        if self.ws is not None:
            self.ws.partials.fill_(float("nan"))
        st = self.launch(op, **kw)
        if st != qg.OK:
            raise qg.QGemmError(st, "qg_run")
        return self.run_result()

    def reset_output(self):
        """Refill D (valid columns and the pitch padding) with its sentinel."""
        self.D.fill_(-7 if self.out in ("i32", "i8") else float("nan"))

    def run_result(self):
        """D after the launch (synchronises), with the padding checked untouched."""
        torch.cuda.synchronize()
        D = host_f64(self.D)
        pad = D[:, self.p["N"]:]
        if self.out in ("i32", "i8"):
            assert (pad == -7).all(), "write past column N"
        else:
            assert np.isnan(pad).all(), "write past column N"
        return np.ascontiguousarray(D[:, :self.p["N"]])

    def plan(self, op=None):
        p = self.p
        return self.g.plan(op or self.op(), self.Ad, self.Ud, self.Bd, self.Vd, self.Cd, self.Dd, p["alpha"], p["beta"],
                           self.ws.desc if self.ws is not None else None)


def check_against_oracle(p, D, rows=None, what=""):
    """Float paths: the tolerance rule; int8 -> int32: exact."""
    import oracle
    from tests import tolerance
    ref, absdot = oracle.gemm(p, rows=rows)
    Dsel = D if rows is None else D[np.asarray(rows)]
    if p["out_dtype"] == "i32":
        assert np.array_equal(Dsel, ref), f"{what}: int32 result differs from the exact sum"
        return 0.0
    c = decode_c(p)
    if c is not None and rows is not None:
        c = c[np.asarray(rows)]
    return tolerance.check(Dsel, ref, absdot, p["alpha"], p["beta"], c, p["out_dtype"], what)


def sample_rows(M, n, seed=1234):
    g = np.random.default_rng(seed)
    rows = {0, M - 1} | set(g.integers(0, M, size=n).tolist())
    return sorted(rows)
