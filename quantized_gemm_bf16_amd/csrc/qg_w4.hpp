// Weight-only int4 GEMM core (W4A16) for gfx950: A bf16, B int4 packed 8 per
// uint32 (element k = 8w + i in bits [4i, 4i+4) of word w), fp16 scale per
// (column n, 128-deep group of k), zero point zp:
//     b(n, k) = (q(n, k) - zp) * s(n, k / 128)
// where zp is one constant, or (asymmetric) a zero point per column and group
// held as a byte in U: zp = U[n, k / 128]
// (the "U, V quantization scale operands" of the page "InternLM Lmdeploy Gemm
// Interface", I/O Contract, and the group tracking of the page "InternLM
// Lmdeploy Gemm MainloopSm80V2": the scale advances once per group along K).
//
// Dequantisation in registers, before the MFMA, without rounding the weight:
// a nibble q becomes the bf16 number 128 + q (bf16 0x4300 is 128 and its last
// mantissa bit weighs 1). Per group the MFMA chain computes
//     P = sum_k a_k (128 + q_k)      and      Z = sum_k a_k (128 + zp)
// with the same A fragments in the same order (Z from a B operand holding
// the constant 128 + zp), and the group adds s_n * (P - Z) to the fp32
// accumulator. Both products are exact; the only rounding is the fp32
// summation, and a column whose nibbles all equal the zero point in a group
// gives P == Z bit for bit, so it contributes exactly 0.
//
// Nibble order: a word w of 8 nibbles (k0 .. k0+7) and y = w >> 4 are merged
// by one byte permute per dword into [byte r of w, -, byte r of y, -], whose
// two low nibbles under the mask 0x000F000F are q(k0 + 2r) and q(k0 + 2r + 1):
// OR-ed with 0x43004300 they are the bf16 pair (128 + q(k0+2r), 128 +
// q(k0+2r+1)), i.e. B comes out in natural k order and the A fragments are
// used exactly as they sit in LDS.
//
// Tile: BM x BN outputs (BM = 16 MT). 8 waves as WN column groups x WK
// k-groups: wave (wn, wk) owns columns [wn BNW, (wn+1) BNW) and, of each
// k-tile of WK scale groups (128 WK deep), group wk. A k-tile's A rows (BM x
// 256 WK bytes), B rows (BN x 64 WK bytes of nibbles), the scales (one dword
// per column: WK = 2 fp16) and the zero points (one dword per column) go
// global -> LDS with direct loads into an S-stage ring. At the end of a unit
// the two k-group waves of a column group exchange halves through LDS and
// each keeps half of the group's n-tiles (deterministic: a + b == b + a).
#pragma once
#include <type_traits>

#include "qg_skinny.hpp"

namespace qg {

template <int MT_, int BN_, int WN_, int WK_, int STAGES_>
struct W4Cfg {
  static constexpr int MT = MT_, BM = 16 * MT_, BN = BN_, WN = WN_, WK = WK_, STAGES = STAGES_;
  static constexpr int NW = WN * WK, NT = NW * 64, BNW = BN / WN, TN = BNW / 16;
  static constexpr int GK = 128;                    // scale group
  static constexpr int BK = GK * WK;                // k per k-tile
  static constexpr int A_ROWB = BK * 2, B_ROWB = BK / 2;
  static constexpr int A_CPR = A_ROWB / 16, A_RPI = 64 / A_CPR;  // 16-byte chunks per row, rows per 64-lane load
  static constexpr int B_CPR = B_ROWB / 16, B_RPI = 64 / B_CPR;
  static constexpr int A_BYTES = BM * A_ROWB, B_BYTES = BN * B_ROWB;
  static constexpr int S_BYTES = BN * 4, Z_BYTES = BN * 4;  // one dword per column each
  static constexpr int STAGE = A_BYTES + B_BYTES + S_BYTES + Z_BYTES;
  static constexpr int DUMMY = STAGES * STAGE;              // 256 bytes the spare dword loads write
  static constexpr int ZX = DUMMY + 256;                    // Z exchange: [2][WK][4][16][MT] floats
  static constexpr int SMEM = ZX + 2 * WK * 4 * 16 * MT * 4;
  static constexpr int LA = BM / A_RPI / NW;  // 64-lane A loads per wave per k-tile
  static constexpr int LB = BN / B_RPI / NW;  // 64-lane B loads per wave per k-tile
  static constexpr int SW = BN / 64;          // waves loading scales (and as many loading zero points)
  static constexpr int LPW = LA + LB + 1;     // + one dword load (scales, zero points or a spare)
  static_assert(WK == 2, "a scale dword holds the k-tile's two fp16 scales");
  static_assert(A_RPI >= 1 && LA * A_RPI * NW == BM, "A rows must split over waves");
  static_assert(LB * B_RPI * NW == BN, "B rows must split over waves");
  static_assert(BN % 64 == 0 && 2 * SW <= NW, "scale and zero-point loaders");
  static_assert(TN >= 1 && BNW % 16 == 0, "columns per wave");
  static_assert(MT <= WN, "one wave per m-tile computes the shared Z chain");
  static_assert(STAGES >= 2 && SMEM <= 160 * 1024 - 8192, "LDS budget");
  static_assert(LPW * (STAGES - 2) < 64, "vmcnt range");
  static_assert(WN * TN * MT * 64 * 16 * (WK - 1) <= SMEM, "space for the k-group sum");
};

// (x & mask) | c with mask = 0x000F000F and a c whose bits under the mask are
// zero. Written as plain code, not inline assembly: the result feeds an MFMA
// operand, and the compiler inserts the wait states between a VALU write and
// an MFMA read of the same register only for instructions it can see (an
// inline-assembly VALU write followed closely by the MFMA read gave stale
// operands). The mask comes from opaque_sgpr and c from opaque_vgpr, so that
// the compiler keeps them in registers and emits one v_and_or_b32 per dword.
__device__ __forceinline__ uint32_t nib_bf16(uint32_t x, uint32_t mask, uint32_t c) { return (x & mask) | c; }

// Registers holding V that the compiler cannot constant-fold. Their only
// consumers are plain VALU instructions (no MFMA reads them directly), so
// writing them from inline assembly needs no wait states.
template <uint32_t V>
__device__ __forceinline__ uint32_t opaque_sgpr() {
  uint32_t r;
  asm("s_mov_b32 %0, %1" : "=s"(r) : "i"(V));
  return r;
}
template <uint32_t V>
__device__ __forceinline__ uint32_t opaque_vgpr() {
  uint32_t r;
  asm("v_mov_b32 %0, %1" : "=v"(r) : "i"(V));
  return r;
}

// XOR key of an A row's 16-byte chunks in LDS (512-byte rows): the low four
// row bits rotated left by one. The fragment reads take one chunk of 16
// consecutive rows per 16-lane group, the lane groups four chunks apart; with
// the plain key (row & 15) the LDS bank-conflict counter reads about one
// conflict cycle per conflict-free cycle for that pattern (a probe of this
// exact access), with the rotated key none.
__device__ __forceinline__ int akey(int row) { return ((row & 7) << 1) | ((row >> 3) & 1); }

template <class Cfg>
struct W4 {
  static constexpr int BM = Cfg::BM, BN = Cfg::BN, NT = Cfg::NT, TN = Cfg::TN, MT = Cfg::MT;
  static constexpr int WN = Cfg::WN, WK = Cfg::WK, BNW = Cfg::BNW;
  static constexpr int SMEM_BYTES = Cfg::SMEM;
  struct Acc {
    f32x4 v[TN][MT];
  };

  __device__ __forceinline__ static int wn_of(int w) { return w % WN; }
  __device__ __forceinline__ static int wk_of(int w) { return w / WN; }

  // The k-group of a wave is a compile-time constant in each of two copies
  // of the loop (a uniform branch picks one per wave): the half of a scale
  // dword that the group uses, the swizzled chunk offsets and the tile split
  // at the end then cost no instructions in the loop.
  __device__ __forceinline__ static void mainloop(const Args& a, const Unit& u, char* smem, Acc& acc) {
    if (wk_of(wave_id()) == 0)
      mainloop_k(std::integral_constant<int, 0>{}, a, u, smem, acc);
    else
      mainloop_k(std::integral_constant<int, 1>{}, a, u, smem, acc);
  }

  template <int WKC>
  __device__ __forceinline__ static void mainloop_k(std::integral_constant<int, WKC>, const Args& a, const Unit& u,
                                                    char* smem, Acc& acc) {
    const int w = wave_id(), l = lane_id();
    const int wn = wn_of(w);
    constexpr int wk = WKC;
    const int64_t lda_b = a.lda * 2, ldb_b = a.ldb * 4, ldv_b = a.ldv * 2;
    const uint32_t abytes = (uint32_t)a.K * 2, bbytes = (uint32_t)a.K / 2;  // valid bytes of an A / B row
    const int groups = a.K / Cfg::GK;
    const int a_rows = max(0, min(BM, u.m_end - u.m0));
    const int b_rows = max(0, min(BN, a.N - u.n0));
    const i32x4 rA = make_rsrc_words((const char*)a.A + (int64_t)u.m0 * lda_b, (uint32_t)(a_rows * lda_b));
    const i32x4 rB = make_rsrc_words((const char*)a.B + (int64_t)u.n0 * ldb_b, (uint32_t)(b_rows * ldb_b));
    // per-group zero points (bytes, U[n, group]); without them the loads read nothing
    const bool has_z = a.U != nullptr;
    const int64_t ldz_b = a.ldu;
    // waves [0, SW) load scales, [SW, 2 SW) zero points, the rest a spare dword
    const int role = w < Cfg::SW ? 0 : (w < 2 * Cfg::SW ? 1 : 2);
    const int dcol = (role == 1 ? w - Cfg::SW : w) * 64 + l;  // column of this lane's dword
    const i32x4 rD = role == 0 ? make_rsrc_words((const char*)a.V + (int64_t)u.n0 * ldv_b, (uint32_t)(b_rows * ldv_b))
                               : make_rsrc_words(has_z ? (const char*)a.U + (int64_t)u.n0 * ldz_b : (const char*)a.V,
                                                 role == 1 && has_z ? (uint32_t)(b_rows * ldz_b) : 0u);

    // load addressing (lane -> LDS position fixed; the lane fetches the
    // logical chunk the swizzle stores there)
    uint32_t offA[Cfg::LA], chA[Cfg::LA], offB[Cfg::LB], chB[Cfg::LB];
#pragma unroll
    for (int i = 0; i < Cfg::LA; ++i) {
      const int row = (w * Cfg::LA + i) * Cfg::A_RPI + l / Cfg::A_CPR;
      chA[i] = (uint32_t)(((l % Cfg::A_CPR) ^ akey(row)) * 16);
      offA[i] = (uint32_t)(row * lda_b) + chA[i];
    }
#pragma unroll
    for (int i = 0; i < Cfg::LB; ++i) {
      const int row = (w * Cfg::LB + i) * Cfg::B_RPI + l / Cfg::B_CPR;
      chB[i] = (uint32_t)(((l % Cfg::B_CPR) ^ ((row >> 1) & 7)) * 16);
      offB[i] = (uint32_t)(row * ldb_b) + chB[i];
    }
    char* dptr = role == 0 ? smem + Cfg::A_BYTES + Cfg::B_BYTES + w * 256
                           : (role == 1 ? smem + Cfg::A_BYTES + Cfg::B_BYTES + Cfg::S_BYTES + (w - Cfg::SW) * 256
                                        : smem + Cfg::DUMMY);
    const uint32_t dstride = role == 2 ? 0u : (uint32_t)Cfg::STAGE;

    auto issue = [&](int stage, int kt) {
      char* sb = smem + stage * Cfg::STAGE;
      const bool live = kt < u.ke;
      const uint32_t ka = (uint32_t)kt * Cfg::A_ROWB, kb = (uint32_t)kt * Cfg::B_ROWB;
      if (live && ka + Cfg::A_ROWB <= abytes) {
        // the whole k-tile lies inside K (the usual case): no per-lane range selects
#pragma unroll
        for (int i = 0; i < Cfg::LA; ++i) load_lds_x4(rA, sb + (w * Cfg::LA + i) * 1024, offA[i] + ka);
#pragma unroll
        for (int i = 0; i < Cfg::LB; ++i) load_lds_x4(rB, sb + Cfg::A_BYTES + (w * Cfg::LB + i) * 1024, offB[i] + kb);
      } else {
#pragma unroll
        for (int i = 0; i < Cfg::LA; ++i)
          load_lds_x4(rA, sb + (w * Cfg::LA + i) * 1024, live && ka + chA[i] < abytes ? offA[i] + ka : kOOB);
#pragma unroll
        for (int i = 0; i < Cfg::LB; ++i)
          load_lds_x4(rB, sb + Cfg::A_BYTES + (w * Cfg::LB + i) * 1024,
                      live && kb + chB[i] < bbytes ? offB[i] + kb : kOOB);
      }
      // scales: the dword holding s(n, 2 kt) and s(n, 2 kt + 1); zero points:
      // the dword holding z(n, 2 kt) (ldu is a multiple of 16)
      const uint32_t doff = role == 0 ? (uint32_t)(dcol * ldv_b) + (uint32_t)kt * 4
                                      : (uint32_t)(dcol * ldz_b) + ((uint32_t)(2 * kt) & ~3u);
      load_lds_x1a(rD, dptr + stage * dstride, live && role < 2 ? doff : kOOB);
    };

    const int orow = l & 15, og = l >> 4;
    // Per-lane LDS offsets of the fragments inside a ring stage, fixed for
    // the whole loop. The swizzle keys depend on the low row bits only, so
    // the m-tile (A) and n-tile (B, scales) parts are whole multiples of 16
    // rows and enter the reads as immediate offsets. A step adds the stage
    // base to each of these once (rebase) and reads at immediate offsets
    // from the result.
    uint32_t lA[4];  // A rows orow of m-tile 0, k chunk 16 wk + 4 og + j
#pragma unroll
    for (int j = 0; j < 4; ++j) lA[j] = (uint32_t)(orow * Cfg::A_ROWB + (((wk * 16 + 4 * og + j) ^ akey(orow)) << 4));
    const uint32_t lZm = (uint32_t)((wn % MT) * 16 * Cfg::A_ROWB);  // m-tile of this wave's Z chain
    const uint32_t lB = (uint32_t)(Cfg::A_BYTES + (wn * BNW + orow) * Cfg::B_ROWB +
                                     (((wk * 4 + og) ^ ((orow >> 1) & 7)) << 4));
    const uint32_t lS = (uint32_t)(Cfg::A_BYTES + Cfg::B_BYTES + (wn * BNW + 4 * og) * 4);
    const uint32_t lZ = (uint32_t)(Cfg::A_BYTES + Cfg::B_BYTES + Cfg::S_BYTES + (wn * BNW + orow) * 4);
    static_assert(BNW % 16 == 0, "n-tiles keep the B swizzle key");
    // stage base + per-lane offset as a value the compiler cannot split
    // again: without this it keeps one register per (m-tile, k-step) address
    // and adds the stage to each of them before every read
    auto rebase = [](uint32_t stage_base, uint32_t off) {
      uint32_t x = stage_base + off;
      asm volatile("" : "+v"(x));
      return x;
    };
    const uint32_t c128 = opaque_vgpr<0x43004300u>(), m4 = opaque_sgpr<0x000F000Fu>();
    // byte permutes: dword r = [byte r of w, 0, byte r of (w >> 4), 0]
    constexpr uint32_t kSel0 = 0x0C040C00u, kSel1 = 0x0C050C01u, kSel2 = 0x0C060C02u, kSel3 = 0x0C070C03u;
    // B operand of the Z chain (symmetric): 128 + zp in every bf16 half
    const uint32_t zsym = c128 | ((uint32_t)a.zero_point * 0x00010001u);
    // Symmetric Z exchange: Z depends on the row only, so for each group the
    // wave with wn = mt computes the chain of m-tile mt and leaves the 16 row
    // values in zx[group parity][wk][lane group][row][mt]; every wave applies
    // the group's correction one k-tile later, after the barrier that makes
    // them visible.
    float* zx = (float*)(smem + Cfg::ZX);
    auto zslot = [](int kt, int wk_, int og_) { return (((kt & 1) * WK + wk_) * 4 + og_) * 16 * MT; };

#pragma unroll
    for (int tn = 0; tn < TN; ++tn)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc.v[tn][mt] = f32x4{};

    // The scale of a group: half wk of the dword holding the k-tile's two
    // fp16 scales (a conversion the FMAs that use it absorb).
    auto scale = [](uint32_t d) { return f16_bits_to_f32((uint16_t)(wk ? d >> 16 : d)); };
    // With K / 128 odd, the second group of the last k-tile lies past K: its
    // P and Z are 0 and its scale slot holds padding (possibly Inf or NaN), so
    // the lane that loaded the slot writes 0 there once its load has landed,
    // before the barrier that hands the stage to the other waves.
    const int ztail = role == 0 && (groups & 1) ? groups / 2 : -1;
    auto scale_tail = [&](int st, int kt) {
      if (kt == ztail) *(uint16_t*)(dptr + st * dstride + 4 * l + 2) = 0;
    };

    // P (and, with zero points, Z) of group 2 kt + wk of the k-tile in ring
    // stage st, plus the scale dwords of the lane's columns.
    auto group = [&](int st, int kt, auto with_z, f32x4 (&P)[TN][MT], uint32_t (&sc)[TN][4], auto&& hook) {
      constexpr bool ZP = decltype(with_z)::value;
      const uint32_t sbase = (uint32_t)(st * Cfg::STAGE);
      const int g = 2 * kt + wk;
      // B words of this lane: row orow of each n-tile, the group's 16-byte
      // chunk og (4 words, one per k-step)
      i32x4 bw[TN];
      const uint32_t bB = rebase(sbase, lB);
#pragma unroll
      for (int tn = 0; tn < TN; ++tn) bw[tn] = *(const i32x4*)(smem + bB + tn * 16 * Cfg::B_ROWB);
      // scale dwords of the lane's output columns n = 4 og + r
      const uint32_t bS = rebase(sbase, lS);
#pragma unroll
      for (int tn = 0; tn < TN; ++tn) {
        const i32x4 sd = *(const i32x4*)(smem + bS + tn * 16 * 4);
#pragma unroll
        for (int r = 0; r < 4; ++r) sc[tn][r] = (uint32_t)sd[r];
      }
      // asymmetric: the zero point of the lane's B row (the MFMA's first
      // operand row, i.e. column n)
      uint32_t zb[TN];
      if constexpr (ZP) {
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) {
          const uint32_t zd = *(const uint32_t*)(smem + rebase(sbase, lZ) + tn * 16 * 4);
          zb[tn] = c128 | (((zd >> (8 * (g & 3))) & 0xFu) * 0x00010001u);
        }
      }
      f32x4 Z[ZP ? TN : 1][MT];
      f32x4 Zc = {};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        // A fragments: k chunk 16 wk + 4 og + j of rows orow of each m-tile
        i32x4 af[MT];
        const uint32_t bA = rebase(sbase, lA[j]);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) af[mt] = *(const i32x4*)(smem + bA + mt * 16 * Cfg::A_ROWB);
        if constexpr (ZP) {
#pragma unroll
          for (int tn = 0; tn < TN; ++tn) {
            const i32x4 bz = {(int)zb[tn], (int)zb[tn], (int)zb[tn], (int)zb[tn]};
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) Z[tn][mt] = mfma16_bf16(bz, af[mt], j == 0 ? f32x4{} : Z[tn][mt]);
          }
        } else {
          // the same LDS bytes as af[wn % MT] (only known at run time); every
          // wave runs the chain so that the loop body has no branch, and the
          // waves with wn < MT publish it
          const i32x4 bz = {(int)zsym, (int)zsym, (int)zsym, (int)zsym};
          const i32x4 am = *(const i32x4*)(smem + bA + lZm);
          Zc = mfma16_bf16(bz, am, Zc);
        }
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) {
          const uint32_t q = (uint32_t)bw[tn][j], y = q >> 4;
          const i32x4 bq = {(int)nib_bf16(__builtin_amdgcn_perm(y, q, kSel0), m4, c128),
                            (int)nib_bf16(__builtin_amdgcn_perm(y, q, kSel1), m4, c128),
                            (int)nib_bf16(__builtin_amdgcn_perm(y, q, kSel2), m4, c128),
                            (int)nib_bf16(__builtin_amdgcn_perm(y, q, kSel3), m4, c128)};
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) P[tn][mt] = mfma16_bf16(bq, af[mt], j == 0 ? f32x4{} : P[tn][mt]);
        }
        // VALU work handed in by the caller, placed between the k-steps so
        // that it runs while this step's MFMAs do
        hook(j);
      }
      if constexpr (ZP) {
        // zero points per column: the correction right away
#pragma unroll
        for (int tn = 0; tn < TN; ++tn)
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              acc.v[tn][mt][r] = __builtin_fmaf(scale(sc[tn][r]), P[tn][mt][r] - Z[tn][mt][r], acc.v[tn][mt][r]);
      } else {
        // lane (og, orow) holds Z of row orow (every output column of the
        // chain carries the same value); each lane writes its own copy, so
        // no lane is masked off (a branch would split the scheduling region)
        zx[zslot(kt, wk, og) + orow * MT + wn % MT] = Zc[0];
      }
    };
    // symmetric: acc += s_n * (P - Z) for the group computed in the previous
    // k-tile (Z from the exchange)
    auto zread = [&](int kt, float (&zv)[MT]) {
      const float* zr = zx + zslot(kt, wk, og) + orow * MT;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) zv[mt] = zr[mt];
    };
    auto correct_mt = [&](int mt, const f32x4 (&P)[TN][MT], const uint32_t (&sc)[TN][4], const float (&zv)[MT]) {
#pragma unroll
      for (int tn = 0; tn < TN; ++tn)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          acc.v[tn][mt][r] = __builtin_fmaf(scale(sc[tn][r]), P[tn][mt][r] - zv[mt], acc.v[tn][mt][r]);
    };
    auto correct = [&](const f32x4 (&P)[TN][MT], const uint32_t (&sc)[TN][4], const float (&zv)[MT]) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) correct_mt(mt, P, sc, zv);
    };
    auto no_hook = [](int) {};

    const int nk = u.ke - u.kb;
    constexpr int S = Cfg::STAGES;
#pragma unroll
    for (int st = 0; st < S - 1; ++st) issue(st, u.kb + st);
    f32x4 P[TN][MT];
    uint32_t sc[TN][4];
    if (has_z) {
      for (int it = 0; it < nk; ++it) {
        wait_vmcnt<Cfg::LPW * (S - 2)>();
        scale_tail(it % S, u.kb + it);
        lds_barrier();
        issue((it + S - 1) % S, u.kb + it + S - 1);
        group(it % S, u.kb + it, std::true_type{}, P, sc, no_hook);
      }
    } else {
      // the first iteration corrects a "previous group" of zeros: P = 0, s = 0
      // and its Z slot zeroed (so that no stale LDS value turns 0 * x into NaN)
#pragma unroll
      for (int tn = 0; tn < TN; ++tn) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) P[tn][mt] = f32x4{};
#pragma unroll
        for (int r = 0; r < 4; ++r) sc[tn][r] = 0u;
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) zx[zslot(u.kb - 1, wk, og) + orow * MT + mt] = 0.f;
      // one k-tile: correct the previous group (Pq, sq) while computing this
      // one into (Pc, sc_); the loop below alternates two register sets
      // instead of copying them
      auto step = [&](int it, f32x4 (&Pc)[TN][MT], uint32_t (&scc)[TN][4], const f32x4 (&Pq)[TN][MT],
                      const uint32_t (&sq)[TN][4]) {
        wait_vmcnt<Cfg::LPW * (S - 2)>();
        scale_tail(it % S, u.kb + it);
        lds_barrier();
        // the previous group's Z values, read before this group writes the
        // other half of the exchange (the compiler cannot tell them apart)
        float zv[MT];
        zread(u.kb + it - 1, zv);
        issue((it + S - 1) % S, u.kb + it + S - 1);
        // the previous group's correction (VALU) and this group's chains
        // (MFMA) are independent: they are interleaved k-step by k-step so
        // that both units stay busy; k-step j corrects m-tiles j, j + 4, ...
        group(it % S, u.kb + it, std::false_type{}, Pc, scc, [&](int j) {
#pragma unroll
          for (int mt = j; mt < MT; mt += 4) correct_mt(mt, Pq, sq, zv);
        });
      };
      f32x4 P2[TN][MT];
      uint32_t sc2[TN][4];
      int it = 0;
      for (; it + 1 < nk; it += 2) {
        step(it, P2, sc2, P, sc);
        step(it + 1, P, sc, P2, sc2);
      }
      if (it < nk) {
        step(it, P2, sc2, P, sc);
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) {
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) P[tn][mt] = P2[tn][mt];
#pragma unroll
          for (int r = 0; r < 4; ++r) sc[tn][r] = sc2[tn][r];
        }
      }
    }
    wait_vmcnt<0>();
    __syncthreads();  // every wave is done with the ring before it is reused below
    if (!has_z && nk > 0) {
      float zv[MT];
      zread(u.ke - 1, zv);
      correct(P, sc, zv);
    }

    // Sum the two k-group waves of a column group, splitting the tile: wave
    // (wn, wk) keeps n-tiles [wk TO, (wk + 1) TO) and hands the other half to
    // its partner through LDS (a + b == b + a exactly, so the result does
    // not depend on which wave adds). Both waves then write, read back and
    // store half of the column group's outputs.
    f32x4* red = (f32x4*)smem;
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) {
      if (tn / TO == wk) continue;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) red[((wn * TN + tn) * MT + mt) * 64 + l] = acc.v[tn][mt];
    }
    __syncthreads();
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) {
      if (tn / TO != wk) continue;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc.v[tn][mt] += red[((wn * TN + tn) * MT + mt) * 64 + l];
    }
    __syncthreads();  // the ring is reused by the next unit
  }

  // Lane holds D[m][n .. n+3] with m = 16 mt + l%16, n = n0 + wn*BNW + 16 tn + 4 (l/16),
  // for the n-tiles tn its k-group wave keeps (see the end of mainloop).
  static constexpr int TO = TN / WK;  // n-tiles kept per wave
  static_assert(TO * WK == TN, "the finished tile splits over the k-group waves by n-tiles");
  // Whether n-tile tn is kept by the calling wave. Register arrays are only
  // ever indexed with compile-time indices (loops over every tn with this
  // uniform test): a wave-dependent index would send them to scratch.
  __device__ __forceinline__ static bool keeps(int tn) { return tn / TO == wk_of(wave_id()); }
  // A whole tile with a plain 16-bit D (no C term, no fused epilogue) goes
  // out through LDS: the waves round their kept n-tiles into a BM x BN tile
  // (rows padded by 16 bytes, so that the 16 rows of a lane group's 8-byte
  // writes fall in different banks), then every thread writes whole 16-byte
  // pieces of 2*BN-byte rows, instead of 8-byte pieces of 16 rows per store.
  static constexpr int SROW = BN * 2 + 16;
  static_assert(BM * SROW <= Cfg::SMEM, "staging tile");
  __device__ __forceinline__ static void store_staged(const Args& a, const Unit& u, Acc& acc, char* smem) {
    const int w = wave_id(), l = lane_id();
    const int wn = wn_of(w);
    const bool bf = a.d_type == DT_BF16;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int row = mt * 16 + (l & 15);
#pragma unroll
      for (int tn = 0; tn < TN; ++tn) {
        if (!keeps(tn)) continue;
        const int col = wn * BNW + tn * 16 + 4 * (l >> 4);
        uint16_t h[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float x = a.alpha * acc.v[tn][mt][j];
          h[j] = bf ? f32_to_bf16_bits(x) : f32_to_f16_bits(x);
        }
        *(u16x4*)(smem + row * SROW + col * 2) = u16x4{h[0], h[1], h[2], h[3]};
      }
    }
    __syncthreads();
    constexpr int CPR = BN * 2 / 16;  // 16-byte pieces per row
    for (int idx = (int)threadIdx.x; idx < BM * CPR; idx += NT) {
      const int row = idx / CPR, ch = idx % CPR;
      const i32x4 v = *(const i32x4*)(smem + row * SROW + ch * 16);
      uint16_t* p = (uint16_t*)a.D + (int64_t)(u.m0 + row) * a.ldd + u.n0 + ch * 8;
      __builtin_nontemporal_store(v, (i32x4*)p);
    }
    __syncthreads();  // the staging area is the next unit's ring
  }

  __device__ __forceinline__ static void store(const Args& a, const Unit& u, Acc& acc, char* smem) {
    const bool plain16 = (a.d_type == DT_BF16 || a.d_type == DT_F16) && (a.c_type < 0 || a.beta == 0.f) && a.epi == 0;
    if (plain16 && u.m0 + BM <= u.m_end && u.n0 + BN <= a.N) {
      store_staged(a, u, acc, smem);
      return;
    }
    const int w = wave_id(), l = lane_id();
    const int wn = wn_of(w);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int m = u.m0 + mt * 16 + (l & 15);
      if (m >= u.m_end) continue;
#pragma unroll
      for (int tn = 0; tn < TN; ++tn) {
        if (!keeps(tn)) continue;
        const int n = u.n0 + wn * BNW + tn * 16 + 4 * (l >> 4);
        if (n < a.N) epi_store4(a, m, n, acc.v[tn][mt]);
      }
    }
  }

  __device__ __forceinline__ static __amdgpu_buffer_rsrc_t slot_rsrc(const Args& a, int slot) {
    return make_rsrc((const char*)a.partials + (size_t)slot * (BM * BN * 4), BM * BN * 4);
  }
  // Partial tile layout: [wn][tn][mt][lane] x 16 bytes (each (wn, tn) written by the wave that keeps it).
  __device__ __forceinline__ static uint32_t pofs(int tn, int mt) {
    return (uint32_t)((((wn_of(wave_id()) * TN + tn) * MT + mt) * 64 + lane_id()) * 16);
  }
  __device__ __forceinline__ static void write_partial(const Args& a, int slot, Acc& acc) {
    const auto r = slot_rsrc(a, slot);
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) {
      if (!keeps(tn)) continue;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) store_sc1_x4(r, pofs(tn, mt), __builtin_bit_cast(i32x4, acc.v[tn][mt]));
    }
  }
  // Chunk c = i * MT + mt of a lane's partial tile: the wave's i-th kept
  // n-tile (wk TO + i), m-tile mt.
  using S4 = f32x4;
  static constexpr int NCH = TO * MT;
  __device__ __forceinline__ static bool holds_partial() { return true; }
  __device__ __forceinline__ static uint32_t chunk_off(int c) {
    return pofs(wk_of(wave_id()) * TO + c / MT, c % MT);
  }
  __device__ __forceinline__ static S4 get4(const Acc& acc, int c) {
    S4 x = acc.v[c / MT][c % MT];
#pragma unroll
    for (int tn = TO; tn < TN; ++tn)
      if (tn / TO == wk_of(wave_id()) && tn % TO == c / MT) x = acc.v[tn][c % MT];
    return x;
  }
  __device__ __forceinline__ static void set4(Acc& acc, int c, const S4& x) {
#pragma unroll
    for (int tn = 0; tn < TN; ++tn)
      if (tn / TO == wk_of(wave_id()) && tn % TO == c / MT) acc.v[tn][c % MT] = x;
  }
};

template <class Cfg>
hipError_t launch_w4(const Args& a, int grid, hipStream_t s) {
  return launch_sched<W4<Cfg>>(a, grid, s);
}

}  // namespace qg
