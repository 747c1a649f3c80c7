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
// a nibble q becomes the bf16 number 128 + q with one bitfield insert (bf16 0x4300 is
// 128 and its last mantissa bit weighs 1), two nibbles per dword. Per group
// the MFMA computes P = sum_k a_k (128 + q_k); a second MFMA against a column
// of ones gives R = sum_k a_k; the group then adds
//     s_n * (P - (128 + zp) * R)
// to the fp32 accumulator. Both MFMA products are exact and accumulate in
// fp32, so the only rounding is fp32 summation.
//
// Tile: BM x BN outputs, one 128-deep k group per k-tile. A k-tile (BM rows x
// 256 bytes), the B k-tile (BN rows x 64 bytes of nibbles) and the k-tile's
// scales (BN dwords) go global -> LDS with direct loads into an S-stage ring
// shared by the NW waves (wave w owns columns [w*BN/NW, (w+1)*BN/NW)). The
// 128 k of a group map to MFMA k-slots as: step j, lane group g (lanes
// 16g..16g+15) takes k 32g + 8j + {0,4,1,5,2,6,3,7}; A fragments are
// byte-permuted into that order (v_perm), B comes out of the bitfield insert in it.
#pragma once
#include <type_traits>

#include "qg_skinny.hpp"

namespace qg {

template <int BM_, int BN_, int NW_, int STAGES_>
struct W4Cfg {
  static constexpr int BM = BM_, BN = BN_, NW = NW_, STAGES = STAGES_;
  static constexpr int NT = NW * 64, MT = BM / 16, BNW = BN / NW, TN = BNW / 16;
  static constexpr int BK = 128;                  // k per k-tile (= one scale group)
  static constexpr int A_ROWB = 256, B_ROWB = 64;  // bytes per row per k-tile
  // scales: every lane of a dword load writes LDS, so each wave gets 64 dword
  // slots; lanes past its BN/NW columns load nothing (zeros).
  static constexpr int A_BYTES = BM * A_ROWB, B_BYTES = BN * B_ROWB, S_BYTES = NW * 64 * 4;
  static constexpr int Z_BYTES = NW * 64 * 4;  // per-group zero points (a dword per lane)
  static constexpr int STAGE = A_BYTES + B_BYTES + S_BYTES + Z_BYTES;
  static constexpr int LA = BM / 4 / NW;   // 64-lane A loads per wave (4 rows x 256 B each)
  static constexpr int LB = BN / 16 / NW;  // 64-lane B loads per wave (16 rows x 64 B each)
  static constexpr int LPW = LA + LB + 2;  // + one scale load and one zero-point load (dword each)
  static_assert(LA * 4 * NW == BM && LB * 16 * NW == BN, "rows must split over waves");
  static_assert(BNW % 16 == 0 && BNW <= 64, "columns per wave");
  static_assert(STAGES >= 2 && STAGES * STAGE <= 160 * 1024 - 4096, "LDS budget");
  static_assert(LPW * (STAGES - 2) < 64, "vmcnt range");
};

// (x & mask) | c with mask = 0x000F000F and a c whose bits under the mask are
// zero: the two nibbles at bits 0 and 16 of x become the low mantissa bits of
// two bf16 halves. Written as plain code, not inline assembly: the result
// feeds an MFMA operand, and the compiler inserts the wait states between a
// VALU write and an MFMA read of the same register only for instructions it
// can see (an inline-assembly VALU write followed closely by the MFMA read
// gave stale operands). The mask comes from opaque_sgpr and c from
// opaque_vgpr, so that the compiler keeps them in registers and emits one
// v_and_or_b32 per dword (with both known it folds them into an and and an
// or with literal operands; with both in scalar registers gfx9's one scalar
// operand per instruction splits it the same way).
__device__ __forceinline__ uint32_t nib_bf16(uint32_t x, uint32_t mask, uint32_t c) { return (x & mask) | c; }

// Registers holding V that the compiler cannot constant-fold. Their only
// consumers are plain VALU instructions (no MFMA reads them), so writing
// them from inline assembly needs no wait states.
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

template <class Cfg>
struct W4 {
  static constexpr int BM = Cfg::BM, BN = Cfg::BN, NT = Cfg::NT, TN = Cfg::TN, MT = Cfg::MT;
  static constexpr int SMEM_BYTES = Cfg::STAGES * Cfg::STAGE;
  struct Acc {
    f32x4 v[TN][MT];
  };

  __device__ __forceinline__ static void mainloop(const Args& a, const Unit& u, char* smem, Acc& acc) {
    const int w = wave_id(), l = lane_id();
    const int64_t lda_b = a.lda * 2, ldb_b = a.ldb * 4, ldv_b = a.ldv * 2;
    const uint32_t kbytes_a = (uint32_t)a.K * 2;  // valid bytes of an A row
    const int a_rows = max(0, min(BM, u.m_end - u.m0));
    const int b_rows = max(0, min(BN, a.N - u.n0));
    const i32x4 rA = make_rsrc_words((const char*)a.A + (int64_t)u.m0 * lda_b, (uint32_t)(a_rows * lda_b));
    const i32x4 rB = make_rsrc_words((const char*)a.B + (int64_t)u.n0 * ldb_b, (uint32_t)(b_rows * ldb_b));
    const i32x4 rV = make_rsrc_words((const char*)a.V + (int64_t)u.n0 * ldv_b, (uint32_t)(b_rows * ldv_b));
    // per-group zero points (bytes, U[n, group]); without them the loads read nothing
    const bool has_z = a.U != nullptr;
    const int64_t ldz_b = a.ldu;
    const i32x4 rZ = make_rsrc_words(has_z ? (const char*)a.U + (int64_t)u.n0 * ldz_b : (const char*)a.V,
                                     has_z ? (uint32_t)(b_rows * ldz_b) : 0u);

    // load addressing (lane -> LDS position fixed; the lane fetches the
    // logical chunk the swizzle stores there)
    uint32_t offA[Cfg::LA], chA[Cfg::LA], offB[Cfg::LB], chB[Cfg::LB];
#pragma unroll
    for (int i = 0; i < Cfg::LA; ++i) {
      const int row = (w * Cfg::LA + i) * 4 + (l >> 4);
      chA[i] = (uint32_t)(((l & 15) ^ (row & 15)) * 16);
      offA[i] = (uint32_t)(row * lda_b) + chA[i];
    }
#pragma unroll
    for (int i = 0; i < Cfg::LB; ++i) {
      const int row = (w * Cfg::LB + i) * 16 + (l >> 2);
      chB[i] = (uint32_t)(((l & 3) ^ ((row >> 2) & 3)) * 16);
      offB[i] = (uint32_t)(row * ldb_b) + chB[i];
    }
    // scales: wave w loads the dwords holding s(n, group) for its BN/NW rows
    const int srow = w * Cfg::BNW + l;
    const bool s_lane = l < Cfg::BNW;

    auto issue = [&](int stage, int kt) {
      char* sb = smem + stage * Cfg::STAGE;
      const bool live = kt < u.ke;
      const uint32_t ka = (uint32_t)kt * Cfg::A_ROWB, kb = (uint32_t)kt * Cfg::B_ROWB;
#pragma unroll
      for (int i = 0; i < Cfg::LA; ++i)
        load_lds_x4(rA, sb + (w * Cfg::LA + i) * 1024, live && ka + chA[i] < kbytes_a ? offA[i] + ka : kOOB);
#pragma unroll
      for (int i = 0; i < Cfg::LB; ++i)
        load_lds_x4(rB, sb + Cfg::A_BYTES + (w * Cfg::LB + i) * 1024, live ? offB[i] + kb : kOOB);
      // dword (aligned) that holds s(n0 + srow, kt); ldv is even, so the half is kt & 1
      const uint32_t soff = (uint32_t)(srow * ldv_b) + ((uint32_t)kt * 2 & ~3u);
      load_lds_x1a(rV, sb + Cfg::A_BYTES + Cfg::B_BYTES + w * 256, live && s_lane ? soff : kOOB);
      // dword (aligned) that holds z(n0 + srow, kt): byte kt & 3 of it (ldu is a multiple of 4)
      const uint32_t zo = (uint32_t)(srow * ldz_b) + ((uint32_t)kt & ~3u);
      load_lds_x1a(rZ, sb + Cfg::A_BYTES + Cfg::B_BYTES + Cfg::S_BYTES + w * 256, live && s_lane && has_z ? zo : kOOB);
    };

    const int orow = l & 15, og = l >> 4;
    // bf16 128.0 in both halves, and the nibble mask
    const uint32_t c128 = opaque_vgpr<0x43004300u>(), m4 = opaque_sgpr<0x000F000Fu>();
    const i32x4 ones = {0x3F803F80, 0x3F803F80, 0x3F803F80, 0x3F803F80};  // bf16 1.0 pairs
    const float zoff = 128.0f + (float)a.zero_point;

#pragma unroll
    for (int tn = 0; tn < TN; ++tn)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc.v[tn][mt] = f32x4{};

    // One k-tile (one scale group) from ring stage st.
    auto group = [&](int st, int kt) {
      const char* sA = smem + st * Cfg::STAGE;
      const char* sB = sA + Cfg::A_BYTES;
      const uint32_t* sS = (const uint32_t*)(sB + Cfg::B_BYTES);
      // B words of this lane: row orow of each n-tile, 16-byte chunk og (4 words, one per step)
      i32x4 bw[TN];
#pragma unroll
      for (int tn = 0; tn < TN; ++tn) {
        const int row = w * Cfg::BNW + tn * 16 + orow;
        bw[tn] = *(const i32x4*)(sB + row * Cfg::B_ROWB + ((og ^ ((row >> 2) & 3)) << 4));
      }
      f32x4 P[TN][MT], R[MT];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        // A fragments: k chunk 4g + j of rows orow of each m-tile, permuted to
        // the element order {0,4,1,5,2,6,3,7} the B dequant produces
        i32x4 af[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const int row = mt * 16 + orow;
          const int c = 4 * og + j;
          const i32x4 d = *(const i32x4*)(sA + row * Cfg::A_ROWB + ((c ^ (row & 15)) << 4));
          af[mt] = i32x4{(int)__builtin_amdgcn_perm((uint32_t)d[2], (uint32_t)d[0], 0x05040100u),
                         (int)__builtin_amdgcn_perm((uint32_t)d[2], (uint32_t)d[0], 0x07060302u),
                         (int)__builtin_amdgcn_perm((uint32_t)d[3], (uint32_t)d[1], 0x05040100u),
                         (int)__builtin_amdgcn_perm((uint32_t)d[3], (uint32_t)d[1], 0x07060302u)};
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) R[mt] = mfma16_bf16(ones, af[mt], j == 0 ? f32x4{} : R[mt]);
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) {
          const uint32_t q = (uint32_t)bw[tn][j];
          // bf16 pairs (128 + q_i, 128 + q_{i+4}) for i = 0..3: one bitfield
          // insert per dword
          const i32x4 bq = {(int)nib_bf16(q, m4, c128), (int)nib_bf16(q >> 4, m4, c128),
                            (int)nib_bf16(q >> 8, m4, c128), (int)nib_bf16(q >> 12, m4, c128)};
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) P[tn][mt] = mfma16_bf16(bq, af[mt], j == 0 ? f32x4{} : P[tn][mt]);
        }
      }
      // acc += s_n * (P - (128 + zp) * R); lane holds columns n = 4*og + r of each n-tile
      const int half = kt & 1;
      const uint32_t* sZ = (const uint32_t*)((const char*)sS + Cfg::S_BYTES);
      auto correct = [&](auto with_z) {
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) {
          float s[4], zo[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const uint32_t dw = sS[w * 64 + tn * 16 + 4 * og + r];
            s[r] = f16_bits_to_f32((uint16_t)(half ? dw >> 16 : dw & 0xFFFF));
            if constexpr (decltype(with_z)::value)
              zo[r] = 128.0f + (float)((sZ[w * 64 + tn * 16 + 4 * og + r] >> (8 * (kt & 3))) & 0xFFu);
            else
              zo[r] = zoff;
          }
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              acc.v[tn][mt][r] = __builtin_fmaf(s[r], __builtin_fmaf(-zo[r], R[mt][r], P[tn][mt][r]), acc.v[tn][mt][r]);
        }
      };
      // uniform branch: the symmetric case reads no zero points
      if (has_z)
        correct(std::true_type{});
      else
        correct(std::false_type{});
    };

    const int nk = u.ke - u.kb;
    constexpr int S = Cfg::STAGES;
#pragma unroll
    for (int st = 0; st < S - 1; ++st) issue(st, u.kb + st);
    for (int it = 0; it < nk; ++it) {
      wait_vmcnt<Cfg::LPW * (S - 2)>();
      lds_barrier();
      issue((it + S - 1) % S, u.kb + it + S - 1);
      group(it % S, u.kb + it);
    }
    wait_vmcnt<0>();
    __syncthreads();
  }

  // Lane holds D[m][n .. n+3] with m = 16 mt + l%16, n = n0 + w*BNW + 16 tn + 4 (l/16).
  __device__ __forceinline__ static void store(const Args& a, const Unit& u, Acc& acc, char* /*smem*/) {
    const int w = wave_id(), l = lane_id();
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int m = u.m0 + mt * 16 + (l & 15);
      if (m >= u.m_end) continue;
#pragma unroll
      for (int tn = 0; tn < TN; ++tn) {
        const int n = u.n0 + w * Cfg::BNW + tn * 16 + 4 * (l >> 4);
        if (n < a.N) epi_store4(a, m, n, acc.v[tn][mt]);
      }
    }
  }

  __device__ __forceinline__ static __amdgpu_buffer_rsrc_t slot_rsrc(const Args& a, int slot) {
    return make_rsrc((const char*)a.partials + (size_t)slot * (BM * BN * 4), BM * BN * 4);
  }
  __device__ __forceinline__ static uint32_t pofs(int tn, int mt) {
    return (uint32_t)((((wave_id() * TN + tn) * MT + mt) * 64 + lane_id()) * 16);
  }
  __device__ __forceinline__ static void write_partial(const Args& a, int slot, Acc& acc) {
    const auto r = slot_rsrc(a, slot);
#pragma unroll
    for (int tn = 0; tn < TN; ++tn)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) store_sc1_x4(r, pofs(tn, mt), __builtin_bit_cast(i32x4, acc.v[tn][mt]));
  }
  // Chunk c = tn * MT + mt of a lane's partial tile.
  using S4 = f32x4;
  static constexpr int NCH = TN * MT;
  __device__ __forceinline__ static bool holds_partial() { return true; }
  __device__ __forceinline__ static uint32_t chunk_off(int c) { return pofs(c / MT, c % MT); }
  __device__ __forceinline__ static S4 get4(const Acc& acc, int c) { return acc.v[c / MT][c % MT]; }
  __device__ __forceinline__ static void set4(Acc& acc, int c, const S4& x) { acc.v[c / MT][c % MT] = x; }
};

template <class Cfg>
hipError_t launch_w4(const Args& a, int grid, hipStream_t s) {
  return launch_sched<W4<Cfg>>(a, grid, s);
}

}  // namespace qg
