// Block-scaled fp8 GEMM core for gfx950: A and B hold OCP E4M3 codes, each
// with fp32 scales over blocks that are 128 deep along K,
//     a(i, k) = qa(i, k) * U[i, k / 128]                (1 x 128 blocks)
//     b(j, k) = qb(j, k) * V[e][j / 128, k / 128]       (128 x 128 blocks)
// (the U, V scale operands of the page "InternLM Lmdeploy Gemm Interface",
// I/O Contract; the scales advance once per group along K as in the page
// "InternLM Lmdeploy Gemm MainloopSm80V2", quantisation group tracking).
//
// One k-tile is exactly one 128-deep scale group. Its two 32x32x64 MFMAs per
// 32x32 output block sum the raw code products (exact in fp32) into a fresh
// block result; the k-tile then adds sa(i) * sb(block) * result to the fp32
// accumulator ("promotion" of a per-block partial sum, which the DeepGEMM
// write-up's fp8 discussion motivates; here the products are exact, so the
// only rounding is fp32 summation). In the swapped operand order each lane
// holds one row i of a block, so sa is one value per lane and sb one value
// per block.
//
// The operand tiles use the LDS ring, swizzle and fragment reads of the tile
// core (128-byte k rows, 16-byte chunks XOR (row >> 1) & 7); each stage also
// carries the k-tile's scales: waves 0 .. BM/64-1 load the A scales of 64 rows
// each, wave BM/64 the B scales of the tile's 128-column blocks, one dword per
// lane with the same direct global->LDS loads, so every wave issues the same
// number of loads per stage and the vmcnt bookkeeping stays uniform.
#pragma once
#include "qg_tile.hpp"

namespace qg {

template <int BM_, int BN_, int WM_, int WN_, int STAGES_>
struct F8Cfg : TileCfg<El::E4M3, BM_, BN_, WM_, WN_, STAGES_, 128> {
  using Base = TileCfg<El::E4M3, BM_, BN_, WM_, WN_, STAGES_, 128>;
  static constexpr int UA = BM_ / 64;                 // waves that load A scales
  static constexpr int SC_BYTES = Base::NW * 256;     // one 64-dword slot per wave
  static constexpr int STAGE8 = Base::STAGE_BYTES + SC_BYTES;
  static constexpr int LPW8 = Base::LPW + 1;          // + the scale load
  static_assert(BM_ % 64 == 0 && BN_ % 128 == 0, "scale blocks must tile the output tile");
  static_assert(Base::NW > UA, "one wave left over for the B scales");
  static_assert(BN_ / 128 <= 64, "B scale blocks per tile");
  static_assert(STAGES_ * STAGE8 <= 160 * 1024 - 1024, "LDS budget");
  static_assert(LPW8 * (STAGES_ - 2) < 64, "vmcnt range");
};

template <class Cfg>
struct F8 : Tile<Cfg> {
  using Base = Tile<Cfg>;
  using Acc = typename Base::Acc;
  static constexpr int TM = Cfg::TM, TN = Cfg::TN, BM = Cfg::BM, BN = Cfg::BN, NT = Cfg::NT;
  static constexpr int SMEM_BYTES = Cfg::STAGES * Cfg::STAGE8;

  __device__ __forceinline__ static void mainloop(const Args& a, const Unit& u, char* smem, Acc& acc) {
    const int w = wave_id(), l = lane_id();
    const int wm = w / Cfg::WAVES_N, wn = w % Cfg::WAVES_N;
    const int64_t lda_b = a.lda, ldb_b = a.ldb, ldu_b = a.ldu * 4, ldv_b = a.ldv * 4;
    const uint32_t kbytes = (uint32_t)a.K;
    const int a_rows = max(0, min(BM, u.m_end - u.m0));
    const int b_rows = max(0, min(BN, a.N - u.n0));
    const int b_blocks = (b_rows + 127) / 128;
    const char* Ab = (const char*)a.A + (int64_t)u.m0 * lda_b;
    const char* Bb = (const char*)a.B + (int64_t)u.expert * a.b_batch + (int64_t)u.n0 * ldb_b;
    const char* Ub = (const char*)a.U + (int64_t)u.m0 * ldu_b;
    const char* Vb = (const char*)a.V + (int64_t)u.expert * a.v_batch * 4 + (int64_t)(u.n0 / 128) * ldv_b;
    const i32x4 rA = make_rsrc_words(Ab, (uint32_t)(a_rows * lda_b));
    const i32x4 rB = make_rsrc_words(Bb, (uint32_t)(b_rows * ldb_b));
    const i32x4 rS = w < Cfg::UA ? make_rsrc_words(Ub, (uint32_t)(a_rows * ldu_b))
                                 : make_rsrc_words(Vb, (uint32_t)(b_blocks * ldv_b));

    constexpr int CPR = Cfg::CPR, RPI = Cfg::RPI;
    uint32_t offA[Cfg::LA], offB[Cfg::LB], chA[Cfg::LA], chB[Cfg::LB];
#pragma unroll
    for (int i = 0; i < Cfg::LA; ++i) {
      const int row = (w * Cfg::LA + i) * RPI + l / CPR;
      chA[i] = (uint32_t)(((l % CPR) ^ swz<CPR>(row)) * 16);
      offA[i] = (uint32_t)(row * lda_b) + chA[i];
    }
#pragma unroll
    for (int i = 0; i < Cfg::LB; ++i) {
      const int row = (w * Cfg::LB + i) * RPI + l / CPR;
      chB[i] = (uint32_t)(((l % CPR) ^ swz<CPR>(row)) * 16);
      offB[i] = (uint32_t)(row * ldb_b) + chB[i];
    }
    // this wave's scale dword: A scale of row 64w + l, or B scale of block l
    bool s_lane;
    uint32_t offS;
    if (w < Cfg::UA) {
      const int row = w * 64 + l;
      s_lane = row < a_rows;
      offS = (uint32_t)(row * ldu_b);
    } else {
      s_lane = (w == Cfg::UA) && l < b_blocks;
      offS = (uint32_t)(l * ldv_b);
    }

    auto issue = [&](int stage, int kt) {
      char* sbase = smem + stage * Cfg::STAGE8;
      const uint32_t kk = (uint32_t)kt * 128;
      const bool live = kt < u.ke;
#pragma unroll
      for (int i = 0; i < Cfg::LA; ++i)
        load_lds_x4(rA, sbase + (w * Cfg::LA + i) * 1024, live && kk + chA[i] < kbytes ? offA[i] + kk : kOOB);
#pragma unroll
      for (int i = 0; i < Cfg::LB; ++i)
        load_lds_x4(rB, sbase + Cfg::A_BYTES + (w * Cfg::LB + i) * 1024, live && kk + chB[i] < kbytes ? offB[i] + kk : kOOB);
      load_lds_x1a(rS, sbase + Cfg::STAGE_BYTES + w * 256, live && s_lane ? offS + (uint32_t)kt * 4 : kOOB);
    };

    // K not a multiple of 16: zero the bytes past K in the chunks this lane
    // loaded for the k-tile that holds K's end (as in the tile core).
    const int ktail = (kbytes & 15) ? (int)((kbytes - 1) / 128) : -1;
    auto trim = [&](int stage, int kt) {
      const uint32_t kb = pinned(kbytes);  // keeps this work inside the branch
      char* sbase = smem + stage * Cfg::STAGE8;
      const uint32_t kk = (uint32_t)kt * 128;
#pragma unroll
      for (int i = 0; i < Cfg::LA; ++i) {
        const int keep = (int)(kb - kk - chA[i]);
        if (keep > 0 && keep < 16) lds_chunk_trim(sbase + (w * Cfg::LA + i) * 1024 + l * 16, keep);
      }
#pragma unroll
      for (int i = 0; i < Cfg::LB; ++i) {
        const int keep = (int)(kb - kk - chB[i]);
        if (keep > 0 && keep < 16) lds_chunk_trim(sbase + Cfg::A_BYTES + (w * Cfg::LB + i) * 1024 + l * 16, keep);
      }
    };

    // Fragments of one 64-deep k-step: lane l takes row l % 32 and the 32
    // contiguous bytes of k selected by l / 32, for A and B alike.
    const int orow = l & 31, ohalf = l >> 5;
    struct Frags {
      i32x8 a[TM], b[TN];
    };
    auto read_frags = [&](int stage, int ks, Frags& f) {
      const char* sA = smem + stage * Cfg::STAGE8;
      const char* sB = sA + Cfg::A_BYTES;
      const int c0 = ks * 4 + ohalf * 2;
#pragma unroll
      for (int tm = 0; tm < TM; ++tm) {
        const int row = wm * Cfg::WTM + tm * 32 + orow;
        const i32x4 x0 = *(const i32x4*)(sA + row * 128 + ((c0 ^ swz<CPR>(row)) << 4));
        const i32x4 x1 = *(const i32x4*)(sA + row * 128 + (((c0 + 1) ^ swz<CPR>(row)) << 4));
        f.a[tm] = i32x8{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
      }
#pragma unroll
      for (int tn = 0; tn < TN; ++tn) {
        const int row = wn * Cfg::WTN + tn * 32 + orow;
        const i32x4 x0 = *(const i32x4*)(sB + row * 128 + ((c0 ^ swz<CPR>(row)) << 4));
        const i32x4 x1 = *(const i32x4*)(sB + row * 128 + (((c0 + 1) ^ swz<CPR>(row)) << 4));
        f.b[tn] = i32x8{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
      }
    };

#pragma unroll
    for (int tn = 0; tn < TN; ++tn)
#pragma unroll
      for (int tm = 0; tm < TM; ++tm) acc.v[tn][tm] = f32x16{};

    const int nk = u.ke - u.kb;
    constexpr int S = Cfg::STAGES;
#pragma unroll
    for (int st = 0; st < S; ++st) issue(st, u.kb + st);
    wait_vmcnt<Cfg::LPW8 * (S - 1)>();
    if (u.kb == ktail) trim(0, ktail);
    lds_barrier();
    for (int it = 0; it < nk; ++it) {
      const int st = it % S;
      const char* sbase = smem + st * Cfg::STAGE8;
      const float* sc = (const float*)(sbase + Cfg::STAGE_BYTES);
      Frags f0, f1;
      read_frags(st, 0, f0);
      read_frags(st, 1, f1);
      float sa[TM], sb[TN];
#pragma unroll
      for (int tm = 0; tm < TM; ++tm) sa[tm] = sc[wm * Cfg::WTM + tm * 32 + orow];
#pragma unroll
      for (int tn = 0; tn < TN; ++tn) sb[tn] = sc[Cfg::UA * 64 + (wn * Cfg::WTN + tn * 32) / 128];
      f32x16 t[TN][TM];
#pragma unroll
      for (int tn = 0; tn < TN; ++tn)
#pragma unroll
        for (int tm = 0; tm < TM; ++tm) t[tn][tm] = mfma_e4m3(f0.b[tn], f0.a[tm], f32x16{});
#pragma unroll
      for (int tn = 0; tn < TN; ++tn)
#pragma unroll
        for (int tm = 0; tm < TM; ++tm) t[tn][tm] = mfma_e4m3(f1.b[tn], f1.a[tm], t[tn][tm]);
      // every wave has read stage st (fragments and scales): refill it with
      // k-tile it + S; the wait makes stage it + 1 resident for the next step
      wait_vmcnt<Cfg::LPW8 * (S - 2)>();
      if (u.kb + it + 1 == ktail) trim((it + 1) % S, ktail);
      lds_barrier();
      issue(st, u.kb + it + S);
      // promotion of the k-tile's raw sums (measured: faster here, after the
      // barrier, than interleaved block by block with the MFMAs)
#pragma unroll
      for (int tn = 0; tn < TN; ++tn)
#pragma unroll
        for (int tm = 0; tm < TM; ++tm) {
          const float f = sa[tm] * sb[tn];
#pragma unroll
          for (int r = 0; r < 16; ++r) acc.v[tn][tm][r] = __builtin_fmaf(f, t[tn][tm][r], acc.v[tn][tm][r]);
        }
    }
    // The last k-steps issued loads for k-tiles past the unit (out-of-range
    // offsets, which still write zeros into the ring). The compiler does not
    // count these inline-assembly loads, so __syncthreads() alone would not
    // wait for them: wait explicitly before the ring is reused (staged
    // epilogue, next unit's prologue).
    wait_vmcnt<0>();
    __syncthreads();
  }
};

template <class Cfg>
hipError_t launch_f8(const Args& a, int grid, hipStream_t s) {
  return launch_sched<F8<Cfg>>(a, grid, s);
}

}  // namespace qg
