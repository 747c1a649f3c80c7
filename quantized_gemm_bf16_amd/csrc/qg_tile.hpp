// LDS-staged MFMA tile kernel for gfx950.
//
// One workgroup owns a BM x BN output tile (or a k-range of it). K is walked
// in k-tiles of ROWB (128 or 64) bytes per row (128 bytes = 64 bf16/fp16 or
// 128 int8/e4m3 elements).
// Operand tiles go from global memory straight into an S-stage LDS ring with
// buffer_load ... lds (16 bytes per lane), so no VGPRs are spent on staging;
// the ring follows the multi-stage mainloop of the page "InternLM Lmdeploy
// Gemm MainloopSm80V2" (prologue fills S-1 stages, each step waits for the
// stage it is about to read, then issues the next stage before computing).
// Rows are 128 bytes = 8 chunks of 16 bytes, stored with chunk' = chunk ^
// ((row >> 1) & 7): the XOR swizzle of the DeepGEMM write-up (section 3.2, and
// the 8-element granularity of section 5.2) taken on 16-byte chunks. gfx950
// serves a 16-byte-per-lane LDS read 16 lanes (256 bytes, all 64 banks) per
// clock; the 16 lanes of a group read the same logical chunk of 16
// consecutive rows, and the key (row >> 1) & 7 sends them to 16 distinct
// 16-byte bank groups (two rows span the 256 bytes of the banks).
// The schedules that drive it (DP / split-K / stream-K / grouped) live in
// qg_sched.hpp.
#pragma once
#include "qg_args.hpp"
#include "qg_device.hpp"
#include "qg_sched.hpp"

namespace qg {

enum class El { BF16, F16, I8, E4M3 };

// ROWB_: bytes of k per row in one k-tile (128: 64 bf16 / 128 int8; 64: half that).
template <El E_, int BM_, int BN_, int WM_, int WN_, int STAGES_, int ROWB_ = 128>
struct TileCfg {
  static constexpr El E = E_;
  static constexpr int BM = BM_, BN = BN_, WAVES_M = WM_, WAVES_N = WN_, STAGES = STAGES_;
  static constexpr int NW = WM_ * WN_, NT = NW * 64;
  static constexpr int WTM = BM / WM_, WTN = BN / WN_;
  static constexpr int TM = WTM / 32, TN = WTN / 32;
  static constexpr int ESIZE = (E_ == El::BF16 || E_ == El::F16) ? 2 : 1;
  static constexpr int CH = (E_ == El::E4M3) ? 2 : 1;  // 16-byte chunks per lane per MFMA
  static constexpr int ROWB = ROWB_;
  static constexpr int CPR = ROWB / 16;                  // 16-byte chunks per row
  static constexpr int RPI = 64 / CPR;                   // rows filled by one 64-lane load
  static constexpr int KSTEPS = CPR / (2 * CH);          // MFMAs along k per k-tile
  static constexpr int BK = ROWB / ESIZE;                // elements per k-tile
  static constexpr int A_BYTES = BM * ROWB, B_BYTES = BN * ROWB;
  static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
  static constexpr int LA = BM / RPI / NW, LB = BN / RPI / NW;  // 64-lane loads per wave slot per stage
  static constexpr int LPW = LA + LB;
  static constexpr bool INT = (E_ == El::I8);
  static_assert(ROWB == 64 || ROWB == 128, "k-tile row bytes");
  static_assert(KSTEPS >= 1, "k-tile shorter than one MFMA");
  static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be a multiple of 32");
  static_assert(LA * RPI * NW == BM && LB * RPI * NW == BN, "tile rows must split evenly over waves");
  static_assert(STAGES >= 2 && STAGES * STAGE_BYTES <= 160 * 1024 - 1024, "LDS budget");
  static_assert(2 * LPW * (STAGES - 1) < 64, "vmcnt range (the first half of the waves issues all loads)");
};

template <bool INT>
struct AccOf;
template <>
struct AccOf<false> {
  using V = f32x16;
  using S = float;
  using S4 = f32x4;
};
template <>
struct AccOf<true> {
  using V = i32x16;
  using S = int;
  using S4 = i32x4;
};

// XOR key of a row's 16-byte chunks in LDS: 16 consecutive rows must cover
// the 16 bank groups of 256 bytes; a row holds CPR chunks, so rows r and
// r + 256/ROWB share banks and get different keys.
template <int CPR>
__device__ __forceinline__ int swz(int row) { return (row / (16 / CPR)) & (CPR - 1); }


// ---- epilogue helpers -------------------------------------------------------
__device__ __forceinline__ void load_c4(const Args& a, int64_t m, int n, float v[4]) {
  const int64_t base = m * a.ldc + n;
  const bool full = n + 3 < a.N;
  switch (a.c_type) {
    case DT_F32: {
      const float* p = (const float*)a.C + base;
      if (full) {
        f32x4 x = *(const f32x4*)p;
        v[0] = x[0], v[1] = x[1], v[2] = x[2], v[3] = x[3];
      } else
        for (int j = 0; j < 4; ++j) v[j] = (n + j < a.N) ? p[j] : 0.f;
      break;
    }
    case DT_BF16:
    case DT_F16: {
      const uint16_t* p = (const uint16_t*)a.C + base;
      uint16_t h[4];
      if (full) {
        u16x4 x = *(const u16x4*)p;
        h[0] = x[0], h[1] = x[1], h[2] = x[2], h[3] = x[3];
      } else
        for (int j = 0; j < 4; ++j) h[j] = (n + j < a.N) ? p[j] : 0;
      for (int j = 0; j < 4; ++j) v[j] = a.c_type == DT_BF16 ? bf16_bits_to_f32(h[j]) : f16_bits_to_f32(h[j]);
      break;
    }
    default:
      v[0] = v[1] = v[2] = v[3] = 0.f;
  }
}

__device__ __forceinline__ void store_d4(const Args& a, int64_t m, int n, const float v[4]) {
  const int64_t base = m * a.ldd + n;
  const bool full = n + 3 < a.N;
  switch (a.d_type) {
    case DT_F32: {
      float* p = (float*)a.D + base;
      if (full)
        *(f32x4*)p = f32x4{v[0], v[1], v[2], v[3]};
      else
        for (int j = 0; j < 4; ++j)
          if (n + j < a.N) p[j] = v[j];
      break;
    }
    case DT_BF16:
    case DT_F16: {
      uint16_t h[4];
      for (int j = 0; j < 4; ++j) h[j] = a.d_type == DT_BF16 ? f32_to_bf16_bits(v[j]) : f32_to_f16_bits(v[j]);
      uint16_t* p = (uint16_t*)a.D + base;
      if (full)
        *(u16x4*)p = u16x4{h[0], h[1], h[2], h[3]};
      else
        for (int j = 0; j < 4; ++j)
          if (n + j < a.N) p[j] = h[j];
      break;
    }
    default:
      break;
  }
}

// Fused epilogue steps after alpha/beta (the DeepGEMM write-up, section 6:
// bias and activation, then per-row output quantisation). The flags are
// kernel arguments: uniform branches, evaluated once per 4 outputs.
__device__ __forceinline__ void epi_fused(const Args& a, int64_t m, int n, float v[4]) {
  if (a.epi & EPI_BIAS) {
    float b[4];
    const bool full = n + 3 < a.N;
    if (a.bias_type == DT_F32) {
      const float* p = (const float*)a.bias + n;
      if (full) {
        const f32x4 x = *(const f32x4*)p;
        b[0] = x[0], b[1] = x[1], b[2] = x[2], b[3] = x[3];
      } else
        for (int j = 0; j < 4; ++j) b[j] = (n + j < a.N) ? p[j] : 0.f;
    } else {
      const uint16_t* p = (const uint16_t*)a.bias + n;
      uint16_t h[4];
      if (full) {
        const u16x4 x = *(const u16x4*)p;
        h[0] = x[0], h[1] = x[1], h[2] = x[2], h[3] = x[3];
      } else
        for (int j = 0; j < 4; ++j) h[j] = (n + j < a.N) ? p[j] : 0;
      for (int j = 0; j < 4; ++j) b[j] = a.bias_type == DT_BF16 ? bf16_bits_to_f32(h[j]) : f16_bits_to_f32(h[j]);
    }
    for (int j = 0; j < 4; ++j) v[j] += b[j];
  }
  if (a.epi & EPI_RELU)
    for (int j = 0; j < 4; ++j) v[j] = v[j] > 0.f ? v[j] : 0.f;
  if (a.epi & EPI_GELU)
    for (int j = 0; j < 4; ++j) v[j] = 0.5f * v[j] * (1.f + erff(v[j] * 0.70710678118654752f));
}

// int8 output codes: saturate(round_half_even(x * row_scale[m] + zero_point))
__device__ __forceinline__ void store_q4(const Args& a, int64_t m, int n, const float v[4]) {
  const float s = a.row_scale[m];
  int q[4];
  for (int j = 0; j < 4; ++j) {
    const float t = rintf(__builtin_fmaf(v[j], s, a.out_zero_point));
    q[j] = (int)fminf(fmaxf(t, -128.f), 127.f);
  }
  int8_t* p = (int8_t*)a.D + m * a.ldd + n;
  if (n + 3 < a.N)
    *(uint32_t*)p = (uint32_t)(q[0] & 0xFF) | ((uint32_t)(q[1] & 0xFF) << 8) | ((uint32_t)(q[2] & 0xFF) << 16) |
                    ((uint32_t)(q[3] & 0xFF) << 24);
  else
    for (int j = 0; j < 4; ++j)
      if (n + j < a.N) p[j] = (int8_t)q[j];
}

// D = alpha * acc (+ beta * c, c already loaded), then the fused steps -> D
__device__ __forceinline__ void epi_store4c(const Args& a, int64_t m, int n, const f32x4& acc, const f32x4& c) {
  float v[4] = {a.alpha * acc[0], a.alpha * acc[1], a.alpha * acc[2], a.alpha * acc[3]};
  if (a.c_type >= 0 && a.beta != 0.f)
    for (int j = 0; j < 4; ++j) v[j] = __builtin_fmaf(a.beta, c[j], v[j]);
  if (a.epi) {
    epi_fused(a, m, n, v);
    if (a.epi & EPI_QUANT_I8) {
      store_q4(a, m, n, v);
      return;
    }
  }
  store_d4(a, m, n, v);
}

__device__ __forceinline__ void epi_store4(const Args& a, int64_t m, int n, const f32x4& acc) {
  float c[4] = {0.f, 0.f, 0.f, 0.f};
  if (a.c_type >= 0 && a.beta != 0.f) load_c4(a, m, n, c);
  epi_store4c(a, m, n, acc, f32x4{c[0], c[1], c[2], c[3]});
}

// int8 path: D = acc (+ C when beta == 1), exact int32; with per-row scales
// of A and B (w8a8) the exact sum is scaled in fp32 and takes the float
// epilogue: x = acc * U[m] * V[n].
__device__ __forceinline__ void epi_store4(const Args& a, int64_t m, int n, const i32x4& acc) {
  if (a.int_scaled) {
    const float sa = ((const float*)a.U)[m * a.ldu];
    const float* vb = (const float*)a.V;
    f32x4 x;
    for (int j = 0; j < 4; ++j) x[j] = (n + j < a.N) ? (float)acc[j] * sa * vb[(int64_t)(n + j) * a.ldv] : 0.f;
    float c[4] = {0.f, 0.f, 0.f, 0.f};
    if (a.c_type >= 0 && a.beta != 0.f) load_c4(a, m, n, c);
    epi_store4c(a, m, n, x, f32x4{c[0], c[1], c[2], c[3]});
    return;
  }
  int v[4] = {acc[0], acc[1], acc[2], acc[3]};
  const bool full = n + 3 < a.N;
  if (a.c_type == DT_I32 && a.beta != 0.f) {
    const int* c = (const int*)a.C + m * a.ldc + n;
    for (int j = 0; j < 4; ++j) v[j] += (n + j < a.N) ? c[j] : 0;
  }
  int* p = (int*)a.D + m * a.ldd + n;
  if (full)
    *(i32x4*)p = i32x4{v[0], v[1], v[2], v[3]};
  else
    for (int j = 0; j < 4; ++j)
      if (n + j < a.N) p[j] = v[j];
}

// Scheduling hint: spread NR LDS reads over the next NM MFMAs (PER reads after
// each MFMA) so that the reads of the next k-step's fragments overlap the
// current k-step's MFMAs instead of being issued after them.
template <int NR, int NM, int PER>
struct Interleave {
  __device__ __forceinline__ static void emit() {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if constexpr (NR > 0) __builtin_amdgcn_sched_group_barrier(0x100, NR < PER ? NR : PER, 0);
    if constexpr (NM > 1) Interleave<(NR > PER ? NR - PER : 0), NM - 1, PER>::emit();
  }
};
template <int NR, int NM>
__device__ __forceinline__ void interleave_reads() {
  Interleave<NR, NM, (NR + NM - 1) / NM>::emit();
}

// ---- the kernel body -----------------------------------------------------
template <class Cfg>
struct Tile {
  using AO = AccOf<Cfg::INT>;
  using AccV = typename AO::V;
  using S4 = typename AO::S4;
  static constexpr int TN = Cfg::TN, TM = Cfg::TM;
  static constexpr int NQ = TN * TM * 4;  // 4-element groups per lane
  static constexpr int BM = Cfg::BM, BN = Cfg::BN, NT = Cfg::NT;
  static constexpr int SMEM_BYTES = Cfg::STAGES * Cfg::STAGE_BYTES;
  struct Acc {
    AccV v[TN][TM];
  };

  __device__ __forceinline__ static void mainloop(const Args& a, const Unit& u, char* smem, Acc& acc) {
    const int w = wave_id(), l = lane_id();
    const int wm = w / Cfg::WAVES_N, wn = w % Cfg::WAVES_N;
    const int64_t lda_b = a.lda * Cfg::ESIZE, ldb_b = a.ldb * Cfg::ESIZE;
    const uint32_t kbytes = (uint32_t)a.K * Cfg::ESIZE;
    const char* Ab = (const char*)a.A + (int64_t)u.m0 * lda_b;
    const char* Bb = (const char*)a.B + (int64_t)u.expert * a.b_batch * Cfg::ESIZE + (int64_t)u.n0 * ldb_b;
    const int a_rows = max(0, min(Cfg::BM, u.m_end - u.m0));
    const int b_rows = max(0, min(Cfg::BN, a.N - u.n0));
    const i32x4 rA = make_rsrc_words(Ab, (uint32_t)(a_rows * lda_b));
    const i32x4 rB = make_rsrc_words(Bb, (uint32_t)(b_rows * ldb_b));

    // Each 64-lane load fills RPI rows x ROWB bytes of LDS (lane l -> row
    // l / CPR, physical chunk l % CPR); the lane fetches the logical chunk
    // that the swizzle stores there.
    constexpr int CPR = Cfg::CPR, RPI = Cfg::RPI, ROWB = Cfg::ROWB;
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

    // Loads k-tile kt into ring stage `stage`; k-tiles outside [u.kb, u.ke)
    // (the ring runs STAGES tiles ahead) get an out-of-range offset, which
    // reads nothing and keeps the per-wave load count, and so vmcnt, uniform.
    // A k-tile that lies wholly inside K (the usual case) takes the uniform
    // branch without per-lane range selects.
    // The first half of the waves issues every load of a stage: wave w < HALF
    // fills its own row slots and those of wave w + HALF (rows HALF LA RPI
    // further on, under the same swizzle key). The two waves of a SIMD are
    // w and w + HALF; the older one wins the issue arbitration and reaches
    // the k-tile barrier first, so the younger one, on the critical path,
    // is the one relieved of the load issue (measured: 2770-2780 instead of
    // 2985 shader cycles per 64-deep k-tile for the 256 x 256 tile).
    constexpr int HALF = Cfg::NW / 2;
    static_assert((HALF * Cfg::LA * RPI) % 16 == 0 && (HALF * Cfg::LB * RPI) % 16 == 0,
                  "the second half's rows keep the swizzle key (period 16 rows)");
    const uint32_t stepA = (uint32_t)(HALF * Cfg::LA * RPI * lda_b), stepB = (uint32_t)(HALF * Cfg::LB * RPI * ldb_b);
    auto issue = [&](int stage, int kt) {
      if (w >= HALF) return;
      char* sbase = smem + stage * Cfg::STAGE_BYTES;
      const uint32_t kk = (uint32_t)kt * ROWB;
      const bool live = kt < u.ke;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int ws = w + h * HALF;
        if (live && kk + ROWB <= kbytes) {
#pragma unroll
          for (int i = 0; i < Cfg::LA; ++i) load_lds_x4(rA, sbase + (ws * Cfg::LA + i) * 1024, offA[i] + h * stepA + kk);
#pragma unroll
          for (int i = 0; i < Cfg::LB; ++i)
            load_lds_x4(rB, sbase + Cfg::A_BYTES + (ws * Cfg::LB + i) * 1024, offB[i] + h * stepB + kk);
        } else {
#pragma unroll
          for (int i = 0; i < Cfg::LA; ++i)
            load_lds_x4(rA, sbase + (ws * Cfg::LA + i) * 1024,
                        live && kk + chA[i] < kbytes ? offA[i] + h * stepA + kk : kOOB);
#pragma unroll
          for (int i = 0; i < Cfg::LB; ++i)
            load_lds_x4(rB, sbase + Cfg::A_BYTES + (ws * Cfg::LB + i) * 1024,
                        live && kk + chB[i] < kbytes ? offB[i] + h * stepB + kk : kOOB);
        }
      }
    };

    // K * ESIZE not a multiple of 16: the k-tile `ktail` holds each row's
    // chunk that straddles K. Once this lane's loads of that k-tile have
    // landed (and before the barrier that publishes the stage), it zeroes the
    // bytes past K in the chunks it loaded.
    const int ktail = (kbytes & 15) ? (int)((kbytes - 1) / ROWB) : -1;
    // zeroes the bytes past K in the chunks this lane loaded (both halves)
    auto trim = [&](int stage, int kt) {
      if (w >= HALF) return;
      const uint32_t kb = pinned(kbytes);  // keeps this work inside the branch
      char* sbase = smem + stage * Cfg::STAGE_BYTES;
      const uint32_t kk = (uint32_t)kt * ROWB;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int ws = w + h * HALF;
#pragma unroll
        for (int i = 0; i < Cfg::LA; ++i) {
          const int keep = (int)(kb - kk - chA[i]);
          if (keep > 0 && keep < 16) lds_chunk_trim(sbase + (ws * Cfg::LA + i) * 1024 + l * 16, keep);
        }
#pragma unroll
        for (int i = 0; i < Cfg::LB; ++i) {
          const int keep = (int)(kb - kk - chB[i]);
          if (keep > 0 && keep < 16) lds_chunk_trim(sbase + Cfg::A_BYTES + (ws * Cfg::LB + i) * 1024 + l * 16, keep);
        }
      }
    };

    // MFMA operand fragments of one k-step, read from LDS.
    const int orow = l & 31, ohalf = l >> 5;
    struct Frags {
      i32x4 a[TM][Cfg::CH], b[TN][Cfg::CH];
    };
    auto read_frags = [&](int stage, int ks, Frags& f) {
      const char* sA = smem + stage * Cfg::STAGE_BYTES;
      const char* sB = sA + Cfg::A_BYTES;
#pragma unroll
      for (int tm = 0; tm < TM; ++tm) {
        const int row = wm * Cfg::WTM + tm * 32 + orow;
#pragma unroll
        for (int c = 0; c < Cfg::CH; ++c) {
          const int lc = ks * 2 * Cfg::CH + ohalf * Cfg::CH + c;
          f.a[tm][c] = *(const i32x4*)(sA + row * ROWB + ((lc ^ swz<CPR>(row)) << 4));
        }
      }
#pragma unroll
      for (int tn = 0; tn < TN; ++tn) {
        const int row = wn * Cfg::WTN + tn * 32 + orow;
#pragma unroll
        for (int c = 0; c < Cfg::CH; ++c) {
          const int lc = ks * 2 * Cfg::CH + ohalf * Cfg::CH + c;
          f.b[tn][c] = *(const i32x4*)(sB + row * ROWB + ((lc ^ swz<CPR>(row)) << 4));
        }
      }
    };
    // MFMAs of one k-step over the n-tiles [tn0, tn1) of the wave tile.
    auto mma = [&](const Frags& f, int tn0, int tn1) {
#pragma unroll
      for (int tn = 0; tn < TN; ++tn)
#pragma unroll
        for (int tm = 0; tm < TM; ++tm) {
          if (tn < tn0 || tn >= tn1) continue;
          if constexpr (Cfg::E == El::BF16)
            acc.v[tn][tm] = mfma_bf16(f.b[tn][0], f.a[tm][0], acc.v[tn][tm]);
          else if constexpr (Cfg::E == El::F16)
            acc.v[tn][tm] = mfma_f16(f.b[tn][0], f.a[tm][0], acc.v[tn][tm]);
          else if constexpr (Cfg::E == El::I8)
            acc.v[tn][tm] = mfma_i8(f.b[tn][0], f.a[tm][0], acc.v[tn][tm]);
        }
    };

#pragma unroll
    for (int tn = 0; tn < TN; ++tn)
#pragma unroll
      for (int tm = 0; tm < TM; ++tm) acc.v[tn][tm] = AccV{};

    const int nk = u.ke - u.kb;
    constexpr int S = Cfg::STAGES, KS = Cfg::KSTEPS;
    // Prologue: fill all S stages, wait for the first.
#pragma unroll
    for (int st = 0; st < S; ++st) issue(st, u.kb + st);
    wait_vmcnt<2 * Cfg::LPW * (S - 1)>();  // the loading waves hold 2 LPW loads per stage
    if (u.kb == ktail) trim(0, ktail);
    lds_barrier();
    Frags cur;
    read_frags(0, 0, cur);
    for (int it = 0; it < nk; ++it) {
      const int st = it % S;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        Frags nxt;
        if (ks + 1 < KS) {
          read_frags(st, ks + 1, nxt);
          mma(cur, 0, TN);
          interleave_reads<(TM + TN) * Cfg::CH, TM * TN>();
        } else {
          // Last k-step of this stage: its fragments are already in registers.
          // Half of its MFMAs cover the wait for the next stage; after the
          // barrier every wave has finished reading stage `st`, which is then
          // refilled with k-tile it + S, and the next stage's first fragments
          // are read while the other half of the MFMAs run.
          mma(cur, 0, TN / 2);
          wait_vmcnt<2 * Cfg::LPW * (S - 2)>();
          if (u.kb + it + 1 == ktail) trim((it + 1) % S, ktail);
          lds_barrier();
          issue(st, u.kb + it + S);
          read_frags((it + 1) % S, 0, nxt);
          mma(cur, TN / 2, TN);
          interleave_reads<(TM + TN) * Cfg::CH, TM * (TN - TN / 2)>();
        }
        cur = nxt;
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

  // Plain epilogue D = alpha * acc in a 16-bit type (no C, no fused steps):
  // the MFMA layout leaves a lane 4 consecutive columns of one row, so stores
  // straight from registers write 16-byte pieces of 32 different rows per
  // instruction. Instead each wave stages its converted WTM x WTN tile in its
  // own part of the (now idle) LDS ring and writes it back as whole row
  // segments of WTN * 2 bytes. Staged rows keep 16-byte chunks under the same
  // XOR key as the operand ring, so the 32 rows written by one instruction
  // spread over the banks.
  static constexpr int WROWB = Cfg::WTN * 2;  // bytes of one staged row
  static constexpr int WCH = WROWB / 16;      // 16-byte chunks per staged row
  static constexpr int WRPI = 64 / WCH;       // staged rows per 64-lane read
  static constexpr bool STAGED = !Cfg::INT && WCH >= 4 && WCH <= 16 &&
                                 Cfg::NW * Cfg::WTM * WROWB <= Cfg::STAGES * Cfg::STAGE_BYTES;
  __device__ __forceinline__ static bool plain16(const Args& a) {
    return (a.d_type == DT_BF16 || a.d_type == DT_F16) && (a.c_type < 0 || a.beta == 0.f) && a.epi == 0;
  }

  __device__ __forceinline__ static void store_staged(const Args& a, const Unit& u, Acc& acc, char* smem) {
    const int w = wave_id(), l = lane_id();
    const int wm = w / Cfg::WAVES_N, wn = w % Cfg::WAVES_N;
    char* st = smem + w * (Cfg::WTM * WROWB);
    const bool bf = a.d_type == DT_BF16;
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) {
      const int row = tm * 32 + (l & 31);
#pragma unroll
      for (int tn = 0; tn < TN; ++tn)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          uint16_t h[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float x = a.alpha * acc.v[tn][tm][4 * g + j];
            h[j] = bf ? f32_to_bf16_bits(x) : f32_to_f16_bits(x);
          }
          const int ch = tn * 4 + g;
          *(u16x4*)(st + row * WROWB + ((ch ^ swz<WCH>(row)) << 4) + 8 * (l >> 5)) = u16x4{h[0], h[1], h[2], h[3]};
        }
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // this wave's LDS writes are done (lgkmcnt 0)
    __builtin_amdgcn_wave_barrier();
    const int ch = l % WCH;
    const int n = u.n0 + wn * Cfg::WTN + ch * 8;
#pragma unroll
    for (int i = 0; i < Cfg::WTM / WRPI; ++i) {
      const int row = i * WRPI + l / WCH;
      const i32x4 v = *(const i32x4*)(st + row * WROWB + ((ch ^ swz<WCH>(row)) << 4));
      const int64_t m = u.m0 + wm * Cfg::WTM + row;
      if (m >= u.m_end || n >= a.N) continue;
      uint16_t* p = (uint16_t*)a.D + m * a.ldd + n;
      if (n + 8 <= a.N) {
        // non-temporal: D is written once and not read back by this launch
        // (measured: about 4k cycles less per 256x256 tile than plain stores)
        __builtin_nontemporal_store(v, (i32x4*)p);
      } else {
        const uint16_t* hv = (const uint16_t*)&v;
        for (int j = 0; j < 8; ++j)
          if (n + j < a.N) p[j] = hv[j];
      }
    }
    __syncthreads();  // the staging area is the next unit's ring
  }

  // Final results of a tile: epilogue + masked store.
  __device__ __forceinline__ static void store(const Args& a, const Unit& u, Acc& acc, char* smem) {
    if constexpr (STAGED) {
      if (plain16(a)) {
        store_staged(a, u, acc, smem);
        return;
      }
    }
    const int w = wave_id(), l = lane_id();
    const int wm = w / Cfg::WAVES_N, wn = w % Cfg::WAVES_N;
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) {
      const int m = u.m0 + wm * Cfg::WTM + tm * 32 + (l & 31);
      if (m >= u.m_end) continue;
#pragma unroll
      for (int tn = 0; tn < TN; ++tn)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int n = u.n0 + wn * Cfg::WTN + tn * 32 + 8 * g + 4 * (l >> 5);
          if (n >= a.N) continue;
          S4 v = {acc.v[tn][tm][4 * g], acc.v[tn][tm][4 * g + 1], acc.v[tn][tm][4 * g + 2], acc.v[tn][tm][4 * g + 3]};
          epi_store4(a, m, n, v);
        }
    }
  }

  // Partial tiles are stored lane-major ([wave][group][lane] x 16 bytes, fully
  // coalesced) and move between workgroups with sc1 (agent-coherent) buffer
  // accesses: they bypass the non-coherent per-XCD L2 state, so no L2
  // write-back or invalidate (what an agent-scope fence costs) is needed.
  __device__ __forceinline__ static __amdgpu_buffer_rsrc_t slot_rsrc(const Args& a, int slot) {
    return make_rsrc((const char*)a.partials + (size_t)slot * (Cfg::BM * Cfg::BN * 4), Cfg::BM * Cfg::BN * 4);
  }

  __device__ __forceinline__ static void write_partial(const Args& a, int slot, Acc& acc) {
    const auto r = slot_rsrc(a, slot);
    const uint32_t base = (uint32_t)((wave_id() * NQ * 64 + lane_id()) * 16);
#pragma unroll
    for (int tn = 0; tn < TN; ++tn)
#pragma unroll
      for (int tm = 0; tm < TM; ++tm)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int q = (tn * TM + tm) * 4 + g;
          S4 v = {acc.v[tn][tm][4 * g], acc.v[tn][tm][4 * g + 1], acc.v[tn][tm][4 * g + 2], acc.v[tn][tm][4 * g + 3]};
          store_sc1_x4(r, base + q * 1024, __builtin_bit_cast(i32x4, v));
        }
  }

  // Chunk c = (tn * TM + tm) * 4 + g of a lane's partial tile: accumulator
  // elements 4g .. 4g+3 of block (tn, tm), stored at base + 1024 c.
  static constexpr int NCH = NQ;
  __device__ __forceinline__ static bool holds_partial() { return true; }
  __device__ __forceinline__ static uint32_t chunk_off(int c) {
    return (uint32_t)((wave_id() * NQ * 64 + lane_id()) * 16 + c * 1024);
  }
  __device__ __forceinline__ static S4 get4(const Acc& acc, int c) {
    const int tn = c / (TM * 4), tm = (c / 4) % TM, g = c % 4;
    return S4{acc.v[tn][tm][4 * g], acc.v[tn][tm][4 * g + 1], acc.v[tn][tm][4 * g + 2], acc.v[tn][tm][4 * g + 3]};
  }
  __device__ __forceinline__ static void set4(Acc& acc, int c, const S4& x) {
    const int tn = c / (TM * 4), tm = (c / 4) % TM, g = c % 4;
#pragma unroll
    for (int j = 0; j < 4; ++j) acc.v[tn][tm][4 * g + j] = x[j];
  }
};

}  // namespace qg

namespace qg {

// Host-side launcher of one registered tile kernel.
template <class Cfg>
hipError_t launch_tile(const Args& a, int grid, hipStream_t s) {
  return launch_sched<Tile<Cfg>>(a, grid, s);
}

}  // namespace qg
