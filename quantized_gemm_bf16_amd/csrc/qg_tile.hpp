// LDS-staged MFMA tile kernel for gfx950.
//
// One workgroup owns a BM x BN output tile (or a k-range of it). K is walked
// in k-tiles of 128 bytes per row (64 bf16/fp16, 128 int8/e4m3 elements).
// Operand tiles go from global memory straight into an S-stage LDS ring with
// buffer_load ... lds (16 bytes per lane), so no VGPRs are spent on staging;
// the ring follows the multi-stage mainloop of the page "InternLM Lmdeploy
// Gemm MainloopSm80V2" (prologue fills S-1 stages, each step waits for the
// stage it is about to read, then issues the next stage before computing).
// Rows are 128 bytes = 8 chunks of 16 bytes, stored with chunk' = chunk ^
// (row & 7): the XOR swizzle of the DeepGEMM write-up (section 3.2, and the
// 8-element granularity of section 5.2) taken on 16-byte chunks, so that the
// 32 rows an MFMA operand read touches spread over all LDS banks.
//
// Work division (one kernel, chosen at run time):
//   DP       one unit = one whole tile; blockIdx remapped so that tiles that
//            share A/B panels run on the same XCD (each XCD has its own L2).
//   SPLITK   tile t, chunk s: k-tiles [s*ips, min(iters, (s+1)*ips)).
//   STREAMK  program p takes the contiguous k-iterations
//            [p*full + min(p, partial), (p+1)*full + min(p+1, partial)) of the
//            stream-K tiles, cut at tile boundaries, then whole "blocking"
//            tiles round-robin (TileLang tutorial "gemm_variants.py",
//            gemm_streamk / streamk_plan; tile ids past the count skipped).
//   GROUPED  persistent loop over the tiles of all experts, found from the
//            device offsets array (tutorial function gemm_grouped: padded
//            per-expert m-block prefix; rows past an expert's end masked).
// Split segments write fp32/int32 partial tiles to the partials workspace,
// publish them with an agent-scope release, and bump the tile's arrival
// counter by their k-iteration count. The segment that completes the count
// sums all segments of the tile in k order (so the result does not depend
// on arrival order), applies the epilogue and zeroes the counter. Nothing
// ever waits on another workgroup.
#pragma once
#include "qg_args.hpp"
#include "qg_device.hpp"

namespace qg {

enum class El { BF16, F16, I8, E4M3 };

template <El E_, int BM_, int BN_, int WM_, int WN_, int STAGES_>
struct TileCfg {
  static constexpr El E = E_;
  static constexpr int BM = BM_, BN = BN_, WAVES_M = WM_, WAVES_N = WN_, STAGES = STAGES_;
  static constexpr int NW = WM_ * WN_, NT = NW * 64;
  static constexpr int WTM = BM / WM_, WTN = BN / WN_;
  static constexpr int TM = WTM / 32, TN = WTN / 32;
  static constexpr int ESIZE = (E_ == El::BF16 || E_ == El::F16) ? 2 : 1;
  static constexpr int CH = (E_ == El::E4M3) ? 2 : 1;  // 16-byte chunks per lane per MFMA
  static constexpr int KSTEPS = 8 / (2 * CH);            // MFMAs along k per 128-byte k-tile
  static constexpr int BK = 128 / ESIZE;                 // elements per k-tile
  static constexpr int ROWB = 128;
  static constexpr int A_BYTES = BM * ROWB, B_BYTES = BN * ROWB;
  static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
  static constexpr int LA = BM / 8 / NW, LB = BN / 8 / NW;  // 64-lane loads per wave per stage
  static constexpr int LPW = LA + LB;
  static constexpr bool INT = (E_ == El::I8);
  static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be a multiple of 32");
  static_assert(LA * 8 * NW == BM && LB * 8 * NW == BN, "tile rows must split evenly over waves");
  static_assert(STAGES >= 2 && STAGES * STAGE_BYTES <= 160 * 1024 - 1024, "LDS budget");
  static_assert(LPW * (STAGES - 2) < 64, "vmcnt range");
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

struct Unit {
  int tile;         // counter / slot index
  int m0, n0;       // first row of A/D, first row of B (= first column of D)
  int m_end;        // rows [m0, m_end) valid
  int expert;
  int kb, ke;       // k-tile range [kb, ke)
};

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

__device__ __forceinline__ void epi_store4(const Args& a, int64_t m, int n, const f32x4& acc) {
  float v[4] = {a.alpha * acc[0], a.alpha * acc[1], a.alpha * acc[2], a.alpha * acc[3]};
  if (a.c_type >= 0 && a.beta != 0.f) {
    float c[4];
    load_c4(a, m, n, c);
    for (int j = 0; j < 4; ++j) v[j] = __builtin_fmaf(a.beta, c[j], v[j]);
  }
  store_d4(a, m, n, v);
}

// int8 path: D = acc (+ C when beta == 1), exact int32.
__device__ __forceinline__ void epi_store4(const Args& a, int64_t m, int n, const i32x4& acc) {
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

// ---- the kernel body -----------------------------------------------------
template <class Cfg>
struct Tile {
  using AO = AccOf<Cfg::INT>;
  using AccV = typename AO::V;
  using S4 = typename AO::S4;
  static constexpr int TN = Cfg::TN, TM = Cfg::TM;
  static constexpr int NQ = TN * TM * 4;  // 4-element groups per lane

  // Tile coordinates of a non-grouped tile id (super-grouped along M).
  __device__ __forceinline__ static void coords(const Args& a, int t, int& tm, int& tn) {
    const int per = a.group_m * a.tiles_n;
    const int g = t / per, first = g * a.group_m;
    const int gm = min(a.tiles_m - first, a.group_m);
    const int r = t - g * per;
    tm = first + r % gm;
    tn = r / gm;
  }

  __device__ __forceinline__ static Unit make_unit(const Args& a, int t, int kb, int ke) {
    int tm, tn;
    coords(a, t, tm, tn);
    Unit u;
    u.tile = t;
    u.m0 = tm * Cfg::BM;
    u.n0 = tn * Cfg::BN;
    u.m_end = a.M;
    u.expert = 0;
    u.kb = kb;
    u.ke = ke;
    return u;
  }

  __device__ __forceinline__ static void mainloop(const Args& a, const Unit& u, char* smem, AccV (&acc)[TN][TM]) {
    const int w = wave_id(), l = lane_id();
    const int wm = w / Cfg::WAVES_N, wn = w % Cfg::WAVES_N;
    const int64_t lda_b = a.lda * Cfg::ESIZE, ldb_b = a.ldb * Cfg::ESIZE;
    const uint32_t kbytes = (uint32_t)a.K * Cfg::ESIZE;
    const char* Ab = (const char*)a.A + (int64_t)u.m0 * lda_b;
    const char* Bb = (const char*)a.B + (int64_t)u.expert * a.b_batch * Cfg::ESIZE + (int64_t)u.n0 * ldb_b;
    const int a_rows = max(0, min(Cfg::BM, u.m_end - u.m0));
    const int b_rows = max(0, min(Cfg::BN, a.N - u.n0));
    const auto rA = make_rsrc(Ab, (uint32_t)(a_rows * lda_b));
    const auto rB = make_rsrc(Bb, (uint32_t)(b_rows * ldb_b));

    // this lane's row and logical chunk for each of its loads
    const int lrow = l >> 3, lchunk = (l & 7) ^ (l >> 3);
    uint32_t offA[Cfg::LA], offB[Cfg::LB];
#pragma unroll
    for (int i = 0; i < Cfg::LA; ++i) offA[i] = (uint32_t)(((w * Cfg::LA + i) * 8 + lrow) * lda_b) + lchunk * 16;
#pragma unroll
    for (int i = 0; i < Cfg::LB; ++i) offB[i] = (uint32_t)(((w * Cfg::LB + i) * 8 + lrow) * ldb_b) + lchunk * 16;

    auto issue = [&](int stage, int kt) {
      char* sbase = smem + stage * Cfg::STAGE_BYTES;
      const uint32_t koff = (uint32_t)kt * 128u + lchunk * 16;
      const bool kin = koff < kbytes;
      const uint32_t kk = (uint32_t)kt * 128u;
#pragma unroll
      for (int i = 0; i < Cfg::LA; ++i)
        load_lds_x4(rA, sbase + (w * Cfg::LA + i) * 8 * 128, kin ? offA[i] + kk : kOOB);
#pragma unroll
      for (int i = 0; i < Cfg::LB; ++i)
        load_lds_x4(rB, sbase + Cfg::A_BYTES + (w * Cfg::LB + i) * 8 * 128, kin ? offB[i] + kk : kOOB);
    };

    // per-lane LDS read addresses (row part) for the MFMA operands
    const int orow = l & 31, ohalf = l >> 5;

    auto compute = [&](int stage) {
      const char* sA = smem + stage * Cfg::STAGE_BYTES;
      const char* sB = sA + Cfg::A_BYTES;
#pragma unroll
      for (int ks = 0; ks < Cfg::KSTEPS; ++ks) {
        i32x4 af[TM][Cfg::CH], bfr[TN][Cfg::CH];
#pragma unroll
        for (int tm = 0; tm < TM; ++tm) {
          const int row = wm * Cfg::WTM + tm * 32 + orow;
#pragma unroll
          for (int c = 0; c < Cfg::CH; ++c) {
            const int lc = ks * 2 * Cfg::CH + ohalf * Cfg::CH + c;
            af[tm][c] = *(const i32x4*)(sA + row * 128 + ((lc ^ (row & 7)) << 4));
          }
        }
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) {
          const int row = wn * Cfg::WTN + tn * 32 + orow;
#pragma unroll
          for (int c = 0; c < Cfg::CH; ++c) {
            const int lc = ks * 2 * Cfg::CH + ohalf * Cfg::CH + c;
            bfr[tn][c] = *(const i32x4*)(sB + row * 128 + ((lc ^ (row & 7)) << 4));
          }
        }
#pragma unroll
        for (int tn = 0; tn < TN; ++tn)
#pragma unroll
          for (int tm = 0; tm < TM; ++tm) {
            if constexpr (Cfg::E == El::BF16)
              acc[tn][tm] = mfma_bf16(bfr[tn][0], af[tm][0], acc[tn][tm]);
            else if constexpr (Cfg::E == El::F16)
              acc[tn][tm] = mfma_f16(bfr[tn][0], af[tm][0], acc[tn][tm]);
            else if constexpr (Cfg::E == El::I8)
              acc[tn][tm] = mfma_i8(bfr[tn][0], af[tm][0], acc[tn][tm]);
          }
      }
    };

#pragma unroll
    for (int tn = 0; tn < TN; ++tn)
#pragma unroll
      for (int tm = 0; tm < TM; ++tm) acc[tn][tm] = AccV{};

    const int nk = u.ke - u.kb;
#pragma unroll
    for (int s = 0; s < Cfg::STAGES - 1; ++s)
      if (s < nk) issue(s, u.kb + s);
    for (int it = 0; it < nk; ++it) {
      if (it + Cfg::STAGES - 2 < nk)
        wait_vmcnt<Cfg::LPW * (Cfg::STAGES - 2)>();
      else
        wait_vmcnt<0>();
      __syncthreads();
      if (it + Cfg::STAGES - 1 < nk) issue((it + Cfg::STAGES - 1) % Cfg::STAGES, u.kb + it + Cfg::STAGES - 1);
      compute(it % Cfg::STAGES);
    }
    __syncthreads();  // the ring is reused by the next unit
  }

  // Final results of a tile: epilogue + masked store.
  __device__ __forceinline__ static void store(const Args& a, const Unit& u, AccV (&acc)[TN][TM]) {
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
          S4 v = {acc[tn][tm][4 * g], acc[tn][tm][4 * g + 1], acc[tn][tm][4 * g + 2], acc[tn][tm][4 * g + 3]};
          epi_store4(a, m, n, v);
        }
    }
  }

  __device__ __forceinline__ static S4* slot_ptr(const Args& a, int slot) {
    return (S4*)((char*)a.partials + (size_t)slot * (Cfg::BM * Cfg::BN * 4));
  }

  __device__ __forceinline__ static void write_partial(const Args& a, int slot, AccV (&acc)[TN][TM]) {
    S4* p = slot_ptr(a, slot) + (size_t)wave_id() * NQ * 64 + lane_id();
#pragma unroll
    for (int tn = 0; tn < TN; ++tn)
#pragma unroll
      for (int tm = 0; tm < TM; ++tm)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int q = (tn * TM + tm) * 4 + g;
          p[q * 64] = S4{acc[tn][tm][4 * g], acc[tn][tm][4 * g + 1], acc[tn][tm][4 * g + 2], acc[tn][tm][4 * g + 3]};
        }
  }

  // tot = (...((seg_0 + seg_1) + seg_2) ...) in k order, read back from the workspace.
  __device__ __forceinline__ static void add_partial(const Args& a, int slot, AccV (&tot)[TN][TM], bool first) {
    const S4* p = slot_ptr(a, slot) + (size_t)wave_id() * NQ * 64 + lane_id();
#pragma unroll
    for (int tn = 0; tn < TN; ++tn)
#pragma unroll
      for (int tm = 0; tm < TM; ++tm)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int q = (tn * TM + tm) * 4 + g;
          S4 x = __builtin_nontemporal_load(p + q * 64);
#pragma unroll
          for (int j = 0; j < 4; ++j) tot[tn][tm][4 * g + j] = first ? x[j] : tot[tn][tm][4 * g + j] + x[j];
        }
  }

  // Publishes a partial segment; returns true in the workgroup that completed the tile.
  __device__ __forceinline__ static bool arrive(const Args& a, const Unit& u, int slot, AccV (&acc)[TN][TM], int* flag) {
    write_partial(a, slot, acc);
    __threadfence();  // agent-scope release of the partial tile (crosses XCD L2s)
    __syncthreads();
    if (threadIdx.x == 0) {
      const int nk = u.ke - u.kb;
      const int old = __hip_atomic_fetch_add(a.counters + u.tile, nk, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
      *flag = (old + nk == a.iters);
    }
    __syncthreads();
    const bool last = *flag;
    if (last) __threadfence();  // acquire side: see every other segment's partial
    return last;
  }

  __device__ __forceinline__ static void finish_counter(const Args& a, const Unit& u) {
    if (threadIdx.x == 0) __hip_atomic_store(a.counters + u.tile, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  // ---- schedules ------------------------------------------------------------
  __device__ __forceinline__ static int xcd_remap(int b, int G) {
    // blocks are dealt to the 8 XCDs round-robin; give each XCD a contiguous range of ids
    const int x = b & 7, q = G >> 3, r = G & 7;
    return x * q + min(x, r) + (b >> 3);
  }

  __device__ __forceinline__ static void run_dp(const Args& a, char* smem) {
    const int total = a.tiles_m * a.tiles_n;
    for (int b = blockIdx.x; b < total; b += gridDim.x) {
      const int t = (gridDim.x == (unsigned)total) ? xcd_remap(b, total) : b;
      AccV acc[TN][TM];
      Unit u = make_unit(a, t, 0, a.iters);
      mainloop(a, u, smem, acc);
      store(a, u, acc);
    }
  }

  __device__ __forceinline__ static void run_splitk(const Args& a, char* smem, int* flag) {
    const int total = a.tiles_m * a.tiles_n * a.splits;
    for (int b = blockIdx.x; b < total; b += gridDim.x) {
      const int t = b / a.splits, s = b % a.splits;
      const int kb = s * a.iters_per_split, ke = min(a.iters, kb + a.iters_per_split);
      AccV acc[TN][TM];
      Unit u = make_unit(a, t, kb, ke);
      mainloop(a, u, smem, acc);
      if (arrive(a, u, t * a.splits + s, acc, flag)) {
        const int ns = (a.iters + a.iters_per_split - 1) / a.iters_per_split;
        for (int q = 0; q < ns; ++q) add_partial(a, t * a.splits + q, acc, q == 0);
        store(a, u, acc);
        finish_counter(a, u);
      }
    }
  }

  __device__ __forceinline__ static int sk_start(const Args& a, int p) { return p * a.sk_full + min(p, a.sk_partial); }
  __device__ __forceinline__ static int sk_owner(const Args& a, int it) {
    const int big = a.sk_partial * (a.sk_full + 1);
    return it < big ? it / (a.sk_full + 1) : a.sk_partial + (it - big) / a.sk_full;
  }

  __device__ __forceinline__ static void run_streamk(const Args& a, char* smem, int* flag) {
    const int ipt = a.iters;
    for (int pid = blockIdx.x; pid < a.programs; pid += gridDim.x) {
      int it = sk_start(a, pid);
      const int last = sk_start(a, pid + 1);
      const int first_it = it;
      while (it < last) {
        const int t = it / ipt, rem = it - t * ipt;
        const int end = min(it + (ipt - rem), last);
        AccV acc[TN][TM];
        Unit u = make_unit(a, t, rem, rem + (end - it));
        mainloop(a, u, smem, acc);
        if (rem == 0 && end - it == ipt) {
          store(a, u, acc);
        } else {
          const int slot = 2 * pid + (it == first_it ? 0 : 1);
          if (arrive(a, u, slot, acc, flag)) {
            const int t0 = t * ipt;
            const int plo = sk_owner(a, t0), phi = sk_owner(a, t0 + ipt - 1);
            for (int q = plo; q <= phi; ++q) add_partial(a, 2 * q + (sk_start(a, q) >= t0 ? 0 : 1), acc, q == plo);
            store(a, u, acc);
            finish_counter(a, u);
          }
        }
        it = end;
      }
      const int total = a.tiles_m * a.tiles_n;
      for (int r = 0; r < a.dp_rounds; ++r) {
        const int t = pid + a.sk_tiles + r * a.programs;
        if (t >= total) break;
        AccV acc[TN][TM];
        Unit u = make_unit(a, t, 0, ipt);
        mainloop(a, u, smem, acc);
        store(a, u, acc);
      }
    }
  }

  // Grouped: per-expert m-tile prefix built in LDS from the device offsets.
  __device__ __forceinline__ static void run_grouped(const Args& a, char* smem, int* pref) {
    // pref[0..E] = prefix of ceil(rows_e / BM); E <= 1023 (host checked)
    if (threadIdx.x == 0) {
      int acc = 0;
      pref[0] = 0;
      for (int e = 0; e < a.E; ++e) {
        const int rows = a.offsets[e + 1] - a.offsets[e];
        acc += rows > 0 ? (rows + Cfg::BM - 1) / Cfg::BM : 0;
        pref[e + 1] = acc;
      }
    }
    __syncthreads();
    const int total = pref[a.E] * a.tiles_n;
    for (int b = blockIdx.x; b < total; b += gridDim.x) {
      const int mt = b / a.tiles_n, tn = b - mt * a.tiles_n;
      int lo = 0, hi = a.E - 1;  // largest e with pref[e] <= mt
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (pref[mid] <= mt)
          lo = mid;
        else
          hi = mid - 1;
      }
      Unit u;
      u.expert = lo;
      u.tile = b;
      u.m0 = a.offsets[lo] + (mt - pref[lo]) * Cfg::BM;
      u.m_end = a.offsets[lo + 1];
      u.n0 = tn * Cfg::BN;
      u.kb = 0;
      u.ke = a.iters;
      AccV acc[TN][TM];
      mainloop(a, u, smem, acc);
      store(a, u, acc);
    }
  }
};

template <class Cfg, int MODE>
__global__ __launch_bounds__(Cfg::NT) void tile_kernel(const Args a) {
  __shared__ __attribute__((aligned(1024))) char smem[Cfg::STAGES * Cfg::STAGE_BYTES];
  __shared__ int misc[MODE == MODE_GROUPED ? 1025 : 1];
  if constexpr (MODE == MODE_DP) Tile<Cfg>::run_dp(a, smem);
  if constexpr (MODE == MODE_SPLITK) Tile<Cfg>::run_splitk(a, smem, misc);
  if constexpr (MODE == MODE_STREAMK) Tile<Cfg>::run_streamk(a, smem, misc);
  if constexpr (MODE == MODE_GROUPED) Tile<Cfg>::run_grouped(a, smem, misc);
}

}  // namespace qg

namespace qg {

// Host-side launcher of one registered tile kernel; one instantiation per schedule.
template <class Cfg>
hipError_t launch_tile(const Args& a, int grid, hipStream_t s) {
  switch (a.mode) {
    case MODE_DP: hipLaunchKernelGGL((tile_kernel<Cfg, MODE_DP>), dim3(grid), dim3(Cfg::NT), 0, s, a); break;
    case MODE_SPLITK: hipLaunchKernelGGL((tile_kernel<Cfg, MODE_SPLITK>), dim3(grid), dim3(Cfg::NT), 0, s, a); break;
    case MODE_STREAMK: hipLaunchKernelGGL((tile_kernel<Cfg, MODE_STREAMK>), dim3(grid), dim3(Cfg::NT), 0, s, a); break;
    case MODE_GROUPED: hipLaunchKernelGGL((tile_kernel<Cfg, MODE_GROUPED>), dim3(grid), dim3(Cfg::NT), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace qg
