// Skinny-M (decode-shaped) GEMM core for gfx950: M <= 16 * MT.
//
// The DeepGEMM write-up (section 5.1) notes that the M=1 shape is load-bound
// and needs its own kernel. Here every wave streams its own k-blocks of B
// (BN rows) and A (BM rows) -- 256 contiguous bytes per row per block -- from
// HBM into a private DEPTH-deep LDS ring with buffer_load ... lds, so a wave
// only ever waits for its own loads (vmcnt) and never for the other waves.
// The waves of a workgroup cover the same BN columns and take interleaved
// k-blocks; their accumulators are summed through LDS in wave order at the
// end, so the result is deterministic. Rows are stored with chunk' = chunk ^
// (row & 15) over their 16 chunks of 16 bytes, so the 16 rows an MFMA operand
// read touches hit 16 different bank groups. Work division (DP / split-K /
// stream-K) is the shared one in qg_sched.hpp.
//
// MFMA 16x16 (bf16/fp16 16x16x32, int8 16x16x64): lane l supplies row l % 16
// and the 16-byte k-slice l / 16 of each operand; output element r of lane l
// is row 4*(l/16) + r, column l % 16. B rows are the MFMA's first operand and
// A rows its second, so a lane ends up holding 4 consecutive columns n of one
// row m of D (one vector store).
#pragma once
#include "qg_tile.hpp"

namespace qg {

// MODE_ 0: the waves share the workgroup's BN columns and interleave k-blocks
// (summed through LDS at the end); 1: each wave owns BN / NW columns over the
// whole k-range (no cross-wave sum); 2: as 1, but the A rows of a k-block are
// loaded once per workgroup into a shared ring instead of once per wave (the
// waves then meet at a barrier per block; a probe of the decode shape showed
// the per-wave A reloads costing about 2.5 us of streaming time).
template <El E_, int BN_, int NW_, int MT_, int DEPTH_, int BLKB_ = 256, int MODE_ = 0>
struct SkinnyCfg {
  static constexpr El E = E_;
  static constexpr bool NSPLIT = MODE_ >= 1, SHARED_A = MODE_ == 2;
  static constexpr int BN = BN_, NW = NW_, MT = MT_, DEPTH = DEPTH_;
  static constexpr int BNW = NSPLIT ? BN / NW : BN;  // columns per wave
  static constexpr int NT = NW * 64, BM = 16 * MT, TN = BNW / 16;
  static constexpr int ESIZE = (E_ == El::BF16 || E_ == El::F16) ? 2 : 1;
  static constexpr int BLKB = BLKB_;              // bytes of k per row per block (256, 512 or 1024)
  static constexpr int CPR = BLKB / 16;           // 16-byte chunks per row
  static constexpr int RPI = 64 / CPR;            // rows filled by one 64-lane load
  static constexpr int STEPS = BLKB / 64;         // MFMA k-steps per block
  static constexpr int BK = BLKB / ESIZE;         // k elements per block
  // LDS bytes of one wave's ring slot (B rows, plus its own A rows unless shared)
  static constexpr int SLOT = (BNW + (SHARED_A ? 0 : BM)) * BLKB;
  static constexpr int ASLOT = SHARED_A ? BM * BLKB : 0;  // one slot of the shared A ring
  static constexpr int LA_SH = BM / RPI;                  // 64-lane loads of one shared A block
  // 64-lane loads per slot and wave (shared A: one A load per wave, waves
  // w and w + LA_SH repeating the same one)
  static constexpr int LPS = SHARED_A ? BNW / RPI + 1 : (BNW + BM) / RPI;
  static constexpr int LDS_BYTES = NW * DEPTH * SLOT + DEPTH * ASLOT;
  static_assert(BLKB == 256 || BLKB == 512 || BLKB == 1024, "block bytes");
  static_assert(LDS_BYTES <= 160 * 1024 - 4096, "LDS budget");
  static_assert(LPS * (DEPTH - 1) < 64, "vmcnt range");
  static_assert(!SHARED_A || (DEPTH >= 2 && LA_SH <= NW), "shared A ring");
  static constexpr bool INT = (E_ == El::I8);
  static_assert(BNW % 16 == 0 && BNW * (NSPLIT ? NW : 1) == BN && DEPTH >= 1, "skinny tile");
};

__device__ __forceinline__ f32x4 mfma16_bf16(i32x4 a, i32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16_f16(i32x4 a, i32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ i32x4 mfma16_i8(i32x4 a, i32x4 b, i32x4 c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

template <class Cfg>
struct Skinny {
  using S4 = typename AccOf<Cfg::INT>::S4;
  static constexpr int TN = Cfg::TN, MT = Cfg::MT, NW = Cfg::NW, DEPTH = Cfg::DEPTH;
  static constexpr int BM = Cfg::BM, BN = Cfg::BN, NT = Cfg::NT, BNW = Cfg::BNW;
  static constexpr int SMEM_BYTES = Cfg::LDS_BYTES;  // per-wave rings (+ shared A ring; reused for the reduction)
  static_assert(NW * TN * MT * 64 * 16 <= SMEM_BYTES, "reduction space");
  // v: accumulators; c: this lane's C values, loaded when the unit starts so
  // that the epilogue does not wait for them at the end of the stream
  struct Acc {
    S4 v[TN][MT];
    f32x4 c[TN][MT];
  };

  __device__ __forceinline__ static bool stores(int w) { return Cfg::NSPLIT || w == 0; }

  __device__ __forceinline__ static void prefetch_c(const Args& a, const Unit& u, Acc& acc) {
    if constexpr (!Cfg::INT) {
      const int w = wave_id(), l = lane_id();
      const bool need = a.c_type >= 0 && a.beta != 0.f && stores(w);
      const int nw0 = Cfg::NSPLIT ? w * BNW : 0;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) {
          const int m = u.m0 + mt * 16 + (l & 15);
          const int n = u.n0 + nw0 + tn * 16 + 4 * (l >> 4);
          float c[4] = {0.f, 0.f, 0.f, 0.f};
          if (need && m < u.m_end && n < a.N) load_c4(a, m, n, c);
          acc.c[tn][mt] = f32x4{c[0], c[1], c[2], c[3]};
        }
    }
  }

  __device__ __forceinline__ static S4 mma(i32x4 b, i32x4 a, S4 c) {
    if constexpr (Cfg::E == El::BF16) return mfma16_bf16(b, a, c);
    else if constexpr (Cfg::E == El::F16) return mfma16_f16(b, a, c);
    else return mfma16_i8(b, a, c);
  }

  __device__ __forceinline__ static void mainloop(const Args& a, const Unit& u, char* smem, Acc& acc) {
    if constexpr (Cfg::SHARED_A) {
      mainloop_shared_a(a, u, smem, acc);
      return;
    }
    const int w = wave_id(), l = lane_id();
    constexpr int ES = Cfg::ESIZE;
    const int64_t lda_b = a.lda * ES, ldb_b = a.ldb * ES;
    const uint32_t kbytes = (uint32_t)a.K * ES;
    const int a_rows = max(0, min(BM, u.m_end - u.m0));
    const int b_rows = max(0, min(BN, a.N - u.n0));
    const i32x4 rA = make_rsrc_words((const char*)a.A + (int64_t)u.m0 * lda_b, (uint32_t)(a_rows * lda_b));
    // N-split: this wave's rows of B start BNW * w rows into the tile
    const int nw0 = Cfg::NSPLIT ? w * BNW : 0;
    const int b_rows_w = max(0, min(BNW, b_rows - nw0));
    const i32x4 rB = make_rsrc_words(
        (const char*)a.B + (int64_t)u.expert * a.b_batch * ES + (int64_t)(u.n0 + nw0) * ldb_b,
        (uint32_t)((Cfg::NSPLIT ? b_rows_w : b_rows) * ldb_b));
    // One 64-lane load fills RPI rows x BLKB bytes of a slot: lane l -> row
    // l / CPR, physical chunk l % CPR, which holds logical chunk
    // (l % CPR) ^ (row & 15).
    constexpr int CPR = Cfg::CPR, RPI = Cfg::RPI;
    char* ring = smem + w * DEPTH * Cfg::SLOT;
    const int lrow = l / CPR;
    constexpr int LB = BNW / RPI, LA = BM / RPI;
    uint32_t offB[LB], offA[LA], chB[LB], chA[LA];
#pragma unroll
    for (int i = 0; i < LB; ++i) {
      const int row = i * RPI + lrow;
      chB[i] = (uint32_t)(((l % CPR) ^ (row & 15)) * 16);
      offB[i] = (uint32_t)(row * ldb_b) + chB[i];
    }
#pragma unroll
    for (int i = 0; i < LA; ++i) {
      const int row = i * RPI + lrow;
      chA[i] = (uint32_t)(((l % CPR) ^ (row & 15)) * 16);
      offA[i] = (uint32_t)(row * lda_b) + chA[i];
    }
    // Loads k-block blk into ring slot d; blocks past the unit read nothing.
    auto issue = [&](int d, int blk) {
      char* base = ring + d * Cfg::SLOT;
      const bool live = blk < u.ke;
      const uint32_t kk = (uint32_t)blk * Cfg::BLKB;
#pragma unroll
      for (int i = 0; i < LB; ++i)
        load_lds_x4(rB, base + i * 1024, live && kk + chB[i] < kbytes ? offB[i] + kk : kOOB);
#pragma unroll
      for (int i = 0; i < LA; ++i)
        load_lds_x4(rA, base + BNW * Cfg::BLKB + i * 1024, live && kk + chA[i] < kbytes ? offA[i] + kk : kOOB);
    };
    // K * ESIZE not a multiple of 16: in the block that holds K's end, zero
    // the bytes past K in the chunks this lane loaded (its own loads have
    // landed; the wave's LDS accesses stay in order, so its reads see this).
    const int ktail = (kbytes & 15) ? (int)((kbytes - 1) / Cfg::BLKB) : -1;
    auto trim = [&](int d, int blk) {
      const uint32_t kb = pinned(kbytes);  // keeps this work inside the branch
      char* base = ring + d * Cfg::SLOT;
      const uint32_t kk = (uint32_t)blk * Cfg::BLKB;
#pragma unroll
      for (int i = 0; i < LB; ++i) {
        const int keep = (int)(kb - kk - chB[i]);
        if (keep > 0 && keep < 16) lds_chunk_trim(base + i * 1024 + l * 16, keep);
      }
#pragma unroll
      for (int i = 0; i < LA; ++i) {
        const int keep = (int)(kb - kk - chA[i]);
        if (keep > 0 && keep < 16) lds_chunk_trim(base + BNW * Cfg::BLKB + i * 1024 + l * 16, keep);
      }
    };
    // Operand fragments of the block in slot d: step j covers bytes
    // [64j, 64j+64) of each row; lane l reads row l%16 of each 16-row group at
    // logical chunk 4j + l/16.
    constexpr int ST = Cfg::STEPS;
    i32x4 fb[ST][TN], fa[ST][MT];
    auto read = [&](int d) {
      const char* base = ring + d * Cfg::SLOT;
#pragma unroll
      for (int j = 0; j < ST; ++j) {
        const int c = 4 * j + (l >> 4);
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) {
          const int row = tn * 16 + (l & 15);
          fb[j][tn] = *(const i32x4*)(base + row * Cfg::BLKB + ((c ^ (row & 15)) << 4));
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const int row = mt * 16 + (l & 15);
          fa[j][mt] = *(const i32x4*)(base + BNW * Cfg::BLKB + row * Cfg::BLKB + ((c ^ (row & 15)) << 4));
        }
      }
    };
    auto compute = [&]() {
#pragma unroll
      for (int j = 0; j < ST; ++j)
#pragma unroll
        for (int tn = 0; tn < TN; ++tn)
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) acc.v[tn][mt] = mma(fb[j][tn], fa[j][mt], acc.v[tn][mt]);
    };

#pragma unroll
    for (int tn = 0; tn < TN; ++tn)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc.v[tn][mt] = S4{};
    prefetch_c(a, u, acc);

    const int nk = u.ke - u.kb;
    // This wave's blocks are kb + w, kb + w + NW, ...; the count is rounded up
    // to a multiple of DEPTH (the extra blocks read nothing and add zeros) so
    // exactly DEPTH - 1 blocks are in flight behind the one being consumed.
    // k-interleaved: block i of this wave is kb + w + i * NW; N-split: kb + i.
    constexpr int KSTRIDE = Cfg::NSPLIT ? 1 : NW;
    const int kfirst = Cfg::NSPLIT ? 0 : w;
    const int count = nk > kfirst ? (nk - kfirst + KSTRIDE - 1) / KSTRIDE : 0;
    const int rounds = (count + DEPTH - 1) / DEPTH;
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) issue(d, u.kb + kfirst + d * KSTRIDE);
    for (int r = 0; r < rounds; ++r) {
#pragma unroll
      for (int d = 0; d < DEPTH; ++d) {
        wait_vmcnt<Cfg::LPS * (DEPTH - 1)>();
        asm volatile("" ::: "memory");
        {
          const int blk = u.kb + kfirst + (r * DEPTH + d) * KSTRIDE;
          if (blk == ktail) trim(d, blk);
        }
        read(d);
        // refill the slot as soon as its fragments are in registers
        __builtin_amdgcn_s_waitcnt(0xc07f);
        asm volatile("" ::: "memory");
        issue(d, u.kb + kfirst + ((r + 1) * DEPTH + d) * KSTRIDE);
        compute();
      }
    }
    wait_vmcnt<0>();
    __syncthreads();  // every wave is done with its ring before it is reused below
    if constexpr (Cfg::NSPLIT) return;  // each wave already holds its own columns

    // Sum the waves' partial sums in wave order into wave 0.
    S4* red = (S4*)smem;
    if (w > 0) {
#pragma unroll
      for (int tn = 0; tn < TN; ++tn)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) red[((w * TN + tn) * MT + mt) * 64 + l] = acc.v[tn][mt];
    }
    __syncthreads();
    if (w == 0) {
      for (int w2 = 1; w2 < NW; ++w2)
#pragma unroll
        for (int tn = 0; tn < TN; ++tn)
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) acc.v[tn][mt] += red[((w2 * TN + tn) * MT + mt) * 64 + l];
    }
    __syncthreads();
  }

  // N-split with a shared A ring: wave w keeps a private DEPTH-slot ring of
  // its B rows; the A rows of each block go to a workgroup ring (load i of
  // the LA_SH 1 KB loads of a block is issued by waves i, i + LA_SH, ...:
  // the repeats write the same bytes to the same place and keep every
  // wave's load count, and so vmcnt, uniform). Per block: wait for this
  // wave's loads of block b, meet (so every wave's part of A(b) has landed
  // and every wave is done reading block b - 1), refill block b - 1's slots
  // with block b + DEPTH - 1, read block b, compute. DEPTH - 1 blocks stay
  // in flight behind the one being consumed; the summation order per
  // output is that of MODE 1, so results are identical.
  __device__ __forceinline__ static void mainloop_shared_a(const Args& a, const Unit& u, char* smem, Acc& acc) {
    const int w = wave_id(), l = lane_id();
    constexpr int ES = Cfg::ESIZE, CPR = Cfg::CPR, RPI = Cfg::RPI, LB = BNW / RPI, ST = Cfg::STEPS;
    const int64_t lda_b = a.lda * ES, ldb_b = a.ldb * ES;
    const uint32_t kbytes = (uint32_t)a.K * ES;
    const int a_rows = max(0, min(BM, u.m_end - u.m0));
    const int b_rows = max(0, min(BN, a.N - u.n0));
    const i32x4 rA = make_rsrc_words((const char*)a.A + (int64_t)u.m0 * lda_b, (uint32_t)(a_rows * lda_b));
    const int nw0 = w * BNW;
    const int b_rows_w = max(0, min(BNW, b_rows - nw0));
    const i32x4 rB = make_rsrc_words((const char*)a.B + (int64_t)u.expert * a.b_batch * ES + (int64_t)(u.n0 + nw0) * ldb_b,
                                     (uint32_t)(b_rows_w * ldb_b));
    char* bring = smem + w * DEPTH * Cfg::SLOT;
    char* aring = smem + NW * DEPTH * Cfg::SLOT;
    const int lrow = l / CPR;
    uint32_t offB[LB], chB[LB];
#pragma unroll
    for (int i = 0; i < LB; ++i) {
      const int row = i * RPI + lrow;
      chB[i] = (uint32_t)(((l % CPR) ^ (row & 15)) * 16);
      offB[i] = (uint32_t)(row * ldb_b) + chB[i];
    }
    const int ia = w % Cfg::LA_SH;
    const int arow = ia * RPI + lrow;
    const uint32_t chA = (uint32_t)(((l % CPR) ^ (arow & 15)) * 16);
    const uint32_t offA = (uint32_t)(arow * lda_b) + chA;
    auto issue = [&](int d, int blk) {
      char* base = bring + d * Cfg::SLOT;
      const bool live = blk < u.ke;
      const uint32_t kk = (uint32_t)blk * Cfg::BLKB;
#pragma unroll
      for (int i = 0; i < LB; ++i) load_lds_x4(rB, base + i * 1024, live && kk + chB[i] < kbytes ? offB[i] + kk : kOOB);
      load_lds_x4(rA, aring + d * Cfg::ASLOT + ia * 1024, live && kk + chA < kbytes ? offA + kk : kOOB);
    };
    // K * ESIZE not a multiple of 16: zero the bytes past K in the chunks
    // this lane loaded for the block that holds K's end, before the barrier
    // that publishes the block. Waves that load the same A chunk each trim it
    // after their own copy has landed, so the last write is a trimmed one.
    const int ktail = (kbytes & 15) ? (int)((kbytes - 1) / Cfg::BLKB) : -1;
    auto trim = [&](int d, int blk) {
      const uint32_t kb = pinned(kbytes);  // keeps this work inside the branch
      char* base = bring + d * Cfg::SLOT;
      const uint32_t kk = (uint32_t)blk * Cfg::BLKB;
#pragma unroll
      for (int i = 0; i < LB; ++i) {
        const int keep = (int)(kb - kk - chB[i]);
        if (keep > 0 && keep < 16) lds_chunk_trim(base + i * 1024 + l * 16, keep);
      }
      const int keep = (int)(kb - kk - chA);
      if (keep > 0 && keep < 16) lds_chunk_trim(aring + d * Cfg::ASLOT + ia * 1024 + l * 16, keep);
    };
    i32x4 fb[ST][TN], fa[ST][MT];
    auto read = [&](int d) {
      const char* bb = bring + d * Cfg::SLOT;
      const char* ab = aring + d * Cfg::ASLOT;
#pragma unroll
      for (int j = 0; j < ST; ++j) {
        const int c = 4 * j + (l >> 4);
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) {
          const int row = tn * 16 + (l & 15);
          fb[j][tn] = *(const i32x4*)(bb + row * Cfg::BLKB + ((c ^ (row & 15)) << 4));
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const int row = mt * 16 + (l & 15);
          fa[j][mt] = *(const i32x4*)(ab + row * Cfg::BLKB + ((c ^ (row & 15)) << 4));
        }
      }
    };
#pragma unroll
    for (int tn = 0; tn < TN; ++tn)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc.v[tn][mt] = S4{};
    prefetch_c(a, u, acc);
    const int nk = u.ke - u.kb;
    // rounded up to whole rounds of DEPTH blocks: blocks past the unit read
    // nothing (zeros) and add nothing
    const int rounds = (nk + DEPTH - 1) / DEPTH;
#pragma unroll
    for (int d = 0; d < DEPTH - 1; ++d) issue(d, u.kb + d);
    for (int r = 0; r < rounds; ++r) {
#pragma unroll
      for (int d = 0; d < DEPTH; ++d) {
        wait_vmcnt<Cfg::LPS * (DEPTH - 2)>();
        if (u.kb + r * DEPTH + d == ktail) trim(d, ktail);
        lds_barrier();
        issue((d + DEPTH - 1) % DEPTH, u.kb + r * DEPTH + d + DEPTH - 1);
        read(d);
#pragma unroll
        for (int j = 0; j < ST; ++j)
#pragma unroll
          for (int tn = 0; tn < TN; ++tn)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) acc.v[tn][mt] = mma(fb[j][tn], fa[j][mt], acc.v[tn][mt]);
      }
    }
    wait_vmcnt<0>();
    __syncthreads();  // the rings are reused by the next unit
  }

  // Epilogue: wave 0 holds the tile (k-interleaved) or each wave its columns (N-split).
  __device__ __forceinline__ static void store(const Args& a, const Unit& u, Acc& acc, char* /*smem*/) {
    if (!Cfg::NSPLIT && wave_id() != 0) return;
    const int l = lane_id();
    const int nw0 = Cfg::NSPLIT ? wave_id() * BNW : 0;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int m = u.m0 + mt * 16 + (l & 15);
      if (m >= u.m_end) continue;
#pragma unroll
      for (int tn = 0; tn < TN; ++tn) {
        const int n = u.n0 + nw0 + tn * 16 + 4 * (l >> 4);
        if (n >= a.N) continue;
        if constexpr (Cfg::INT)
          epi_store4(a, m, n, acc.v[tn][mt]);
        else
          epi_store4c(a, m, n, acc.v[tn][mt], acc.c[tn][mt]);
      }
    }
  }

  __device__ __forceinline__ static __amdgpu_buffer_rsrc_t slot_rsrc(const Args& a, int slot) {
    return make_rsrc((const char*)a.partials + (size_t)slot * (BM * BN * 4), BM * BN * 4);
  }
  // Partial tile layout: [wave (N-split) ][tn][mt][lane] x 16 bytes.
  __device__ __forceinline__ static uint32_t pofs(int tn, int mt) {
    const int w = Cfg::NSPLIT ? wave_id() : 0;
    return (uint32_t)((((w * TN + tn) * MT + mt) * 64 + lane_id()) * 16);
  }
  __device__ __forceinline__ static void write_partial(const Args& a, int slot, Acc& acc) {
    if (!Cfg::NSPLIT && wave_id() != 0) return;
    const auto r = slot_rsrc(a, slot);
#pragma unroll
    for (int tn = 0; tn < TN; ++tn)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) store_sc1_x4(r, pofs(tn, mt), __builtin_bit_cast(i32x4, acc.v[tn][mt]));
  }
  // Chunk c = tn * MT + mt of a lane's partial tile.
  static constexpr int NCH = TN * MT;
  __device__ __forceinline__ static bool holds_partial() { return Cfg::NSPLIT || wave_id() == 0; }
  __device__ __forceinline__ static uint32_t chunk_off(int c) { return pofs(c / MT, c % MT); }
  __device__ __forceinline__ static S4 get4(const Acc& acc, int c) { return acc.v[c / MT][c % MT]; }
  __device__ __forceinline__ static void set4(Acc& acc, int c, const S4& x) { acc.v[c / MT][c % MT] = x; }
};

template <class Cfg>
hipError_t launch_skinny(const Args& a, int grid, hipStream_t s) {
  return launch_sched<Skinny<Cfg>>(a, grid, s);
}

}  // namespace qg
