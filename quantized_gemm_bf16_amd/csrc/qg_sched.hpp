// Work division shared by every kernel core (DP, split-K, stream-K, grouped).
//
// A core supplies: BM, BN (output tile), NT (threads), SMEM_BYTES, an Acc
// type holding one tile's accumulators, mainloop(a, unit, smem, acc) over the
// unit's k-tiles, store(a, unit, acc) (epilogue), write_partial on the
// partials workspace and, for reading partial tiles back, the lane's NCH
// 16-byte chunks (chunk_off, get4 / set4, holds_partial).
//
//   DP       one unit = one whole tile; with one workgroup per tile the block
//            id is remapped so each XCD (own L2) gets a contiguous range.
//   SPLITK   tile t, chunk s: k-tiles [s*ips, min(iters, (s+1)*ips)).
//   STREAMK  program p takes its whole tiles round-robin, then a balanced
//            contiguous range of the remaining tiles' k-iterations, cut at
//            tile boundaries (qg_streamk.hpp).
//   GROUPED  persistent loop over the tiles of all experts, found from the
//            device offsets array (tutorial function gemm_grouped: padded
//            per-expert m-block prefix; rows past an expert's end masked).
//            Without an offsets array the groups are E batches of M rows each
//            (tutorial function gemm_batched: the (batch, m-block, n-block)
//            triple flattened into one tile id).
// Split segments write fp32/int32 partial tiles to the partials workspace and
// bump the tile's arrival counter by their k-iteration count. The segment
// that completes the count sums all segments of the tile in k order (so the
// result does not depend on arrival order), applies the epilogue and zeroes
// the counter. Nothing ever waits on another workgroup.
#pragma once
#include "qg_args.hpp"
#include "qg_device.hpp"
#include "qg_streamk.hpp"

namespace qg {

struct Unit {
  int tile;         // counter / slot index
  int m0, n0;       // first row of A/D, first row of B (= first column of D)
  int m_end;        // rows [m0, m_end) valid
  int expert;
  int kb, ke;       // k-tile range [kb, ke)
};

template <class Core>
struct Sched {
  using Acc = typename Core::Acc;

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
    u.m0 = tm * Core::BM;
    u.n0 = tn * Core::BN;
    u.m_end = a.M;
    u.expert = 0;
    u.kb = kb;
    u.ke = ke;
    return u;
  }

  // Publishes a partial segment; returns true in the workgroup that completed
  // the tile. Order: every lane's sc1 stores are acknowledged (vmcnt 0) before
  // the workgroup barrier, the counter is bumped only after the barrier, and
  // the completing workgroup reads partials only after the counter returned.
  __device__ __forceinline__ static bool arrive(const Args& a, const Unit& u, int slot, Acc& acc, int* flag) {
    Core::write_partial(a, slot, acc);
    wait_vmcnt<0>();
    __syncthreads();
    if (threadIdx.x == 0) {
      const int nk = u.ke - u.kb;
      const int old = __hip_atomic_fetch_add(a.counters + u.tile, nk, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      *flag = (old + nk == a.iters);
    }
    __syncthreads();
    return *flag;
  }

  // tot = (...((seg_0 + seg_1) + seg_2) ...) over the ns segments of a tile,
  // in k order, read back from the workspace (slot_of(i) = slot of segment
  // i). Small partial tiles (NCH < 32 chunks per lane) issue the loads of RB
  // segments together (at most 32 16-byte loads per lane) before summing any
  // of them, so they do not pay one memory round trip per segment; the empty
  // asm ends a round so that the compiler does not hoist the next round's
  // loads (which would spill). Large tiles go segment by segment.
  template <class SlotOf>
  __device__ __forceinline__ static void reduce(const Args& a, int ns, SlotOf slot_of, Acc& tot) {
    if (!Core::holds_partial()) return;
    using S4 = decltype(Core::get4(tot, 0));
    constexpr int NCH = Core::NCH;
    if constexpr (NCH >= 32) {
      for (int q = 0; q < ns; ++q) {
        const auto r = Core::slot_rsrc(a, slot_of(q));
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
          const S4 x = __builtin_bit_cast(S4, load_sc1_x4(r, Core::chunk_off(c)));
          Core::set4(tot, c, q == 0 ? x : Core::get4(tot, c) + x);
        }
      }
    } else {
      constexpr int RB = 32 / NCH > 8 ? 8 : 32 / NCH;
      for (int q0 = 0; q0 < ns; q0 += RB) {
        S4 x[RB][NCH];
#pragma unroll
        for (int j = 0; j < RB; ++j) {
          const auto r = Core::slot_rsrc(a, slot_of(min(q0 + j, ns - 1)));
#pragma unroll
          for (int c = 0; c < NCH; ++c) x[j][c] = __builtin_bit_cast(S4, load_sc1_x4(r, Core::chunk_off(c)));
        }
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
          S4 t = Core::get4(tot, c);
#pragma unroll
          for (int j = 0; j < RB; ++j)
            if (q0 + j < ns) t = (q0 + j == 0) ? x[j][c] : t + x[j][c];
          Core::set4(tot, c, t);
        }
        asm volatile("" ::: "memory");
      }
    }
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

  // Measurement only (a.stamps set by qg_run_timed): thread 0 records for
  // unit b, at stamps[8 b + i], the constant 100 MHz clock at i = 0 the
  // unit's start, 1 the end of its mainloop, 2 after arrive (split-K; the
  // mainloop's end in a data-parallel unit, which publishes nothing),
  // 3 once all waves of the completing unit have read the partials back and
  // summed them (0 in the other split-K units; the mainloop's end in a
  // data-parallel unit), 4 after its stores have completed (= [2] in the
  // split-K units that do not complete their tile), 5 = 1 in a unit that
  // completes its tile, and the shader clock at 6 (start) and 7 (end).
  // Uniform branches on a kernel argument, outside the mainloop.
  __device__ __forceinline__ static void stamp(const Args& a, int b, int i, uint64_t v) {
    if (a.stamps && threadIdx.x == 0) a.stamps[(size_t)b * 8 + i] = v;
  }

  __device__ __forceinline__ static void run_dp(const Args& a, char* smem) {
    const int total = a.tiles_m * a.tiles_n;
    for (int b = blockIdx.x; b < total; b += gridDim.x) {
      const int t = (gridDim.x == (unsigned)total) ? xcd_remap(b, total) : b;
      if (a.stamps) {
        stamp(a, t, 0, __builtin_amdgcn_s_memrealtime());
        stamp(a, t, 6, __builtin_amdgcn_s_memtime());
      }
      Acc acc;
      Unit u = make_unit(a, t, 0, a.iters);
      Core::mainloop(a, u, smem, acc);
      if (a.stamps) {
        const uint64_t t1 = __builtin_amdgcn_s_memrealtime();
        stamp(a, t, 1, t1);
        stamp(a, t, 2, t1);
        stamp(a, t, 3, t1);
      }
      Core::store(a, u, acc, smem);
      if (a.stamps) {
        wait_vmcnt<0>();
        __syncthreads();
        stamp(a, t, 4, __builtin_amdgcn_s_memrealtime());
        stamp(a, t, 5, 1);
        stamp(a, t, 7, __builtin_amdgcn_s_memtime());
      }
    }
  }

  __device__ __forceinline__ static void run_splitk(const Args& a, char* smem, int* flag) {
    const int total = a.tiles_m * a.tiles_n * a.splits;
    for (int b = blockIdx.x; b < total; b += gridDim.x) {
      const int t = b / a.splits, s = b % a.splits;
      const int kb = s * a.iters_per_split, ke = min(a.iters, kb + a.iters_per_split);
      if (a.stamps) {
        stamp(a, b, 0, __builtin_amdgcn_s_memrealtime());
        stamp(a, b, 6, __builtin_amdgcn_s_memtime());
      }
      Acc acc;
      Unit u = make_unit(a, t, kb, ke);
      Core::mainloop(a, u, smem, acc);
      if (a.stamps) stamp(a, b, 1, __builtin_amdgcn_s_memrealtime());
      const bool last = arrive(a, u, t * a.splits + s, acc, flag);
      uint64_t t2 = 0;
      if (a.stamps) stamp(a, b, 2, t2 = __builtin_amdgcn_s_memrealtime());
      if (last) {
        const int ns = (a.iters + a.iters_per_split - 1) / a.iters_per_split;
        reduce(a, ns, [&](int q) { return t * a.splits + q; }, acc);
        if (a.stamps) {
          __syncthreads();  // every wave has its partial tiles summed
          stamp(a, b, 3, __builtin_amdgcn_s_memrealtime());
        }
        Core::store(a, u, acc, smem);
        finish_counter(a, u);
      }
      if (a.stamps) {
        if (last) {
          wait_vmcnt<0>();
          __syncthreads();
          stamp(a, b, 4, __builtin_amdgcn_s_memrealtime());
        } else {
          stamp(a, b, 3, 0);
          stamp(a, b, 4, t2);
        }
        stamp(a, b, 5, last ? 1 : 0);
        stamp(a, b, 7, __builtin_amdgcn_s_memtime());
      }
    }
  }

  // Stream-K (qg_streamk.hpp): whole tiles first, then the program's
  // balanced range of the shared region; a tile's partial pieces are summed
  // in k order by the workgroup that completes it.
  __device__ __forceinline__ static void run_streamk(const Args& a, char* smem, int* flag) {
    StreamK sk;
    sk.tiles = a.tiles_m * a.tiles_n;
    sk.iters = a.iters;
    sk.programs = a.programs;
    sk.dp_tiles = a.dp_tiles;
    sk.work = a.sk_work;
    sk.f = a.sk_work / a.programs;
    sk.r = a.sk_work % a.programs;
    for (int pid = blockIdx.x; pid < a.programs; pid += gridDim.x) {
      StreamKCursor cur(sk, pid);
      int t, kb, ke, slot;
      while (cur.next(t, kb, ke, slot)) {
        Acc acc;
        Unit u = make_unit(a, t, kb, ke);
        Core::mainloop(a, u, smem, acc);
        if (slot < 0) {
          Core::store(a, u, acc, smem);
        } else if (arrive(a, u, slot, acc, flag)) {
          const int w0 = (t - sk.dp_tiles) * sk.iters;
          reduce(a, sk.pieces(w0), [&](int i) { return sk.piece_slot(w0, i); }, acc);
          Core::store(a, u, acc, smem);
          finish_counter(a, u);
        }
      }
    }
  }

  // Grouped: per-expert m-tile prefix built in LDS from the device offsets.
  // Batched (a.offsets == nullptr): E batches of a.M rows, batch e owning rows
  // [e*M, (e+1)*M) of A, C and D; a.tiles_m m-tiles per batch.
  __device__ __forceinline__ static void run_grouped(const Args& a, char* smem, int* pref) {
    const bool batched = a.offsets == nullptr;
    if (!batched) {
      // pref[0..E] = prefix of ceil(rows_e / BM), E <= 1023 (host checked),
      // built by the first wave: lane l takes experts [16 l, 16 l + 16) (its
      // 17 offsets load together), sums them, and a wave-wide scan of the
      // lane sums gives each lane its starting value.
      if (threadIdx.x < 64) {
        constexpr int PER = 16;
        const int l = threadIdx.x, e0 = l * PER;
        int cnt[PER], off[PER + 1];
#pragma unroll
        for (int j = 0; j <= PER; ++j) off[j] = e0 + j <= a.E ? a.offsets[e0 + j] : 0;
        int tot = 0;
#pragma unroll
        for (int j = 0; j < PER; ++j) {
          const int rows = e0 + j < a.E ? off[j + 1] - off[j] : 0;
          cnt[j] = rows > 0 ? (rows + Core::BM - 1) / Core::BM : 0;
          tot += cnt[j];
        }
        int incl = tot;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
          const int y = __shfl_up(incl, d, 64);
          if (l >= d) incl += y;
        }
        int run = incl - tot;
        if (l == 0) pref[0] = 0;
#pragma unroll
        for (int j = 0; j < PER; ++j) {
          run += cnt[j];
          if (e0 + j < a.E) pref[e0 + j + 1] = run;
        }
      }
      __syncthreads();
    }
    const int mtiles = batched ? a.E * a.tiles_m : pref[a.E];
    const int total = mtiles * a.tiles_n;
    for (int b = blockIdx.x; b < total; b += gridDim.x) {
      const int mt = b / a.tiles_n, tn = b - mt * a.tiles_n;
      Unit u;
      if (batched) {
        const int e = mt / a.tiles_m;
        u.expert = e;
        u.m0 = e * a.M + (mt - e * a.tiles_m) * Core::BM;
        u.m_end = (e + 1) * a.M;
      } else {
        int lo = 0, hi = a.E - 1;  // largest e with pref[e] <= mt
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (pref[mid] <= mt)
            lo = mid;
          else
            hi = mid - 1;
        }
        u.expert = lo;
        u.m0 = a.offsets[lo] + (mt - pref[lo]) * Core::BM;
        u.m_end = a.offsets[lo + 1];
      }
      u.tile = b;
      u.n0 = tn * Core::BN;
      u.kb = 0;
      u.ke = a.iters;
      Acc acc;
      Core::mainloop(a, u, smem, acc);
      Core::store(a, u, acc, smem);
    }
  }
};

template <class Core, int MODE>
__global__ __launch_bounds__(Core::NT) void sched_kernel(const Args a) {
  __shared__ __attribute__((aligned(1024))) char smem[Core::SMEM_BYTES];
  __shared__ int misc[MODE == MODE_GROUPED ? 1025 : 1];
  if constexpr (MODE == MODE_DP) Sched<Core>::run_dp(a, smem);
  if constexpr (MODE == MODE_SPLITK) Sched<Core>::run_splitk(a, smem, misc);
  if constexpr (MODE == MODE_STREAMK) Sched<Core>::run_streamk(a, smem, misc);
  if constexpr (MODE == MODE_GROUPED) Sched<Core>::run_grouped(a, smem, misc);
}

// Host-side launcher: one kernel instantiation per schedule.
template <class Core>
hipError_t launch_sched(const Args& a, int grid, hipStream_t s) {
  switch (a.mode) {
    case MODE_DP: hipLaunchKernelGGL((sched_kernel<Core, MODE_DP>), dim3(grid), dim3(Core::NT), 0, s, a); break;
    case MODE_SPLITK: hipLaunchKernelGGL((sched_kernel<Core, MODE_SPLITK>), dim3(grid), dim3(Core::NT), 0, s, a); break;
    case MODE_STREAMK: hipLaunchKernelGGL((sched_kernel<Core, MODE_STREAMK>), dim3(grid), dim3(Core::NT), 0, s, a); break;
    case MODE_GROUPED: hipLaunchKernelGGL((sched_kernel<Core, MODE_GROUPED>), dim3(grid), dim3(Core::NT), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace qg
