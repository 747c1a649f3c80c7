// Stream-K work division, shared by the host planner, the device schedule
// and the engine's introspection call (so that tests on the CPU check the
// very arithmetic the kernels run).
//
// The idea is the one the TileLang tutorial page "gemm_variants.py" illustrates
// with its gemm_streamk kernel: a fixed number of programs (one workgroup
// each) share the k-iterations of the output tiles so that no program idles
// while a last, partly filled wave of tiles finishes. The split below is
// derived here from that goal:
//
//   T tiles of I k-iterations each, P programs.
//   * If T is a multiple of P, every program takes T / P whole tiles: no
//     tile is shared.
//   * Otherwise whole waves of P tiles are taken whole, except the last full
//     wave (when there is one), which joins the ragged remainder: the last
//     P + T % P tiles (all T tiles when T < P) are the shared region. Every
//     program then does the same number of whole tiles plus between one and
//     two tiles' worth of shared iterations, so at least one whole tile of
//     work stands behind every partial one.
//   * The shared region's W = sk_tiles * I iterations are numbered tile-major
//     and cut into P contiguous, balanced ranges: program p owns
//     [floor(p W / P), floor((p + 1) W / P)).
//
// Whole tiles come first (program p: tiles p, p + P, ...), then the program's
// range of the shared region, cut at tile boundaries into pieces. A piece
// that covers a whole tile is stored directly; a partial piece goes to the
// partials workspace, in slot 2p for the program's first piece and 2p + 1
// for its last (a range holds at most two partial pieces: its head and its
// tail; everything between them is whole tiles).
//
// The host keeps T * I below 2^31 and P at most 65535, so the per-unit
// arithmetic runs in 32 bits: floor(p W / P) = p f + floor(p r / P) with
// W = f P + r, and p r < P^2 < 2^32.
#pragma once
#include <stdint.h>

#ifndef __HIPCC__
#define QG_HD inline
#else
#define QG_HD __host__ __device__ __forceinline__
#endif

namespace qg {

constexpr int kStreamKMaxPrograms = 65535;

struct StreamK {
  int tiles;     // T
  int iters;     // I
  int programs;  // P
  int dp_tiles;  // whole tiles taken round-robin before the shared region
  int work;      // W: k-iterations of the shared region
  int f, r;      // W = f P + r

  QG_HD static StreamK make(int tiles, int iters, int programs) {
    StreamK s;
    s.tiles = tiles;
    s.iters = iters;
    s.programs = programs;
    const int rem = tiles % programs;
    int shared = 0;
    if (rem != 0) shared = tiles >= programs ? programs + rem : tiles;
    s.dp_tiles = tiles - shared;
    s.work = shared * iters;
    s.f = s.work / programs;
    s.r = s.work % programs;
    return s;
  }

  // First shared iteration of program p (p = P gives W).
  QG_HD int begin(int p) const { return p * f + (int)(((uint32_t)p * (uint32_t)r) / (uint32_t)programs); }

  // Program whose range holds shared iteration w (0 <= w < W): the largest p
  // with begin(p) <= w, i.e. ceil((w + 1) P / W) - 1.
  QG_HD int owner(int w) const { return (int)((((int64_t)w + 1) * programs + work - 1) / work) - 1; }

  // Slot of program q's piece of the shared tile whose first iteration is w0:
  // its first piece when its range starts inside that tile, else its last.
  QG_HD int slot(int q, int w0) const { return 2 * q + (begin(q) >= w0 ? 0 : 1); }

  // The pieces of the shared tile whose first iteration is w0, in k order.
  // With W >= P every range is non-empty, so the pieces belong to the
  // consecutive programs owner(w0) .. owner(w0 + I - 1). With W < P some
  // ranges are empty (and may lie between owners) while the others hold one
  // iteration each: piece i is then iteration w0 + i.
  QG_HD int pieces(int w0) const { return work < programs ? iters : owner(w0 + iters - 1) - owner(w0) + 1; }
  QG_HD int piece_slot(int w0, int i) const {
    const int q = work < programs ? owner(w0 + i) : owner(w0) + i;
    return slot(q, w0);
  }
};

// The units of one program in execution order: whole tiles, then the pieces
// of its shared range. next() yields (tile, k-iteration range, slot), with
// slot = -1 for a whole tile (stored directly).
struct StreamKCursor {
  int iters, programs, dp_tiles;
  int pid;
  int t;           // next whole tile
  int w, w0, end;  // shared iterations: next, first, one past the last

  QG_HD StreamKCursor(const StreamK& s, int pid_) {
    iters = s.iters;
    programs = s.programs;
    dp_tiles = s.dp_tiles;
    pid = pid_;
    t = pid_;
    w0 = w = s.begin(pid_);
    end = s.begin(pid_ + 1);
  }

  QG_HD bool next(int& tile, int& kb, int& ke, int& slot) {
    if (t < dp_tiles) {
      tile = t;
      kb = 0;
      ke = iters;
      slot = -1;
      t += programs;
      return true;
    }
    if (w >= end) return false;
    const int ts = w / iters;
    kb = w - ts * iters;
    ke = kb + (end - w) < iters ? kb + (end - w) : iters;
    tile = dp_tiles + ts;
    slot = (kb == 0 && ke == iters) ? -1 : 2 * pid + (w == w0 ? 0 : 1);
    w += ke - kb;
    return true;
  }
};

}  // namespace qg
