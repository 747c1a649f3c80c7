// Host engine behind the C ABI of libqgemm.so.
//
// Mirrors the Gemm class of the page "InternLM Lmdeploy Gemm Interface": a
// handle (created once per device) owns the kernel registry view, a dispatch
// cache keyed by problem, a context that analyses the problem and filters the
// registry, and a measurer that times candidates when asked to. Run validates
// the operands, finds a plan (cache -> heuristic, or measurement), checks the
// workspace, fills the kernel argument block and launches on the caller's
// stream. Export/Import serialise the cache as versioned text.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <sstream>
#include <string>
#include <unordered_map>
#include <vector>

#include "../../include/qgemm.h"
#include "qg_args.hpp"
#include "qg_registry.hpp"
#include "qg_streamk.hpp"

using namespace qg;

namespace {

const char* kVersion = "qgemm 0.1.0";
const size_t kBarriersSize = size_t(1) << 20;
const size_t kPartialsSize = size_t(32) << 20;
const int kTuningSeq[] = {1,   2,   4,   8,    16,   24,   32,   48,   64,   96,   128,  192,
                          256, 384, 512, 768, 1024, 1536, 2048, 3072, 4096, 6144, 8192};

int esize(int t) {
  switch (t) {
    case DT_F32:
    case DT_I32:
    case DT_U4: return 4;  // U4: ld counted in 32-bit words
    case DT_F16:
    case DT_BF16: return 2;
    case DT_E4M3:
    case DT_I8: return 1;
    default: return 0;
  }
}
const char* dt_name(int t) {
  static const char* n[] = {"f32", "f16", "bf16", "e4m3", "i8", "i32", "u4"};
  return (t >= 0 && t <= 6) ? n[t] : "-";
}
const char* sched_name(int m) {
  switch (m) {
    case MODE_DP: return "dp";
    case MODE_SPLITK: return "splitk";
    case MODE_STREAMK: return "streamk";
    case MODE_GROUPED: return "grouped";
    default: return "?";
  }
}
int sched_from_name(const std::string& s) {
  if (s == "dp") return MODE_DP;
  if (s == "splitk") return MODE_SPLITK;
  if (s == "streamk") return MODE_STREAMK;
  if (s == "grouped") return MODE_GROUPED;
  return -1;
}
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }
int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// A validated, normalised problem.
struct Problem {
  int ta = -1, tb = -1, tc = -1, td = -1;
  int qa = QG_QUANT_NONE, qb = QG_QUANT_NONE;
  int64_t M = 0, N = 0, K = 0;
  int E = 0;  // > 0: grouped (offsets) or batched (E batches of M rows)
  bool batched = false;
  const void *A = nullptr, *B = nullptr, *C = nullptr, *U = nullptr, *V = nullptr;
  void* D = nullptr;
  int64_t lda = 0, ldb = 0, ldc = 0, ldd = 0, ldu = 0, ldv = 0, b_batch = 0, v_batch = 0;
  const int32_t* offsets = nullptr;
  float alpha = 1.f, beta = 0.f;
  int zp = 8, group_k = 128;
  int epi = 0, bias_type = -1;
  const void* bias = nullptr;
  const float* row_scale = nullptr;
  float out_zp = 0.f;
  bool w8a8 = false;  // int8 A, B with fp32 scales per row of A and per row of B

  std::string key() const {
    char buf[160];
    snprintf(buf, sizeof buf, "%s.%s.%s.%s.q%d%d.e%d%s.x%d.n%lld.k%lld", dt_name(ta), dt_name(tb),
             tc < 0 ? "-" : dt_name(tc), dt_name(td), qa, qb, E, batched ? "b" : "", epi, (long long)N, (long long)K);
    return std::string(buf);
  }
};

struct Choice {
  int kernel = -1;
  int mode = MODE_DP;
  int split = 1;
  int programs = 0;
};

struct Entry {
  Choice c;
  double us = 0;
};

struct Plan {
  Choice c;
  Args a;
  int grid = 0;
  size_t partials = 0, barriers = 0;
  int tiles = 0;
  bool batched = false;
};

}  // namespace

namespace {

// Memo of resolved DEFAULT-policy choices, keyed by everything the cache
// lookup and the heuristic read (exact M, problem key fields, workspace
// sizes). It turns a repeated call into one hash lookup instead of
// formatting text keys and probing the tuning-sequence buckets; any change to
// the cache (measure, import) clears it.
struct MemoKey {
  int64_t M, N, K;
  int32_t ta, tb, tc, td, qa, qb, E, batched, epi, pad;
  uint64_t ws_partials, ws_barriers;
  bool operator==(const MemoKey& o) const { return memcmp(this, &o, sizeof o) == 0; }
};
struct MemoHash {
  size_t operator()(const MemoKey& k) const {
    const unsigned char* b = reinterpret_cast<const unsigned char*>(&k);
    uint64_t h = 1469598103934665603ull;  // FNV-1a
    for (size_t i = 0; i < sizeof k; ++i) h = (h ^ b[i]) * 1099511628211ull;
    return (size_t)h;
  }
};

}  // namespace

struct qg_handle {
  int device = -1;
  int cus = 256;
  std::string arch = "gfx950";
  bool online = false;
  std::mutex mu;
  std::map<std::string, Entry> cache;  // key: "<M>|<problem key>"
  std::unordered_map<MemoKey, Choice, MemoHash> memo;
};

namespace {

std::string cache_key(int64_t M, const std::string& pk) { return std::to_string(M) + "|" + pk; }

// ---- validation -----------------------------------------------------------
int check_layout(const qg_layout* L, bool need_rows_cols_ok = true) {
  if (!L) return QG_ERR_INVALID_ARG;
  if (L->order != QG_ROW_MAJOR) return L->order == QG_COL_MAJOR ? QG_ERR_UNSUPPORTED : QG_ERR_INVALID_ARG;
  if (L->type < 0 || L->type > QG_U4) return QG_ERR_INVALID_ARG;
  if (need_rows_cols_ok && (L->rows < 0 || L->cols < 0)) return QG_ERR_INVALID_ARG;
  if (L->ld < 0) return QG_ERR_INVALID_ARG;
  // the kernels index rows, columns and pitches in 32 bits; bounding them
  // here also keeps the size arithmetic of the checks below from overflowing
  if (L->rows > INT32_MAX || L->cols > INT32_MAX || L->ld > INT32_MAX) return QG_ERR_UNSUPPORTED;
  return QG_OK;
}

int validate(const qg_operation* op, float alpha, const void* A, const qg_layout* Ad, const void* U, const qg_layout* Ud,
             const void* B, const qg_layout* Bd, const void* V, const qg_layout* Vd, float beta, const void* C,
             const qg_layout* Cd, void* D, const qg_layout* Dd, Problem& p) {
  if (!op || !Ad || !Bd || !Dd) return QG_ERR_INVALID_ARG;
  int st;
  if ((st = check_layout(Ad)) || (st = check_layout(Bd)) || (st = check_layout(Dd))) return st;
  // epilogue flags and their operands
  {
    const int e = op->epilogue;
    if (e & ~(QG_EPI_BIAS | QG_EPI_RELU | QG_EPI_GELU | QG_EPI_QUANT_I8)) return QG_ERR_INVALID_ARG;
    if ((e & QG_EPI_RELU) && (e & QG_EPI_GELU)) return QG_ERR_INVALID_ARG;
    p.epi = e;
    if (e & QG_EPI_BIAS) {
      const int bt = op->epi.bias_type;
      if (!(bt == QG_F32 || bt == QG_BF16 || bt == QG_F16)) return QG_ERR_UNSUPPORTED;
      if (!op->epi.bias) return QG_ERR_INVALID_ARG;
      if (!aligned16(op->epi.bias)) return QG_ERR_ALIGNMENT;
      p.bias = op->epi.bias;
      p.bias_type = bt;
    }
    if (e & QG_EPI_QUANT_I8) {
      if (!op->epi.row_scale) return QG_ERR_INVALID_ARG;
      if (reinterpret_cast<uintptr_t>(op->epi.row_scale) & 3) return QG_ERR_ALIGNMENT;
      if (!std::isfinite(op->epi.zero_point)) return QG_ERR_INVALID_ARG;
      p.row_scale = op->epi.row_scale;
      p.out_zp = op->epi.zero_point;
    }
  }
  if (!std::isfinite(alpha) || !std::isfinite(beta)) return QG_ERR_INVALID_ARG;
  p.alpha = alpha;
  p.beta = beta;
  p.ta = Ad->type;
  p.tb = Bd->type;
  p.td = Dd->type;
  p.M = Ad->rows;
  p.K = Ad->cols;
  p.N = Bd->rows;
  p.qa = op->quant_a.kind;
  p.qb = op->quant_b.kind;
  if (Bd->cols != p.K || Dd->rows != p.M || Dd->cols != p.N) return QG_ERR_INVALID_ARG;
  if (p.M > INT32_MAX || p.N > INT32_MAX || p.K > INT32_MAX) return QG_ERR_UNSUPPORTED;
  // grouped (device offsets) or batched (num > 1 without offsets: E batches of
  // M rows, A/C/D batches contiguous, B batches `stride` apart)
  const bool grouped = Ad->num > 1 || Bd->num > 1 || Dd->num > 1 || Ad->offsets != nullptr;
  if (grouped) {
    if (Ad->num < 1 || Bd->num != Ad->num) return QG_ERR_INVALID_ARG;
    p.E = Ad->num;
    if (Ad->offsets) {
      if (Dd->num != Ad->num && Dd->num > 1) return QG_ERR_INVALID_ARG;
      if (Dd->offsets && Dd->offsets != Ad->offsets) return QG_ERR_UNSUPPORTED;
      if (Ad->num > 1023) return QG_ERR_UNSUPPORTED;
      p.offsets = Ad->offsets;
      if (!aligned16(p.offsets) && (reinterpret_cast<uintptr_t>(p.offsets) & 3)) return QG_ERR_ALIGNMENT;
    } else {
      p.batched = true;
      if (Dd->num != Ad->num || Dd->offsets) return QG_ERR_INVALID_ARG;
      if (Ad->stride != Ad->rows * Ad->ld || Dd->stride != Dd->rows * Dd->ld) return QG_ERR_UNSUPPORTED;
      if ((int64_t)p.E * p.M > INT32_MAX) return QG_ERR_UNSUPPORTED;
    }
  }
  // dtype combinations
  const bool float16ish = (p.ta == QG_BF16 || p.ta == QG_F16);
  if (p.ta == QG_I8 && (p.qa || p.qb)) {
    // w8a8: a(i,k) = qa * U[i], b(j,k) = qb * V[j] (fp32 scales over whole
    // rows: block quantisation with group_mn = 1 and group_k covering K);
    // exact int32 sums, then the float epilogue
    if (p.tb != QG_I8 || p.qa != QG_QUANT_BLOCK_F32 || p.qb != QG_QUANT_BLOCK_F32) return QG_ERR_UNSUPPORTED;
    const qg_quant &qa = op->quant_a, &qb = op->quant_b;
    if (qa.group_mn != 1 || qb.group_mn != 1) return QG_ERR_UNSUPPORTED;
    if ((qa.group_k != 0 && qa.group_k < p.K) || (qb.group_k != 0 && qb.group_k < p.K)) return QG_ERR_UNSUPPORTED;
    if (grouped) return QG_ERR_UNSUPPORTED;
    if (!Ud || !Vd) return QG_ERR_INVALID_ARG;
    if ((st = check_layout(Ud)) || (st = check_layout(Vd))) return st;
    if (Ud->type != QG_F32 || Vd->type != QG_F32) return QG_ERR_UNSUPPORTED;
    if (Ud->rows != p.M || Vd->rows != p.N || Ud->cols < 1 || Vd->cols < 1 || Ud->ld < 1 || Vd->ld < 1)
      return QG_ERR_INVALID_ARG;
    if (p.M > 0 && p.N > 0 && (!U || !V)) return QG_ERR_INVALID_ARG;
    if ((reinterpret_cast<uintptr_t>(U) & 3) || (reinterpret_cast<uintptr_t>(V) & 3)) return QG_ERR_ALIGNMENT;
    if (!(p.td == QG_F32 || p.td == QG_BF16 || p.td == QG_F16 || p.td == QG_I8)) return QG_ERR_UNSUPPORTED;
    p.w8a8 = true;
    p.U = U;
    p.V = V;
    p.ldu = Ud->ld;
    p.ldv = Vd->ld;
  } else if (p.ta == QG_I8) {
    if (p.tb != QG_I8 || p.td != QG_I32 || p.epi) return QG_ERR_UNSUPPORTED;
    if (alpha != 1.f || !(beta == 0.f || beta == 1.f)) return QG_ERR_UNSUPPORTED;
  } else if (float16ish) {
    if (p.tb == QG_U4) {
      // weight-only int4: bf16 A, 128-deep groups of fp16 scales in V
      if (p.ta != QG_BF16 || p.qa != QG_QUANT_NONE || p.qb != QG_QUANT_INT4_ZP) return QG_ERR_UNSUPPORTED;
      if (op->quant_b.group_k != 128 || p.K % 128) return QG_ERR_UNSUPPORTED;
      if (op->quant_b.zero_point < 0 || op->quant_b.zero_point > 15) return QG_ERR_INVALID_ARG;
      if (grouped) return QG_ERR_UNSUPPORTED;
      if (!Vd || (p.M > 0 && p.N > 0 && p.K > 0 && !V)) return QG_ERR_INVALID_ARG;
      if ((st = check_layout(Vd))) return st;
      if (Vd->type != QG_F16 || Vd->rows != p.N || Vd->cols != p.K / 128 || Vd->ld < Vd->cols) return QG_ERR_INVALID_ARG;
      if ((Vd->ld * 2) % 16 || !aligned16(V)) return QG_ERR_ALIGNMENT;
      p.V = V;
      p.ldv = Vd->ld;
      p.zp = op->quant_b.zero_point;
      p.group_k = 128;
      // optional per-group zero points (asymmetric int4): one byte per column
      // and group in U, replacing the constant zero point
      if (U || Ud) {
        if (!U || !Ud) return QG_ERR_INVALID_ARG;
        if ((st = check_layout(Ud))) return st;
        if (Ud->type != QG_I8) return QG_ERR_UNSUPPORTED;
        if (Ud->rows != p.N || Ud->cols != p.K / 128 || Ud->ld < Ud->cols) return QG_ERR_INVALID_ARG;
        if (Ud->ld % 16 || !aligned16(U)) return QG_ERR_ALIGNMENT;
        p.U = U;
        p.ldu = Ud->ld;
      }
    } else if (p.tb != p.ta || p.qa || p.qb) {
      return QG_ERR_UNSUPPORTED;
    }
    if (!(p.td == QG_F32 || p.td == QG_BF16 || p.td == QG_F16 || p.td == QG_I8)) return QG_ERR_UNSUPPORTED;
  } else if (p.ta == QG_E4M3) {
    // block-scaled fp8: U fp32 per row and 128-deep k group, V fp32 per
    // 128 x 128 block of B (per expert when grouped)
    if (p.tb != QG_E4M3 || p.qa != QG_QUANT_BLOCK_F32 || p.qb != QG_QUANT_BLOCK_F32) return QG_ERR_UNSUPPORTED;
    if (op->quant_a.group_k != 128 || op->quant_b.group_k != 128 || op->quant_a.group_mn != 1 ||
        op->quant_b.group_mn != 128)
      return QG_ERR_UNSUPPORTED;
    if (!Ud || !Vd) return QG_ERR_INVALID_ARG;
    if ((st = check_layout(Ud)) || (st = check_layout(Vd))) return st;
    if (Ud->type != QG_F32 || Vd->type != QG_F32) return QG_ERR_UNSUPPORTED;
    const int64_t kg = cdiv(p.K, 128);
    if (Ud->rows != p.M || Ud->cols != kg || Ud->ld < kg) return QG_ERR_INVALID_ARG;
    if (Vd->rows != cdiv(p.N, 128) || Vd->cols != kg || Vd->ld < kg) return QG_ERR_INVALID_ARG;
    if (p.M > 0 && p.N > 0 && p.K > 0 && (!U || !V)) return QG_ERR_INVALID_ARG;
    if ((Ud->ld * 4) % 16 || (Vd->ld * 4) % 16 || !aligned16(U) || !aligned16(V)) return QG_ERR_ALIGNMENT;
    if (grouped) {
      if (Vd->num != Ad->num) return QG_ERR_INVALID_ARG;
      p.v_batch = Vd->stride;
      if (p.v_batch != 0 && p.v_batch < Vd->rows * Vd->ld) return QG_ERR_INVALID_ARG;
      if (!Ad->offsets && Ud->stride != Ud->rows * Ud->ld) return QG_ERR_UNSUPPORTED;
    }
    p.U = U;
    p.V = V;
    p.ldu = Ud->ld;
    p.ldv = Vd->ld;
    if (!(p.td == QG_F32 || p.td == QG_BF16 || p.td == QG_F16 || p.td == QG_I8)) return QG_ERR_UNSUPPORTED;
  } else {
    return QG_ERR_UNSUPPORTED;
  }
  // int8 output only as quantised codes, and quantised codes only as int8
  if ((p.td == QG_I8) != ((p.epi & QG_EPI_QUANT_I8) != 0)) return QG_ERR_UNSUPPORTED;
  // pointers, leading dimensions, alignment
  if (p.M > 0 && p.N > 0) {
    if (!D) return QG_ERR_INVALID_ARG;
    if (p.K > 0 && (!A || !B)) return QG_ERR_INVALID_ARG;
  }
  p.A = A;
  p.B = B;
  p.D = D;
  p.lda = Ad->ld;
  p.ldb = Bd->ld;
  p.ldd = Dd->ld;
  const int64_t b_row_elems = p.tb == QG_U4 ? p.ldb * 8 : p.ldb;  // U4: ld counts words
  if (p.lda < p.K || b_row_elems < p.K || p.ldd < p.N) return QG_ERR_INVALID_ARG;
  if (p.tb == QG_U4 && p.K % 8) return QG_ERR_ALIGNMENT;
  if ((p.lda * esize(p.ta)) % 16 || (p.ldb * esize(p.tb)) % 16 || (p.ldd * esize(p.td)) % 16) return QG_ERR_ALIGNMENT;
  // K itself need not keep rows 16-byte aligned: the kernels read a row's
  // last partial 16-byte chunk whole (it lies inside the row pitch) and zero
  // its bytes past K on chip
  if (!aligned16(A) || !aligned16(B) || !aligned16(D)) return QG_ERR_ALIGNMENT;
  if (grouped) {
    p.b_batch = Bd->stride;  // 0: every group uses the same B
    if (p.b_batch != 0 && p.b_batch < p.N * p.ldb) return QG_ERR_INVALID_ARG;
  }
  // C: only read when beta != 0
  p.tc = -1;
  if (beta != 0.f) {
    if (!C || !Cd) return QG_ERR_INVALID_ARG;
    if ((st = check_layout(Cd))) return st;
    if (Cd->rows != p.M || Cd->cols != p.N || Cd->ld < p.N) return QG_ERR_INVALID_ARG;
    if (p.ta == QG_I8 && !p.w8a8) {
      if (Cd->type != QG_I32) return QG_ERR_UNSUPPORTED;
    } else if (!(Cd->type == QG_F32 || Cd->type == QG_BF16 || Cd->type == QG_F16)) {
      return QG_ERR_UNSUPPORTED;
    }
    if ((Cd->ld * esize(Cd->type)) % 16 || !aligned16(C)) return QG_ERR_ALIGNMENT;
    if (p.batched && (Cd->num != p.E || Cd->offsets || Cd->stride != Cd->rows * Cd->ld)) return QG_ERR_UNSUPPORTED;
    p.tc = Cd->type;
    p.C = C;
    p.ldc = Cd->ld;
  }
  (void)U;
  (void)Ud;
  (void)V;
  (void)Vd;
  // 32-bit buffer offsets: a tile's rows must span less than 2 GiB
  if (p.lda * esize(p.ta) * 256 >= (int64_t(1) << 31) || p.ldb * esize(p.tb) * 256 >= (int64_t(1) << 31))
    return QG_ERR_UNSUPPORTED;
  return QG_OK;
}

// ---- registry filtering ("Context") ------------------------------------------
bool compatible(const KernelInfo& k, const Problem& p) {
  if (k.family == FAM_W4) return p.ta == QG_BF16 && p.tb == QG_U4 && p.E == 0;
  if (k.family == FAM_F8) return p.ta == QG_E4M3 && p.tb == QG_E4M3;
  if (k.family != FAM_TILE && k.family != FAM_SKINNY) return false;
  if (k.family == FAM_SKINNY && p.M > k.bm && p.E == 0) return false;  // skinny tiles cover all rows
  return k.in_type == p.ta && p.tb == p.ta;
}

int find_kernel(const char* name) {
  for (int i = 0; i < kNumKernels; ++i)
    if (!strcmp(kKernels[i].name, name)) return i;
  return -1;
}

// Builds the launch for a choice; checks the workspace.
int make_plan(const qg_handle* h, const Problem& p, const Choice& c, const qg_workspace* ws, Plan& pl) {
  if (c.kernel < 0 || c.kernel >= kNumKernels) return QG_ERR_NO_KERNEL;
  const KernelInfo& k = kKernels[c.kernel];
  if (!compatible(k, p)) return QG_ERR_NO_KERNEL;
  pl = Plan();
  pl.c = c;
  Args& a = pl.a;
  memset(&a, 0, sizeof a);
  a.A = p.A;
  a.B = p.B;
  a.C = p.C;
  a.D = p.D;
  a.U = p.U;
  a.V = p.V;
  a.offsets = p.offsets;
  a.lda = p.lda;
  a.ldb = p.ldb;
  a.ldc = p.ldc;
  a.ldd = p.ldd;
  a.ldu = p.ldu;
  a.ldv = p.ldv;
  a.b_batch = p.b_batch;
  a.v_batch = p.v_batch;
  a.M = (int32_t)p.M;
  a.N = (int32_t)p.N;
  a.K = (int32_t)p.K;
  a.E = p.E;
  a.alpha = p.alpha;
  a.beta = p.beta;
  a.c_type = p.tc;
  a.d_type = p.td;
  a.zero_point = p.zp;
  a.group_k = p.group_k;
  a.epi = p.epi;
  a.int_scaled = p.w8a8 ? 1 : 0;
  a.bias_type = p.bias_type;
  a.bias = p.bias;
  a.row_scale = p.row_scale;
  a.out_zero_point = p.out_zp;
  a.tiles_n = (int32_t)cdiv(p.N, k.bn);
  a.iters = (int32_t)cdiv(p.K, k.bk);
  a.group_m = 4;
  int mode = c.mode;
  if (p.E > 0) mode = MODE_GROUPED;
  if (a.iters == 0 && mode != MODE_GROUPED) mode = MODE_DP;
  pl.c.mode = mode;
  a.mode = mode;
  if (mode == MODE_GROUPED && p.batched) {
    a.tiles_m = (int32_t)cdiv(p.M, k.bm);  // m-tiles per batch
    const int64_t tiles = (int64_t)p.E * a.tiles_m * a.tiles_n;
    if (tiles > INT32_MAX / 2) return QG_ERR_UNSUPPORTED;
    pl.tiles = (int)tiles;
    pl.grid = (int)std::max<int64_t>(1, std::min<int64_t>(tiles, (int64_t)h->cus * 4));
    pl.c.split = 1;
    pl.c.programs = 0;
    pl.batched = true;
  } else if (mode == MODE_GROUPED) {
    a.tiles_m = (int32_t)(cdiv(p.M, k.bm) + p.E);  // upper bound on the padded m-tiles
    const int64_t ub = (int64_t)a.tiles_m * a.tiles_n;
    pl.tiles = (int)std::min<int64_t>(ub, INT32_MAX);
    pl.grid = (int)std::max<int64_t>(1, std::min<int64_t>(ub, (int64_t)h->cus * 2));
    pl.c.split = 1;
    pl.c.programs = 0;
  } else {
    a.tiles_m = (int32_t)cdiv(p.M, k.bm);
    const int64_t tiles = (int64_t)a.tiles_m * a.tiles_n;
    if (tiles > INT32_MAX / 64) return QG_ERR_UNSUPPORTED;
    pl.tiles = (int)tiles;
    if (mode == MODE_DP) {
      pl.grid = (int)tiles;
      pl.c.split = 1;
      pl.c.programs = 0;
    } else if (mode == MODE_SPLITK) {
      int s = std::max(1, std::min(c.split, a.iters));
      const int ips = (int)cdiv(a.iters, s);
      s = (int)cdiv(a.iters, ips);  // no empty chunks
      a.splits = s;
      a.iters_per_split = ips;
      pl.c.split = s;
      pl.grid = (int)(tiles * s);
      pl.partials = (size_t)tiles * s * k.slot_bytes;
      pl.barriers = (size_t)tiles * 4;
      if (s == 1) {
        mode = MODE_DP;
        a.mode = pl.c.mode = MODE_DP;
        pl.partials = pl.barriers = 0;
        pl.grid = (int)tiles;
      }
    } else if (mode == MODE_STREAMK) {
      const int P = c.programs > 0 ? c.programs : h->cus;
      // the device arithmetic runs in 32 bits (qg_streamk.hpp)
      if (P > kStreamKMaxPrograms || tiles * a.iters > INT32_MAX) return QG_ERR_UNSUPPORTED;
      const StreamK sk = StreamK::make((int)tiles, a.iters, P);
      a.programs = P;
      a.dp_tiles = sk.dp_tiles;
      a.sk_work = sk.work;
      pl.c.programs = P;
      pl.c.split = 1;
      pl.grid = P;
      pl.partials = (size_t)2 * P * k.slot_bytes;
      pl.barriers = (size_t)tiles * 4;
    } else {
      return QG_ERR_INVALID_ARG;
    }
  }
  if (pl.partials || pl.barriers) {
    if (!ws || !ws->partials || !ws->barriers) return QG_ERR_WORKSPACE;
    if (ws->partials_size < pl.partials || ws->barriers_size < pl.barriers) return QG_ERR_WORKSPACE;
    if (!aligned16(ws->partials) || (reinterpret_cast<uintptr_t>(ws->barriers) & 3)) return QG_ERR_ALIGNMENT;
    a.partials = ws->partials;
    a.counters = (int32_t*)ws->barriers;
  }
  a.grid = pl.grid;
  return QG_OK;
}

int kernel_by_shape(const Problem& p, int bm, int bn) {
  for (int i = 0; i < kNumKernels; ++i)
    if (kKernels[i].bm == bm && kKernels[i].bn == bn && compatible(kKernels[i], p)) return i;
  return -1;
}

// Skinny kernel (M <= its row tile) for a target column-tile width: the
// smallest registered width >= target (the widest if none is that wide);
// among equal widths the one with the smallest row tile that covers M.
int skinny_for(const Problem& p, int64_t target_bn) {
  int best = -1;
  for (int i = 0; i < kNumKernels; ++i) {
    const KernelInfo& k = kKernels[i];
    if (k.family != FAM_SKINNY || !compatible(k, p)) continue;
    if (best < 0) {
      best = i;
      continue;
    }
    const KernelInfo& b = kKernels[best];
    const bool k_ok = k.bn >= target_bn, b_ok = b.bn >= target_bn;
    if (k_ok != b_ok) {
      if (k_ok) best = i;
      continue;
    }
    const bool better_bn = k_ok ? k.bn < b.bn : k.bn > b.bn;
    if (better_bn || (k.bn == b.bn && k.bm < b.bm)) best = i;
  }
  return best;
}

// Shape heuristic used on a cache miss. `mode` / `split` are the schedule the
// caller forces (MODE_DP with split 0 = nothing forced).
Choice heuristic(const qg_handle* h, const Problem& p, const qg_workspace* ws, int forced_mode = -1,
                 int forced_split = 0) {
  Choice c;
  const int cus = h->cus;
  if (p.E > 0 && p.ta == QG_E4M3) {
    c.kernel = kernel_by_shape(p, p.batched && p.M <= 64 ? 64 : 128, 256);
    c.mode = MODE_GROUPED;
    return c;
  }
  if (p.batched) {
    // per-batch shape decides the tile; skinny kernels for small M, sized so
    // that all batches together give about one tile per compute unit
    c.mode = MODE_GROUPED;
    if (p.M <= 32) c.kernel = skinny_for(p, cdiv(p.N * p.E, cus));
    if (c.kernel < 0)
      c.kernel = kernel_by_shape(p, p.M >= 256 && p.N >= 256 ? 256 : 128, p.M >= 256 && p.N >= 256 ? 256 : 128);
    if (c.kernel < 0) c.kernel = kernel_by_shape(p, 128, 128);
    return c;
  }
  if (p.E > 0) {
    const int64_t avg = p.M / std::max(1, p.E);
    c.kernel = kernel_by_shape(p, avg >= 256 ? 256 : 128, avg >= 256 ? 256 : 128);
    if (c.kernel < 0) c.kernel = kernel_by_shape(p, 128, 128);
    c.mode = MODE_GROUPED;
    return c;
  }
  const bool ws_ok = ws && ws->partials && ws->barriers;
  if (p.tb == QG_U4) {
    // the smallest row tile that covers M (16, 32, then 64-row tiles), so B
    // is read once per 64 rows
    c.kernel = kernel_by_shape(p, p.M <= 16 ? 16 : (p.M <= 32 ? 32 : 64), 128);
    if (c.kernel < 0) return c;
    const KernelInfo& k = kKernels[c.kernel];
    const int64_t tiles = cdiv(p.M, k.bm) * cdiv(p.N, k.bn), iters = cdiv(p.K, k.bk);
    c.mode = MODE_DP;
    if (forced_mode < 0 && tiles < cus && iters >= 4 && ws_ok) {
      const int s = (int)std::max<int64_t>(1, std::min<int64_t>(cdiv(cus, tiles), iters / 2));
      if (s > 1 && (size_t)tiles * s * k.slot_bytes <= ws->partials_size && (size_t)tiles * 4 <= ws->barriers_size) {
        c.mode = MODE_SPLITK;
        c.split = s;
      }
    }
    return c;
  }
  if (p.ta == QG_E4M3) {
    c.kernel = kernel_by_shape(p, p.M <= 64 ? 64 : 128, 256);
  } else if (p.M <= 32) {
    // Skinny GEMM: aim for about one workgroup per compute unit.
    int64_t target = cdiv(p.N, cus);
    if (forced_mode == MODE_SPLITK && forced_split > 1) target = cdiv(p.N * forced_split, cus);
    // stream-K: far fewer tiles than programs, so that tiles really are
    // shared; at the decode shape this picks the 128-column shared-A kernel
    // (measured 26.3-26.7 us against 27.0 us for 32-column tiles)
    if (forced_mode == MODE_STREAMK) target = cdiv(p.N * 8, cus);
    c.kernel = skinny_for(p, target);
    if (c.kernel >= 0) {
      const KernelInfo& k = kKernels[c.kernel];
      const int64_t tiles = cdiv(p.N, k.bn), iters = cdiv(p.K, k.bk);
      c.mode = MODE_DP;
      if (forced_mode < 0 && tiles < cus && iters >= 8 && ws_ok) {
        const int s = (int)std::max<int64_t>(1, std::min<int64_t>(cdiv(cus, tiles), iters / 4));
        if (s > 1 && (size_t)tiles * s * k.slot_bytes <= ws->partials_size && (size_t)tiles * 4 <= ws->barriers_size) {
          c.mode = MODE_SPLITK;
          c.split = s;
        }
      }
      return c;
    }
    c.kernel = kernel_by_shape(p, 32, 128);
  } else if (p.M >= 2048 && p.N >= 2048) {
    c.kernel = kernel_by_shape(p, 256, 256);
  } else {
    c.kernel = kernel_by_shape(p, 128, 128);
  }
  if (c.kernel < 0) {
    for (int i = 0; i < kNumKernels; ++i)
      if (compatible(kKernels[i], p) && kKernels[i].family == FAM_TILE) {
        c.kernel = i;
        break;
      }
  }
  if (c.kernel < 0) return c;
  const KernelInfo& k = kKernels[c.kernel];
  const int64_t tiles = cdiv(p.M, k.bm) * cdiv(p.N, k.bn);
  const int64_t iters = cdiv(p.K, k.bk);
  c.mode = MODE_DP;
  if (forced_mode < 0 && tiles < cus && iters >= 16) {
    int s = (int)std::min<int64_t>(cdiv(cus, tiles), iters / 8);
    s = std::max(1, std::min(s, 16));
    if (s > 1 && ws_ok && (size_t)tiles * s * k.slot_bytes <= ws->partials_size &&
        (size_t)tiles * 4 <= ws->barriers_size) {
      c.mode = MODE_SPLITK;
      c.split = s;
    }
  }
  return c;
}

bool lookup(qg_handle* h, const Problem& p, Choice& c, bool exact_only) {
  std::lock_guard<std::mutex> g(h->mu);
  const std::string pk = p.key();
  auto it = h->cache.find(cache_key(p.M, pk));
  if (it != h->cache.end()) {
    c = it->second.c;
    return true;
  }
  if (exact_only) return false;
  for (int m : kTuningSeq) {
    if (m < p.M) continue;
    auto jt = h->cache.find(cache_key(m, pk));
    if (jt != h->cache.end()) {
      c = jt->second.c;
      return true;
    }
  }
  return false;
}

int launch(const Plan& pl, hipStream_t s) {
  if (pl.grid <= 0) return QG_OK;
  const KernelInfo& k = kKernels[pl.c.kernel];
  hipError_t e = k.launch(pl.a, pl.grid, s);
  if (e != hipSuccess) {
    // the status code carries no HIP detail; QG_VERBOSE=1 prints it
    static const bool verbose = getenv("QG_VERBOSE") && atoi(getenv("QG_VERBOSE")) > 0;
    if (verbose) fprintf(stderr, "qgemm: launch of %s failed: %s\n", k.name, hipGetErrorString(e));
    return QG_ERR_HIP;
  }
  return QG_OK;
}

std::string describe(const Plan& pl) {
  char buf[320];
  const KernelInfo& k = kKernels[pl.c.kernel];
  snprintf(buf, sizeof buf,
           "kernel=%s schedule=%s split=%d programs=%d tiles=%d grid=%d partials=%zu barriers=%zu bm=%d bn=%d bk=%d",
           k.name, pl.batched ? "batched" : sched_name(pl.c.mode), pl.c.split, pl.c.programs, pl.tiles, pl.grid, pl.partials, pl.barriers, k.bm,
           k.bn, k.bk);
  return std::string(buf);
}

// Candidate choices for the measurer.
std::vector<Choice> candidates(const qg_handle* h, const Problem& p) {
  std::vector<Choice> out;
  for (int i = 0; i < kNumKernels; ++i) {
    if (!compatible(kKernels[i], p)) continue;
    Choice c;
    c.kernel = i;
    if (p.E > 0) {
      c.mode = MODE_GROUPED;
      out.push_back(c);
      continue;
    }
    c.mode = MODE_DP;
    out.push_back(c);
    for (int s : {2, 4, 8, 16}) {
      c.mode = MODE_SPLITK;
      c.split = s;
      out.push_back(c);
    }
    c.mode = MODE_STREAMK;
    c.split = 1;
    c.programs = h->cus;
    out.push_back(c);
  }
  return out;
}

int measure(qg_handle* h, const Problem& p, const qg_workspace* ws, hipStream_t s, Choice& best) {
  if (p.tc >= 0 && p.C == p.D) return QG_ERR_UNSUPPORTED;  // repeated runs would compound
  hipEvent_t e0, e1;
  if (hipEventCreate(&e0) != hipSuccess) return QG_ERR_HIP;
  if (hipEventCreate(&e1) != hipSuccess) {
    (void)hipEventDestroy(e0);
    return QG_ERR_HIP;
  }
  double best_us = 1e30;
  int found = 0, st = QG_OK;
  for (const Choice& c : candidates(h, p)) {
    Plan pl;
    if (make_plan(h, p, c, ws, pl) != QG_OK) continue;
    if ((st = launch(pl, s)) != QG_OK) break;  // warm-up
    if (hipStreamSynchronize(s) != hipSuccess) {
      st = QG_ERR_HIP;
      break;
    }
    float ms_min = 1e30f;
    for (int r = 0; r < 3; ++r) {
      (void)hipEventRecord(e0, s);
      if ((st = launch(pl, s)) != QG_OK) break;
      (void)hipEventRecord(e1, s);
      if (hipEventSynchronize(e1) != hipSuccess) {
        st = QG_ERR_HIP;
        break;
      }
      float ms = 0;
      (void)hipEventElapsedTime(&ms, e0, e1);
      ms_min = std::min(ms_min, ms);
    }
    if (st != QG_OK) break;
    if (ms_min * 1e3 < best_us) {
      best_us = ms_min * 1e3;
      best = pl.c;
      found = 1;
    }
  }
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  if (st != QG_OK) return st;
  if (!found) return QG_ERR_NO_KERNEL;
  std::lock_guard<std::mutex> g(h->mu);
  Entry en;
  en.c = best;
  en.us = best_us;
  h->cache[cache_key(p.M, p.key())] = en;
  h->memo.clear();
  return QG_OK;
}

MemoKey memo_key(const Problem& p, const qg_workspace* ws) {
  MemoKey k;
  memset(&k, 0, sizeof k);
  k.M = p.M, k.N = p.N, k.K = p.K;
  k.ta = p.ta, k.tb = p.tb, k.tc = p.tc, k.td = p.td, k.qa = p.qa, k.qb = p.qb;
  k.E = p.E, k.batched = p.batched, k.epi = p.epi;
  const bool ws_ok = ws && ws->partials && ws->barriers;
  k.ws_partials = ws_ok ? ws->partials_size : 0;
  k.ws_barriers = ws_ok ? ws->barriers_size : 0;
  return k;
}

constexpr size_t kMemoMax = 4096;

// Resolves the plan for a run (shared by qg_run and qg_plan).
int resolve(qg_handle* h, const qg_operation* op, const Problem& p, const qg_workspace* ws, Plan& pl,
            bool allow_measure, hipStream_t s) {
  Choice c;
  switch (op->policy) {
    case QG_POLICY_FORCE: {
      int fmode = -1;
      if (op->schedule == QG_SCHED_DP) fmode = MODE_DP;
      else if (op->schedule == QG_SCHED_SPLITK) fmode = MODE_SPLITK;
      else if (op->schedule == QG_SCHED_STREAMK) fmode = MODE_STREAMK;
      else if (op->schedule != QG_SCHED_AUTO) return QG_ERR_INVALID_ARG;
      c = heuristic(h, p, ws, fmode, op->split_k);
      if (op->kernel >= 0) c.kernel = op->kernel;
      if (fmode >= 0) c.mode = fmode;
      if (op->split_k > 0) c.split = op->split_k;
      if (c.mode == MODE_SPLITK && op->split_k <= 0 && c.split <= 1) c.split = 2;
      c.programs = op->programs;
      if (op->split_k < 0 || op->programs < 0) return QG_ERR_INVALID_ARG;
      return make_plan(h, p, c, ws, pl);
    }
    case QG_POLICY_REUSE:
      if (!lookup(h, p, c, false)) return QG_ERR_NO_KERNEL;
      return make_plan(h, p, c, ws, pl);
    case QG_POLICY_MEASURE:
      if (allow_measure && !lookup(h, p, c, true)) {
        // Measuring synchronises the stream, which a stream being captured
        // into a graph does not allow: while capturing, resolve as DEFAULT
        // (cache, else heuristic) and leave the measurement to a later call.
        hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
        if (hipStreamIsCapturing(s, &cs) != hipSuccess) {
          (void)hipGetLastError();
          return QG_ERR_HIP;
        }
        if (cs == hipStreamCaptureStatusNone) {
          int st = measure(h, p, ws, s, c);
          if (st != QG_OK) return st;
          return make_plan(h, p, c, ws, pl);
        }
      }
      // fallthrough
    case QG_POLICY_DEFAULT: {
      const MemoKey mk = memo_key(p, ws);
      bool hit = false;
      {
        std::lock_guard<std::mutex> g(h->mu);
        auto it = h->memo.find(mk);
        if (it != h->memo.end()) {
          c = it->second;
          hit = true;
        }
      }
      if (hit && make_plan(h, p, c, ws, pl) == QG_OK) return QG_OK;
      if (!(lookup(h, p, c, false) && make_plan(h, p, c, ws, pl) == QG_OK)) {
        c = heuristic(h, p, ws);
        if (c.kernel < 0) return QG_ERR_NO_KERNEL;
        const int st = make_plan(h, p, c, ws, pl);
        if (st != QG_OK) return st;
      }
      std::lock_guard<std::mutex> g(h->mu);
      if (h->memo.size() >= kMemoMax) h->memo.clear();
      h->memo[mk] = c;
      return QG_OK;
    }
    default:
      return QG_ERR_INVALID_ARG;
  }
}

bool log_enabled() {
  static int v = -1;
  if (v < 0) {
    const char* e = getenv("QG_LOG");
    v = (e && *e && strcmp(e, "0") != 0) ? 1 : 0;
  }
  return v == 1;
}

}  // namespace

// ============================================================================
// C ABI
// ============================================================================
extern "C" {

int qg_create(qg_handle** out) {
  if (!out) return QG_ERR_INVALID_ARG;
  *out = nullptr;
  qg_handle* h = new (std::nothrow) qg_handle();
  if (!h) return QG_ERR_HIP;
  int dev = -1, n = 0;
  if (hipGetDeviceCount(&n) == hipSuccess && n > 0 && hipGetDevice(&dev) == hipSuccess) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) == hipSuccess) {
      h->device = dev;
      h->cus = prop.multiProcessorCount;
      std::string arch = prop.gcnArchName;
      h->arch = arch.substr(0, arch.find(':'));
      h->online = true;
      if (h->arch != "gfx950") {
        delete h;
        return QG_ERR_UNSUPPORTED;
      }
    }
  }
  (void)hipGetLastError();
  *out = h;
  return QG_OK;
}

int qg_destroy(qg_handle* h) {
  if (!h) return QG_ERR_INVALID_ARG;
  delete h;
  return QG_OK;
}

size_t qg_barriers_size(void) { return kBarriersSize; }
size_t qg_partials_size(void) { return kPartialsSize; }

int qg_run(qg_handle* h, const qg_operation* op, float alpha, const void* A, const qg_layout* Adesc, const void* U,
           const qg_layout* Udesc, const void* B, const qg_layout* Bdesc, const void* V, const qg_layout* Vdesc,
           float beta, const void* C, const qg_layout* Cdesc, void* D, const qg_layout* Ddesc, const qg_workspace* ws,
           hipStream_t stream) {
  if (!h) return QG_ERR_INVALID_ARG;
  Problem p;
  int st = validate(op, alpha, A, Adesc, U, Udesc, B, Bdesc, V, Vdesc, beta, C, Cdesc, D, Ddesc, p);
  if (st != QG_OK) return st;
  if (p.M == 0 || p.N == 0) return QG_OK;
  Plan pl;
  st = resolve(h, op, p, ws, pl, h->online, stream);
  if (st != QG_OK) return st;
  if (log_enabled()) fprintf(stderr, "[qgemm] m=%lld %s %s\n", (long long)p.M, p.key().c_str(), describe(pl).c_str());
  if (!h->online) return QG_ERR_HIP;
  return launch(pl, stream);
}

int qg_run_timed(qg_handle* h, const qg_operation* op, float alpha, const void* A, const qg_layout* Adesc,
                 const void* U, const qg_layout* Udesc, const void* B, const qg_layout* Bdesc, const void* V,
                 const qg_layout* Vdesc, float beta, const void* C, const qg_layout* Cdesc, void* D,
                 const qg_layout* Ddesc, const qg_workspace* ws, hipStream_t stream, uint64_t* stamps,
                 int64_t units_cap, int64_t* units) {
  if (!h || !op) return QG_ERR_INVALID_ARG;
  if (units) *units = 0;
  // measuring creates events and synchronises; the timeline is of one launch
  if (op->policy == QG_POLICY_MEASURE) return QG_ERR_UNSUPPORTED;
  Problem p;
  int st = validate(op, alpha, A, Adesc, U, Udesc, B, Bdesc, V, Vdesc, beta, C, Cdesc, D, Ddesc, p);
  if (st != QG_OK) return st;
  if (p.M == 0 || p.N == 0) return QG_ERR_UNSUPPORTED;  // nothing is launched, nothing to time
  Plan pl;
  st = resolve(h, op, p, ws, pl, h->online, stream);
  if (st != QG_OK) return st;
  if (pl.a.mode != MODE_SPLITK && pl.a.mode != MODE_DP) return QG_ERR_UNSUPPORTED;
  const int64_t n = (int64_t)pl.a.tiles_m * pl.a.tiles_n * (pl.a.mode == MODE_SPLITK ? pl.a.splits : 1);
  if (units) *units = n;
  if (!stamps || (uintptr_t)stamps % 8 != 0 || units_cap < n) return QG_ERR_INVALID_ARG;
  pl.a.stamps = stamps;
  if (!h->online) return QG_ERR_HIP;
  return launch(pl, stream);
}

int qg_plan(qg_handle* h, const qg_operation* op, const qg_layout* Adesc, const qg_layout* Udesc,
            const qg_layout* Bdesc, const qg_layout* Vdesc, const qg_layout* Cdesc, const qg_layout* Ddesc, float alpha,
            float beta, const qg_workspace* ws, char* desc, size_t cap) {
  if (!h || !desc || cap == 0) return QG_ERR_INVALID_ARG;
  desc[0] = 0;
  // placeholder (non-null, aligned) device addresses: qg_plan never dereferences them
  const void* dummy = reinterpret_cast<const void*>(uintptr_t(1) << 20);
  Problem p;
  int st = validate(op, alpha, dummy, Adesc, Udesc ? dummy : nullptr, Udesc, dummy, Bdesc, Vdesc ? dummy : nullptr,
                    Vdesc, beta, Cdesc ? dummy : nullptr, Cdesc, const_cast<void*>(dummy), Ddesc, p);
  if (st != QG_OK) return st;
  if (p.M == 0 || p.N == 0) {
    snprintf(desc, cap, "kernel=none schedule=none split=0 programs=0 tiles=0 grid=0 partials=0 barriers=0 bm=0 bn=0 bk=0");
    return QG_OK;
  }
  Plan pl;
  st = resolve(h, op, p, ws, pl, false, nullptr);
  if (st != QG_OK) return st;
  std::string d = describe(pl);
  if (d.size() + 1 > cap) return QG_ERR_BUFFER_SMALL;
  memcpy(desc, d.c_str(), d.size() + 1);
  return QG_OK;
}

int qg_export(qg_handle* h, char* buf, size_t cap, size_t* len) {
  if (!h || !len) return QG_ERR_INVALID_ARG;
  std::ostringstream os;
  {
    std::lock_guard<std::mutex> g(h->mu);
    os << "qgemm-cache 2 arch=" << h->arch << " entries=" << h->cache.size() << "\n";
    for (auto& kv : h->cache) {
      const Entry& e = kv.second;
      char line[256];
      snprintf(line, sizeof line, " kernel=%s schedule=%s split=%d programs=%d us=%.9g\n", kKernels[e.c.kernel].name,
               sched_name(e.c.mode), e.c.split, e.c.programs, e.us);
      os << kv.first << line;
    }
  }
  const std::string s = os.str();
  *len = s.size() + 1;
  if (!buf) return QG_OK;
  if (cap < s.size() + 1) return QG_ERR_BUFFER_SMALL;
  memcpy(buf, s.c_str(), s.size() + 1);
  return QG_OK;
}

int qg_import(qg_handle* h, const char* buf, size_t len) {
  if (!h || (!buf && len)) return QG_ERR_INVALID_ARG;
  std::string text(buf ? buf : "", buf ? strnlen(buf, len) : 0);
  std::istringstream is(text);
  std::string line;
  if (!std::getline(is, line)) return QG_ERR_FORMAT;
  {
    std::istringstream hs(line);
    std::string magic, ver, arch, entries;
    hs >> magic >> ver >> arch >> entries;
    if (magic != "qgemm-cache" || ver != "2") return QG_ERR_FORMAT;  // version 2: keys carry the epilogue flags
    if (arch != "arch=" + h->arch) return QG_ERR_FORMAT;
    if (entries.rfind("entries=", 0) != 0) return QG_ERR_FORMAT;
    long n = strtol(entries.c_str() + 8, nullptr, 10);
    if (n < 0) return QG_ERR_FORMAT;
    std::map<std::string, Entry> staged;
    long got = 0;
    while (std::getline(is, line)) {
      if (line.empty()) continue;
      std::istringstream ls(line);
      std::string key, kk, sk, spk, pk, uk, extra;
      if (!(ls >> key >> kk >> sk >> spk >> pk >> uk) || (ls >> extra)) return QG_ERR_FORMAT;
      if (key.find('|') == std::string::npos) return QG_ERR_FORMAT;
      if (kk.rfind("kernel=", 0) || sk.rfind("schedule=", 0) || spk.rfind("split=", 0) || pk.rfind("programs=", 0) ||
          uk.rfind("us=", 0))
        return QG_ERR_FORMAT;
      Entry e;
      e.c.kernel = find_kernel(kk.c_str() + 7);
      e.c.mode = sched_from_name(sk.substr(9));
      char* end = nullptr;
      e.c.split = (int)strtol(spk.c_str() + 6, &end, 10);
      if (*end) return QG_ERR_FORMAT;
      e.c.programs = (int)strtol(pk.c_str() + 9, &end, 10);
      if (*end) return QG_ERR_FORMAT;
      e.us = strtod(uk.c_str() + 3, &end);
      if (*end) return QG_ERR_FORMAT;
      if (e.c.kernel < 0 || e.c.mode < 0 || e.c.split < 1 || e.c.programs < 0) return QG_ERR_FORMAT;
      if (!std::isfinite(e.us) || e.us < 0) return QG_ERR_FORMAT;
      staged[key] = e;
      ++got;
    }
    if (got != n) return QG_ERR_FORMAT;
    std::lock_guard<std::mutex> g(h->mu);
    for (auto& kv : staged) h->cache[kv.first] = kv.second;
    h->memo.clear();
  }
  return QG_OK;
}

int qg_get_tuning_seq(qg_handle* h, int* out, int cap, int* count) {
  if (!h || !count || cap < 0 || (cap > 0 && !out)) return QG_ERR_INVALID_ARG;
  const int n = (int)(sizeof(kTuningSeq) / sizeof(kTuningSeq[0]));
  for (int i = 0; i < n && i < cap; ++i) out[i] = kTuningSeq[i];
  *count = n;
  return QG_OK;
}

int qg_cache_size(qg_handle* h, int* count) {
  if (!h || !count) return QG_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> g(h->mu);
  *count = (int)h->cache.size();
  return QG_OK;
}

int qg_streamk_units(int tiles, int iters, int programs, int32_t* rows, int cap, int* count) {
  if (tiles < 0 || iters < 1 || programs < 1 || cap < 0 || !count || (cap > 0 && !rows)) return QG_ERR_INVALID_ARG;
  if (programs > kStreamKMaxPrograms || (int64_t)tiles * iters > INT32_MAX) return QG_ERR_UNSUPPORTED;
  const StreamK sk = StreamK::make(tiles, iters, programs);
  int n = 0;
  for (int p = 0; p < programs; ++p) {
    StreamKCursor cur(sk, p);
    int t, kb, ke, slot;
    while (cur.next(t, kb, ke, slot)) {
      if (n < cap) {
        int32_t* r = rows + 5 * (int64_t)n;
        r[0] = p, r[1] = t, r[2] = kb, r[3] = ke, r[4] = slot;
      }
      ++n;
    }
  }
  *count = n;
  return n > cap ? QG_ERR_BUFFER_SMALL : QG_OK;
}

int qg_streamk_fixup(int tiles, int iters, int programs, int tile, int32_t* slots, int cap, int* count) {
  if (tiles < 1 || iters < 1 || programs < 1 || tile < 0 || tile >= tiles || cap < 0 || !count ||
      (cap > 0 && !slots))
    return QG_ERR_INVALID_ARG;
  if (programs > kStreamKMaxPrograms || (int64_t)tiles * iters > INT32_MAX) return QG_ERR_UNSUPPORTED;
  const StreamK sk = StreamK::make(tiles, iters, programs);
  if (tile < sk.dp_tiles) {
    *count = 0;
    return QG_OK;
  }
  const int w0 = (tile - sk.dp_tiles) * iters;
  const int n = sk.pieces(w0);
  for (int i = 0; i < n && i < cap; ++i) slots[i] = sk.piece_slot(w0, i);
  *count = n;
  return n > cap ? QG_ERR_BUFFER_SMALL : QG_OK;
}

int qg_kernel_count(void) { return kNumKernels; }

const char* qg_kernel_name(int index) { return (index >= 0 && index < kNumKernels) ? kKernels[index].name : nullptr; }

const char* qg_status_str(int status) {
  switch (status) {
    case QG_OK: return "ok";
    case QG_ERR_INVALID_ARG: return "invalid argument";
    case QG_ERR_UNSUPPORTED: return "unsupported";
    case QG_ERR_ALIGNMENT: return "misaligned pointer or row pitch";
    case QG_ERR_WORKSPACE: return "workspace missing or too small";
    case QG_ERR_NO_KERNEL: return "no kernel";
    case QG_ERR_HIP: return "HIP runtime error";
    case QG_ERR_FORMAT: return "malformed cache text";
    case QG_ERR_BUFFER_SMALL: return "buffer too small";
    default: return "unknown status";
  }
}

const char* qg_version(void) { return kVersion; }

}  // extern "C"
