// Host-side exerciser of libqgemm's C ABI for AddressSanitizer /
// UndefinedBehaviorSanitizer builds (host code instrumented, GPU code not).
// It runs on a machine without a GPU: the handle is then offline, so every
// qg_run stops at validation or before its launch, while planning, the
// dispatch cache (export / import of untrusted text) and the stream-K
// introspection run in full. Exit status 0 when every expectation held; a
// sanitizer report aborts the run.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include <hip/hip_runtime_api.h>

#include "../../include/qgemm.h"

namespace {

int g_fail = 0;
#define EXPECT(c)                                                          \
  do {                                                                     \
    if (!(c)) {                                                            \
      std::fprintf(stderr, "FAIL %s:%d: %s\n", __FILE__, __LINE__, #c);   \
      ++g_fail;                                                            \
    }                                                                      \
  } while (0)

// never dereferenced: offline runs and qg_plan do not touch device memory
const void* const kFake = reinterpret_cast<const void*>(uintptr_t(1) << 20);

qg_layout lay(int t, int64_t rows, int64_t cols, int64_t ld = -1, int num = 0, const int32_t* off = nullptr,
              int64_t stride = 0) {
  qg_layout l;
  std::memset(&l, 0, sizeof l);
  l.type = t;
  l.order = QG_ROW_MAJOR;
  l.rows = rows;
  l.cols = cols;
  l.ld = ld >= 0 ? ld : (t == QG_U4 ? cols / 8 : cols);
  l.num = num;
  l.offsets = off;
  l.stride = stride;
  return l;
}

qg_operation opn(int policy = QG_POLICY_DEFAULT, int sched = QG_SCHED_AUTO, int split = 0, int programs = 0,
                 int kernel = -1) {
  qg_operation o;
  std::memset(&o, 0, sizeof o);
  o.policy = policy;
  o.schedule = sched;
  o.split_k = split;
  o.programs = programs;
  o.kernel = kernel;
  return o;
}

qg_workspace ws_full() {
  qg_workspace w;
  w.barriers = const_cast<void*>(kFake);
  w.barriers_size = qg_barriers_size();
  w.partials = const_cast<void*>(kFake);
  w.partials_size = qg_partials_size();
  return w;
}

// qg_plan into buffers of every small size and a large one; the text must
// always be NUL-terminated within the buffer.
int plan_all_caps(qg_handle* h, const qg_operation& op, const qg_layout* A, const qg_layout* U, const qg_layout* B,
                  const qg_layout* V, const qg_layout* C, const qg_layout* D, float alpha, float beta,
                  const qg_workspace* ws) {
  char big[512];
  const int st = qg_plan(h, &op, A, U, B, V, C, D, alpha, beta, ws, big, sizeof big);
  if (st == QG_OK) EXPECT(std::strlen(big) < sizeof big);
  for (size_t cap = 1; cap < 24; cap += 5) {
    std::vector<char> buf(cap, 'x');
    qg_plan(h, &op, A, U, B, V, C, D, alpha, beta, ws, buf.data(), cap);
    EXPECT(std::memchr(buf.data(), 0, cap) != nullptr);
  }
  return st;
}

void dense_plans(qg_handle* h) {
  const qg_workspace ws = ws_full();
  const int64_t shapes[][3] = {{1, 1, 8},      {1, 130, 520},    {16, 4096, 14336}, {300, 200, 136},
                               {4096, 4096, 4096}, {257, 513, 264}, {5, 77, 6},       {1 << 20, 8, 8}};
  const int types[][3] = {{QG_BF16, QG_BF16, QG_F32}, {QG_F16, QG_F16, QG_F16}, {QG_I8, QG_I8, QG_I32}};
  const int n_kernels = qg_kernel_count();
  for (auto& s : shapes)
    for (auto& t : types) {
      const int64_t M = s[0], N = s[1], K = s[2];
      const int64_t ldk = (K + 15) / 16 * 16;  // 16-byte rows for every element size
      const qg_layout A = lay(t[0], M, K, ldk), B = lay(t[1], N, K, ldk);
      const qg_layout D = lay(t[2], M, N, (N + 15) / 16 * 16);
      const qg_layout C = lay(t[2], M, N, (N + 15) / 16 * 16);
      const float beta = t[0] == QG_I8 ? 1.f : 0.5f;
      const int scheds[] = {QG_SCHED_AUTO, QG_SCHED_DP, QG_SCHED_SPLITK, QG_SCHED_STREAMK};
      for (int sc : scheds)
        for (int split : {0, 1, 3, 8, 1000000})
          for (int prog : {0, 1, 7, 256, 65535, 65536}) {
            const qg_operation op = opn(sc == QG_SCHED_AUTO ? QG_POLICY_DEFAULT : QG_POLICY_FORCE, sc, split, prog);
            plan_all_caps(h, op, &A, nullptr, &B, nullptr, &C, &D, 1.f, beta, &ws);
            plan_all_caps(h, op, &A, nullptr, &B, nullptr, nullptr, &D, 1.f, 0.f, nullptr);
          }
      for (int k = -1; k <= n_kernels; ++k) {
        const qg_operation op = opn(QG_POLICY_FORCE, QG_SCHED_SPLITK, 2, 0, k);
        plan_all_caps(h, op, &A, nullptr, &B, nullptr, &C, &D, 1.f, beta, &ws);
      }
      // offline: a valid run stops before its launch
      const qg_operation op = opn();
      const int st = qg_run(h, &op, 1.f, kFake, &A, nullptr, nullptr, kFake, &B, nullptr, nullptr, beta, kFake, &C,
                            const_cast<void*>(kFake), &D, &ws, nullptr);
      EXPECT(st != QG_OK);
      const int st2 = qg_run_noalloc(h, &op, 1.f, kFake, &A, nullptr, nullptr, kFake, &B, nullptr, nullptr, beta,
                                     kFake, &C, const_cast<void*>(kFake), &D, nullptr);
      EXPECT(st2 != QG_OK);
      // the timed run: every schedule and split, short, missing and
      // misaligned stamp buffers (offline, nothing is launched)
      uint64_t* stamps = reinterpret_cast<uint64_t*>(const_cast<void*>(kFake));
      for (int sc : scheds)
        for (int split : {0, 1, 3, 8, 1000000}) {
          const qg_operation top = opn(sc == QG_SCHED_AUTO ? QG_POLICY_DEFAULT : QG_POLICY_FORCE, sc, split, 7);
          for (int64_t cap : {int64_t(-1), int64_t(0), int64_t(1), int64_t(1) << 40}) {
            int64_t units = -5;
            const int st3 = qg_run_timed(h, &top, 1.f, kFake, &A, nullptr, nullptr, kFake, &B, nullptr, nullptr, beta,
                                         kFake, &C, const_cast<void*>(kFake), &D, &ws, nullptr, stamps, cap, &units);
            EXPECT(st3 != QG_OK && units >= 0);
            EXPECT(qg_run_timed(h, &top, 1.f, kFake, &A, nullptr, nullptr, kFake, &B, nullptr, nullptr, beta, kFake,
                                &C, const_cast<void*>(kFake), &D, &ws, nullptr, nullptr, cap, nullptr) != QG_OK);
            EXPECT(qg_run_timed(h, &top, 1.f, kFake, &A, nullptr, nullptr, kFake, &B, nullptr, nullptr, beta, kFake,
                                &C, const_cast<void*>(kFake), &D, &ws, nullptr,
                                reinterpret_cast<uint64_t*>(reinterpret_cast<uintptr_t>(kFake) + 4), cap,
                                &units) != QG_OK);
          }
        }
    }
}

void quantised_and_grouped_plans(qg_handle* h) {
  const qg_workspace ws = ws_full();
  char buf[512];
  // int4 weights, symmetric and asymmetric
  for (int64_t M : {1, 16, 64, 100}) {
    const int64_t N = 8192, K = 8192;
    qg_operation op = opn();
    op.quant_b.kind = QG_QUANT_INT4_ZP;
    op.quant_b.group_k = 128;
    op.quant_b.group_mn = 1;
    op.quant_b.zero_point = 8;
    const qg_layout A = lay(QG_BF16, M, K), B = lay(QG_U4, N, K), V = lay(QG_F16, N, K / 128, 64);
    const qg_layout U = lay(QG_I8, N, K / 128, 64), D = lay(QG_BF16, M, N);
    EXPECT(qg_plan(h, &op, &A, nullptr, &B, &V, nullptr, &D, 1.f, 0.f, &ws, buf, sizeof buf) == QG_OK);
    EXPECT(qg_plan(h, &op, &A, &U, &B, &V, nullptr, &D, 1.f, 0.f, &ws, buf, sizeof buf) == QG_OK);
    op.quant_b.group_k = 64;
    EXPECT(qg_plan(h, &op, &A, nullptr, &B, &V, nullptr, &D, 1.f, 0.f, &ws, buf, sizeof buf) != QG_OK);
  }
  // block-scaled fp8, plain and grouped; a grouped problem reads its offsets
  // only on the device, so fake ones suffice here
  {
    const int64_t M = 65536, N = 2048, K = 7168, E = 64;
    qg_operation op = opn();
    op.quant_a = {QG_QUANT_BLOCK_F32, 128, 1, 0};
    op.quant_b = {QG_QUANT_BLOCK_F32, 128, 128, 0};
    const auto off = static_cast<const int32_t*>(kFake);
    const qg_layout A = lay(QG_E4M3, M, K, -1, E, off), B = lay(QG_E4M3, N, K, -1, E, nullptr, N * K);
    const qg_layout U = lay(QG_F32, M, K / 128, 56, E, off), V = lay(QG_F32, N / 128, K / 128, 56, E, nullptr, 16 * 56);
    const qg_layout D = lay(QG_BF16, M, N, -1, E, off);
    EXPECT(plan_all_caps(h, op, &A, &U, &B, &V, nullptr, &D, 1.f, 0.f, &ws) == QG_OK);
    const qg_layout A1 = lay(QG_E4M3, 200, 1001, 1008), B1 = lay(QG_E4M3, 300, 1001, 1008);
    const qg_layout U1 = lay(QG_F32, 200, 8, 8), V1 = lay(QG_F32, 3, 8, 8), D1 = lay(QG_BF16, 200, 300, 304);
    EXPECT(plan_all_caps(h, op, &A1, &U1, &B1, &V1, nullptr, &D1, 1.f, 0.f, &ws) == QG_OK);
  }
  // grouped and batched bf16
  {
    const auto off = static_cast<const int32_t*>(kFake);
    const qg_layout A = lay(QG_BF16, 65536, 7168, -1, 64, off), B = lay(QG_BF16, 2048, 7168, -1, 64, nullptr, 0);
    const qg_layout D = lay(QG_BF16, 65536, 2048, -1, 64, off);
    EXPECT(plan_all_caps(h, opn(), &A, nullptr, &B, nullptr, nullptr, &D, 1.f, 0.f, &ws) == QG_OK);
    const qg_layout Ab = lay(QG_BF16, 33, 72, -1, 5, nullptr, 33 * 72), Bb = lay(QG_BF16, 40, 72, -1, 5, nullptr, 40 * 72);
    const qg_layout Db = lay(QG_F32, 33, 40, -1, 5, nullptr, 33 * 40);
    EXPECT(plan_all_caps(h, opn(), &Ab, nullptr, &Bb, nullptr, nullptr, &Db, 1.f, 0.f, &ws) == QG_OK);
    // too many experts, inconsistent counts
    const qg_layout Abad = lay(QG_BF16, 100, 64, -1, 5000, off), Bbad = lay(QG_BF16, 64, 64, -1, 5000);
    const qg_operation dflt = opn();
    EXPECT(qg_plan(h, &dflt, &Abad, nullptr, &Bbad, nullptr, nullptr, &D, 1.f, 0.f, &ws, buf, sizeof buf) != QG_OK);
  }
}

void invalid_requests(qg_handle* h) {
  const qg_workspace ws = ws_full();
  const qg_layout A = lay(QG_BF16, 64, 64), B = lay(QG_BF16, 64, 64), D = lay(QG_BF16, 64, 64);
  const qg_operation op = opn();
  void* Dp = const_cast<void*>(kFake);
  auto run = [&](const qg_operation* o, const void* a, const qg_layout* Ad, const qg_layout* Bd, const qg_layout* Dd,
                 float beta, const qg_layout* Cd, const qg_workspace* w) {
    return qg_run(h, o, 1.f, a, Ad, nullptr, nullptr, kFake, Bd, nullptr, nullptr, beta, Cd ? kFake : nullptr, Cd,
                  Dp, Dd, w, nullptr);
  };
  EXPECT(run(nullptr, kFake, &A, &B, &D, 0.f, nullptr, &ws) == QG_ERR_INVALID_ARG);
  EXPECT(run(&op, nullptr, &A, &B, &D, 0.f, nullptr, &ws) == QG_ERR_INVALID_ARG);
  EXPECT(run(&op, kFake, nullptr, &B, &D, 0.f, nullptr, &ws) == QG_ERR_INVALID_ARG);
  EXPECT(run(&op, static_cast<const char*>(kFake) + 2, &A, &B, &D, 0.f, nullptr, &ws) == QG_ERR_ALIGNMENT);
  for (int t : {-5, -1, 7, 99}) {
    const qg_layout bad = lay(t, 64, 64);
    EXPECT(run(&op, kFake, &bad, &B, &D, 0.f, nullptr, &ws) != QG_OK);
  }
  for (int64_t r : {int64_t(-1), int64_t(1) << 40, INT64_MIN, INT64_MAX}) {
    const qg_layout bad = lay(QG_BF16, r, 64);
    EXPECT(run(&op, kFake, &bad, &B, &D, 0.f, nullptr, &ws) != QG_OK);
    const qg_layout badk = lay(QG_BF16, 64, r, r);
    EXPECT(run(&op, kFake, &badk, &B, &D, 0.f, nullptr, &ws) != QG_OK);
    const qg_layout badld = lay(QG_BF16, 64, 64, r);
    EXPECT(run(&op, kFake, &badld, &B, &D, 0.f, nullptr, &ws) != QG_OK);
  }
  const qg_layout Cw = lay(QG_F32, 64, 63);
  EXPECT(run(&op, kFake, &A, &B, &D, 1.f, &Cw, &ws) != QG_OK);
  EXPECT(run(&op, kFake, &A, &B, &D, 1.f, nullptr, &ws) == QG_ERR_INVALID_ARG);
  qg_operation bad_policy = opn(17);
  EXPECT(run(&bad_policy, kFake, &A, &B, &D, 0.f, nullptr, &ws) == QG_ERR_INVALID_ARG);
  qg_operation bad_sched = opn(QG_POLICY_FORCE, 9);
  EXPECT(run(&bad_sched, kFake, &A, &B, &D, 0.f, nullptr, &ws) != QG_OK);
  qg_operation bad_epi = opn();
  bad_epi.epilogue = 0x7fffffff;
  EXPECT(run(&bad_epi, kFake, &A, &B, &D, 0.f, nullptr, &ws) == QG_ERR_INVALID_ARG);
  const float nan = std::strtof("nan", nullptr);
  EXPECT(qg_run(h, &op, nan, kFake, &A, nullptr, nullptr, kFake, &B, nullptr, nullptr, 0.f, nullptr, nullptr, Dp, &D,
                &ws, nullptr) == QG_ERR_INVALID_ARG);
  // a workspace too small for a forced split
  qg_workspace tiny = ws_full();
  tiny.partials_size = 16;
  const qg_layout Ak = lay(QG_BF16, 16, 14336), Bk = lay(QG_BF16, 4096, 14336), Dk = lay(QG_BF16, 16, 4096);
  const qg_operation split8 = opn(QG_POLICY_FORCE, QG_SCHED_SPLITK, 8);
  EXPECT(run(&split8, kFake, &Ak, &Bk, &Dk, 0.f, nullptr, &tiny) == QG_ERR_WORKSPACE);
  EXPECT(qg_run(nullptr, &op, 1.f, kFake, &A, nullptr, nullptr, kFake, &B, nullptr, nullptr, 0.f, nullptr, nullptr,
                Dp, &D, &ws, nullptr) == QG_ERR_INVALID_ARG);
  int64_t units = 0;
  EXPECT(qg_run_timed(nullptr, &op, 1.f, kFake, &A, nullptr, nullptr, kFake, &B, nullptr, nullptr, 0.f, nullptr,
                      nullptr, Dp, &D, &ws, nullptr, nullptr, 0, &units) == QG_ERR_INVALID_ARG);
  EXPECT(qg_run_timed(h, nullptr, 1.f, kFake, &A, nullptr, nullptr, kFake, &B, nullptr, nullptr, 0.f, nullptr,
                      nullptr, Dp, &D, &ws, nullptr, nullptr, 0, &units) == QG_ERR_INVALID_ARG);
}

// xorshift64*: a fixed pseudo-random sequence for the import fuzzing
uint64_t g_rng = 0x9E3779B97F4A7C15ull;
uint64_t rnd() {
  g_rng ^= g_rng >> 12;
  g_rng ^= g_rng << 25;
  g_rng ^= g_rng >> 27;
  return g_rng * 2685821657736338717ull;
}

void cache_text(qg_handle* h) {
  int count = -1;
  EXPECT(qg_cache_size(h, &count) == QG_OK && count == 0);
  size_t len = 0;
  EXPECT(qg_export(h, nullptr, 0, &len) == QG_OK && len > 0);
  std::vector<char> out(len);
  EXPECT(qg_export(h, out.data(), len, &len) == QG_OK);
  EXPECT(qg_export(h, out.data(), len - 1, &len) == QG_ERR_BUFFER_SMALL);
  // entries naming real kernels and problem keys, with extreme split and
  // program counts that later plans must refuse or clamp
  std::string text = "qgemm-cache 2 arch=gfx950 entries=6\n";
  const char* k0 = qg_kernel_name(0);
  const char* kl = qg_kernel_name(qg_kernel_count() - 1);
  text += std::string("16|bf16.bf16.bf16.bf16.q00.e0.x0.n4096.k14336 kernel=") + k0 +
          " schedule=splitk split=2147483647 programs=0 us=1.5\n";
  text += std::string("4096|bf16.bf16.-.bf16.q00.e0.x0.n4096.k4096 kernel=") + k0 +
          " schedule=streamk split=1 programs=2147483647 us=100\n";
  text += std::string("64|bf16.u4.-.bf16.q01.e0.x0.n8192.k8192 kernel=") + kl +
          " schedule=dp split=1 programs=0 us=1e308\n";
  text += std::string("1|bf16.bf16.bf16.bf16.q00.e0.x0.n4096.k14336 kernel=") + kl +
          " schedule=grouped split=1 programs=0 us=0.001\n";
  text += std::string("8192|i8.i8.i32.i32.q00.e0.x0.n4096.k4096 kernel=") + k0 +
          " schedule=dp split=65536 programs=65536 us=0\n";
  text += "|x kernel=" + std::string(k0) + " schedule=dp split=1 programs=0 us=0\n";
  EXPECT(qg_import(h, text.c_str(), text.size()) == QG_OK);
  EXPECT(qg_cache_size(h, &count) == QG_OK && count == 6);
  // times must be finite and non-negative; a refused text changes nothing
  for (const char* us : {"-5", "nan", "inf", "1e999", "0x1p3x"}) {
    const std::string t = std::string("qgemm-cache 2 arch=gfx950 entries=1\n2|k kernel=") + k0 +
                          " schedule=dp split=1 programs=0 us=" + us + "\n";
    EXPECT(qg_import(h, t.c_str(), t.size()) == QG_ERR_FORMAT);
  }
  EXPECT(qg_cache_size(h, &count) == QG_OK && count == 6);
  // every prefix of the valid text: accepted only when whole (or when the
  // cut falls after the last line's end), never a crash
  for (size_t cut = 0; cut < text.size(); ++cut) {
    std::vector<char> part(text.begin(), text.begin() + cut);
    qg_import(h, part.data(), part.size());
  }
  // mutations: random bytes overwritten, inserted, deleted
  for (int it = 0; it < 3000; ++it) {
    std::string m = text;
    const int edits = 1 + (int)(rnd() % 4);
    for (int e = 0; e < edits; ++e) {
      const size_t pos = rnd() % (m.size() + 1);
      switch (rnd() % 3) {
        case 0:
          if (pos < m.size()) m[pos] = (char)(rnd() & 0xff);
          break;
        case 1: m.insert(m.begin() + pos, (char)(rnd() & 0xff)); break;
        default:
          if (pos < m.size()) m.erase(m.begin() + pos);
      }
    }
    qg_import(h, m.data(), m.size());
  }
  // pure noise, long lines, huge numbers
  for (int it = 0; it < 200; ++it) {
    std::vector<char> noise(rnd() % 600);
    for (auto& c : noise) c = (char)(rnd() & 0xff);
    qg_import(h, noise.data(), noise.size());
  }
  const std::string longline = "qgemm-cache 2 arch=gfx950 entries=1\n" + std::string(100000, 'a') + "|b kernel=" + k0 +
                               " schedule=dp split=1 programs=0 us=1\n";
  qg_import(h, longline.c_str(), longline.size());
  const std::string huge = "qgemm-cache 2 arch=gfx950 entries=99999999999999999999999\n";
  EXPECT(qg_import(h, huge.c_str(), huge.size()) == QG_ERR_FORMAT);
  EXPECT(qg_import(h, nullptr, 5) == QG_ERR_INVALID_ARG);
  EXPECT(qg_import(h, nullptr, 0) == QG_ERR_FORMAT);
  // plans that hit the imported entries (exact M and tuning buckets)
  const qg_workspace ws = ws_full();
  char buf[512];
  for (int64_t M : {1, 2, 9, 16, 17, 64, 4096, 5000, 8192, 9000}) {
    const qg_layout A = lay(QG_BF16, M, 14336), B = lay(QG_BF16, 4096, 14336), D = lay(QG_BF16, M, 4096);
    const qg_layout C = lay(QG_BF16, M, 4096);
    for (int pol : {QG_POLICY_DEFAULT, QG_POLICY_REUSE}) {
      const qg_operation o = opn(pol);
      qg_plan(h, &o, &A, nullptr, &B, nullptr, &C, &D, 1.f, 1.f, &ws, buf, sizeof buf);
    }
    const qg_layout A2 = lay(QG_BF16, M, 4096), B2 = lay(QG_BF16, 4096, 4096), D2 = lay(QG_BF16, M, 4096);
    const qg_operation reuse = opn(QG_POLICY_REUSE);
    qg_plan(h, &reuse, &A2, nullptr, &B2, nullptr, nullptr, &D2, 1.f, 0.f, &ws, buf, sizeof buf);
  }
  // export of whatever the cache now holds, and a round trip
  EXPECT(qg_export(h, nullptr, 0, &len) == QG_OK);
  out.assign(len, 0);
  EXPECT(qg_export(h, out.data(), len, &len) == QG_OK);
  EXPECT(qg_import(h, out.data(), len) == QG_OK);
}

void introspection(qg_handle* h) {
  int count = 0;
  std::vector<int> seq(64);
  for (int cap = 0; cap < 30; ++cap) EXPECT(qg_get_tuning_seq(h, cap ? seq.data() : nullptr, cap, &count) == QG_OK);
  EXPECT(qg_get_tuning_seq(h, nullptr, 3, &count) == QG_ERR_INVALID_ARG);
  for (int t : {0, 1, 5, 32, 255, 256, 257, 1000})
    for (int it : {1, 2, 7, 64, 448})
      for (int p : {1, 3, 37, 256, 1000}) {
        int n = 0;
        qg_streamk_units(t, it, p, nullptr, 0, &n);
        std::vector<int32_t> rows(5 * (size_t)n + 5);
        EXPECT(qg_streamk_units(t, it, p, rows.data(), n, &n) == QG_OK);
        if (n > 1) EXPECT(qg_streamk_units(t, it, p, rows.data(), n - 1, &n) == QG_ERR_BUFFER_SMALL);
        for (int tile = 0; tile < t; tile += 1 + t / 7) {
          int m = 0;
          qg_streamk_fixup(t, it, p, tile, nullptr, 0, &m);
          std::vector<int32_t> s((size_t)m + 1);
          EXPECT(qg_streamk_fixup(t, it, p, tile, s.data(), m, &m) == QG_OK);
        }
      }
  EXPECT(qg_streamk_units(10, 1 << 30, 4, nullptr, 0, &count) == QG_ERR_UNSUPPORTED);
  EXPECT(qg_streamk_units(10, 4, 65536, nullptr, 0, &count) == QG_ERR_UNSUPPORTED);
  EXPECT(qg_streamk_fixup(10, 4, 3, 10, nullptr, 0, &count) == QG_ERR_INVALID_ARG);
  for (int s = -20; s <= 5; ++s) EXPECT(qg_status_str(s) != nullptr);
  EXPECT(qg_version() != nullptr);
  EXPECT(qg_kernel_name(-1) == nullptr && qg_kernel_name(qg_kernel_count()) == nullptr);
}

}  // namespace

int main() {
  // offline only: with a GPU visible, the valid runs below would launch on
  // placeholder addresses
  int devices = 0;
  if (hipGetDeviceCount(&devices) == hipSuccess && devices > 0) {
    std::printf("abi_asan: a GPU is visible; this program only runs without one\n");
    return 77;
  }
  qg_handle* h = nullptr;
  EXPECT(qg_create(&h) == QG_OK && h);
  if (!h) return 1;
  dense_plans(h);
  quantised_and_grouped_plans(h);
  invalid_requests(h);
  cache_text(h);
  introspection(h);
  EXPECT(qg_destroy(h) == QG_OK);
  EXPECT(qg_create(nullptr) == QG_ERR_INVALID_ARG);
  std::printf("abi_asan: %s (%d failed expectations)\n", g_fail ? "FAILED" : "ok", g_fail);
  return g_fail ? 1 : 0;
}
