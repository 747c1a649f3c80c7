/*
 * qgemm.h -- C ABI of libqgemm.so, a GEMM engine for AMD MI355X (gfx950).
 *
 * The engine computes
 *
 *     D = alpha * (A @ B) + beta * C
 *
 * with operands A, U, B, V, C, D, a caller-owned workspace and a stream, the
 * operation and argument order stated on the page "InternLM Lmdeploy Gemm
 * Interface" (Description; Signature of Gemm::Run; I/O Contract). U and V are
 * the optional quantisation scale operands of that contract; the group-wise
 * stepping of U/V along K follows the page "InternLM Lmdeploy Gemm
 * MainloopSm80V2" (Description, quantisation group tracking).
 *
 * Conventions used throughout
 *   - "B" is the operand stored N x K with K contiguous (row-major N x K), so
 *     (A @ B)(i, j) = sum_k A[i, k] * B[j, k]. A is M x K row-major; C and D
 *     are M x N row-major.
 *   - All matrix pointers are DEVICE pointers on the handle's device. Layout
 *     descriptors (qg_layout, qg_operation, qg_workspace) are HOST structs
 *     read during the call only; the engine keeps no reference to them.
 *   - Every call returns 0 on success (the page's "0 on success") or one of
 *     the negative qg_status codes below. qg_run enqueues work on `stream`
 *     and returns without synchronising; device faults surface at the
 *     caller's next synchronisation. It never allocates or frees device
 *     memory (the measure policy allocates nothing either; it synchronises).
 *   - Accumulation is fp32 for float inputs and exact int32 for int8.
 *   - Alignment: every device pointer and every row pitch (ld * element size)
 *     must be a multiple of 16 bytes. K need not be: a row of A or B is read
 *     in 16-byte chunks up to the first 16-byte boundary at or past its K-th
 *     element, which lies inside the row pitch (so the storage of the last
 *     row must reach that boundary; rows x ld elements always do). Whatever
 *     those bytes past K hold (NaN included) is zeroed on chip before use.
 *
 * Threading: one handle may be used from several host threads except under
 * QG_POLICY_MEASURE (which mutates the dispatch cache and synchronises the
 * stream). Runs that execute concurrently on the device need separate
 * workspaces.
 */
#ifndef QGEMM_H
#define QGEMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* hipStream_t, declared here so that the header needs no HIP include. */
typedef struct ihipStream_t* hipStream_t;

typedef struct qg_handle qg_handle;

/* ---- status codes ------------------------------------------------------ */
enum qg_status {
  QG_OK = 0,
  QG_ERR_INVALID_ARG = -1,  /* null handle/pointer, bad shape, inconsistent layouts */
  QG_ERR_UNSUPPORTED = -2,  /* valid request this engine does not implement */
  QG_ERR_ALIGNMENT = -3,    /* pointer or row pitch not 16-byte aligned */
  QG_ERR_WORKSPACE = -4,    /* workspace missing or too small for the plan */
  QG_ERR_NO_KERNEL = -5,    /* no registered kernel fits / REUSE policy missed the cache */
  QG_ERR_HIP = -6,          /* a HIP runtime call failed */
  QG_ERR_FORMAT = -7,       /* qg_import: malformed, truncated or foreign cache text */
  QG_ERR_BUFFER_SMALL = -8  /* output buffer too small (the needed size is reported) */
};

/* ---- element types ------------------------------------------------------ */
typedef enum qg_dtype {
  QG_F32 = 0,
  QG_F16 = 1,
  QG_BF16 = 2,
  QG_E4M3 = 3, /* OCP 8-bit float E4M3 ("fn": no infinities, max 448) */
  QG_I8 = 4,
  QG_I32 = 5,
  QG_U4 = 6    /* unsigned 4-bit, packed 8 per uint32: element k = 8w + i in
                  bits [4i, 4i+4) of word w of its row; ld counts words */
} qg_dtype;

typedef enum qg_order { QG_ROW_MAJOR = 0, QG_COL_MAJOR = 1 } qg_order;

/* Describes one operand ("MatrixLayout" of the Run signature).
 *   type, order  element type and storage order (only QG_ROW_MAJOR today).
 *   rows, cols   logical shape. A: M x K, B: N x K, C/D: M x N,
 *                U (fp8 A scales): ceil(M/group_mn) x ceil(K/group_k) fp32,
 *                U (int4 zero points): N x K/group_k int8 (values 0..15),
 *                V (int4 scales): N x ceil(K/group_k) fp16,
 *                V (fp8 B scales): ceil(N/group_mn) x ceil(K/group_k) fp32.
 *                For a grouped problem rows of A/C/D/U is the total row count
 *                and B/V give ONE group's shape.
 *   ld           leading dimension (elements; uint32 words for QG_U4).
 *   num          number of groups (MoE experts) or batches; 0 or 1 = plain GEMM.
 *   offsets      grouped A/C/D/U: DEVICE int32 array of num+1 row offsets,
 *                offsets[0] = 0, non-decreasing, offsets[num] <= rows; group e
 *                owns rows [offsets[e], offsets[e+1]). May be empty groups.
 *                NULL with num > 1 on A: a BATCHED problem (the batched
 *                variant of the TileLang tutorial "gemm_variants.py",
 *                gemm_batched): num batches of the same M x N x K shape; rows
 *                of A/C/D/U then give ONE batch and every operand carries num.
 *   stride       grouped / batched B/V: elements (words) from group e to group
 *                e+1, or 0 when all groups share one B (V). Batched A/C/D/U:
 *                must be rows * ld (batches stored back to back), else
 *                QG_ERR_UNSUPPORTED. */
typedef struct qg_layout {
  int32_t type;
  int32_t order;
  int64_t rows;
  int64_t cols;
  int64_t ld;
  int32_t num;
  int32_t reserved;
  const int32_t* offsets;
  int64_t stride;
} qg_layout;

/* ---- operation descriptor ("Dispatch policy, epilogue, quantization config") */
typedef enum qg_policy {
  QG_POLICY_DEFAULT = 0, /* cache hit (exact key, else nearest tuning bucket >= M), else heuristic */
  QG_POLICY_MEASURE = 1, /* as DEFAULT on a hit; on an exact-key miss time the candidates
                            on `stream` (synchronises), cache the fastest, then run it */
  QG_POLICY_REUSE = 2,   /* cache only: a miss returns QG_ERR_NO_KERNEL */
  QG_POLICY_FORCE = 3    /* use schedule / split_k / programs / kernel exactly as given */
} qg_policy;

/* Epilogue, applied to each output element once its sum is complete (the
 * fused GEMM + bias + activation and the fused output quantisation of the
 * DeepGEMM write-up, section 6). Flags combine; the steps run in this order:
 *   x = alpha * acc + beta * C[m, n]              (always)
 *   x = x + bias[n]                               QG_EPI_BIAS
 *   x = max(x, 0)                                 QG_EPI_RELU
 *   x = x * Phi(x) = 0.5 x (1 + erf(x / sqrt 2))  QG_EPI_GELU (exact erf form)
 *   D[m, n] = saturate_int8(round_half_even(x * row_scale[m] + zero_point))
 *                                                 QG_EPI_QUANT_I8 (D type QG_I8)
 * otherwise D[m, n] = x rounded (RNE) to D's type. RELU and GELU exclude each
 * other. The int8-input path (exact int32 results) takes no epilogue flags. */
typedef enum qg_epilogue {
  QG_EPI_ALPHA_BETA = 0,
  QG_EPI_BIAS = 1,
  QG_EPI_RELU = 2,
  QG_EPI_GELU = 4,
  QG_EPI_QUANT_I8 = 8
} qg_epilogue;

/* Operands of the epilogue flags (ignored when the flag is not set). */
typedef struct qg_epilogue_args {
  const void* bias;        /* DEVICE, N elements of bias_type (QG_F32, QG_BF16 or
                              QG_F16), one per column of D, 16-byte aligned */
  int32_t bias_type;
  int32_t reserved0;
  const float* row_scale;  /* DEVICE, one fp32 scale per row of D (grouped /
                              batched: per row of the whole A), 4-byte aligned */
  float zero_point;        /* added after scaling, before rounding */
  int32_t reserved1;
} qg_epilogue_args;

typedef enum qg_quant_kind {
  QG_QUANT_NONE = 0,
  QG_QUANT_INT4_ZP = 1,   /* B only: b = (q - zero_point) * V[n, k / group_k], V fp16;
                             with U given (asymmetric), zero_point = U[n, k / group_k],
                             U QG_I8 bytes (N x K/group_k, ld a multiple of 16) */
  QG_QUANT_BLOCK_F32 = 2  /* e4m3 A or B: value = code * scale of its (group_mn x group_k) block */
} qg_quant_kind;

typedef struct qg_quant {
  int32_t kind;      /* qg_quant_kind */
  int32_t group_k;   /* K extent of a scale group (128 for the kernels here) */
  int32_t group_mn;  /* M (for A) or N (for B) extent of a scale block; 1 = per row */
  int32_t zero_point;
} qg_quant;

typedef enum qg_schedule {
  QG_SCHED_AUTO = 0,
  QG_SCHED_DP = 1,       /* one workgroup per output tile, whole K */
  QG_SCHED_SPLITK = 2,   /* each tile's K cut into split_k contiguous chunks */
  QG_SCHED_STREAMK = 3   /* `programs` workgroups share the k-iterations evenly */
} qg_schedule;

typedef struct qg_operation {
  int32_t policy;    /* qg_policy */
  int32_t epilogue;  /* qg_epilogue flags */
  qg_quant quant_a;
  qg_quant quant_b;
  int32_t schedule;  /* qg_schedule (honoured under FORCE; a hint otherwise) */
  int32_t split_k;   /* SPLITK chunk count, 0 = engine's choice */
  int32_t programs;  /* STREAMK program count, 0 = number of compute units */
  int32_t kernel;    /* FORCE: registry index from qg_kernel_name, -1 = engine's choice */
  qg_epilogue_args epi;
} qg_operation;

/* Caller-owned workspace. `barriers` holds one int32 arrival counter per
 * output tile of a split run; it must be zeroed once by the caller before
 * first use, and every run leaves it zeroed again. `partials` holds fp32
 * (int32 for int8) partial tiles of split-K / stream-K segments. */
typedef struct qg_workspace {
  void* barriers;
  size_t barriers_size;
  void* partials;
  size_t partials_size;
} qg_workspace;

/* ---- lifetime ------------------------------------------------------------ */
/* Creates a handle bound to the HIP device current on the calling thread
 * ("created once per model/device"). It owns the kernel registry and the
 * dispatch cache; it holds no device memory. */
int qg_create(qg_handle** out);
int qg_destroy(qg_handle* h);

/* Workspace sizes the engine is built for (kBarriersSize, kPartialsSize of
 * the Gemm class): 1 MiB and 32 MiB. */
size_t qg_barriers_size(void);
size_t qg_partials_size(void);

/* ---- the GEMM ------------------------------------------------------------ */
/* Operand order and meaning follow Gemm::Run. U, V and C may be NULL when
 * unused (C only when beta == 0: then C is never read, so NaNs in it do not
 * propagate). alpha == 0 still reads A and B. Supported combinations:
 *   A, B bf16 | fp16            -> D f32 | bf16 | fp16, C f32 | bf16 | fp16
 *   A bf16, B u4 + V fp16 (QG_QUANT_INT4_ZP on B, group_k = 128), optional
 *     per-group zero points in U
 *   A, B e4m3 + U, V fp32 (QG_QUANT_BLOCK_F32 on both; A 1 x 128, B 128 x 128)
 *   A, B int8 -> D int32, C int32; alpha must be 1 and beta 0 or 1 (exact)
 *   A, B int8 + U, V fp32 (w8a8: QG_QUANT_BLOCK_F32 on both with group_mn = 1
 *     and group_k = 0 or >= K, i.e. one scale per row of A and per row of B;
 *     U is M x >=1, V is N x >=1, any ld >= 1, 4-byte aligned) -> the exact
 *     int32 sum times U[m] * V[n] in fp32, then the float epilogue; D f32 |
 *     bf16 | fp16 (or int8 codes), C f32 | bf16 | fp16; not grouped/batched
 *   float paths with QG_EPI_QUANT_I8 -> D int8
 *   any of these grouped over experts (Adesc.num = Bdesc.num = E, offsets),
 *   and all but int4 batched (num = batch count on every operand, no offsets).
 * Returns QG_ERR_* without launching on any invalid or unsupported request. */
int qg_run(qg_handle* h, const qg_operation* op, float alpha,
           const void* A, const qg_layout* Adesc,
           const void* U, const qg_layout* Udesc,
           const void* B, const qg_layout* Bdesc,
           const void* V, const qg_layout* Vdesc,
           float beta,
           const void* C, const qg_layout* Cdesc,
           void* D, const qg_layout* Ddesc,
           const qg_workspace* ws, hipStream_t stream);

/* qg_run without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation). The split-K / stream-K workspace is a device array
 * inside the library, one per GPU, held until the process ends:
 * qg_noalloc_barriers_size() bytes of arrival counters (64 KiB: 16384 split
 * tiles) and qg_noalloc_partials_size() bytes of partial tiles (16 MiB). The
 * first call on a device looks the array up and clears its counters on
 * `stream`; every run leaves them zero again. Arguments, plans and kernels
 * are those of qg_run (the heuristic sees the smaller workspace, so it may
 * pick a smaller split); a plan that needs more workspace than the array
 * holds returns QG_ERR_WORKSPACE, and QG_POLICY_MEASURE returns
 * QG_ERR_UNSUPPORTED (measuring creates events and synchronises). No device
 * memory is allocated or freed. All calls on one GPU share its array: calls
 * whose kernels may overlap on that GPU (other streams, other threads) race
 * and must be serialised by the caller. */
int qg_run_noalloc(qg_handle* h, const qg_operation* op, float alpha,
                   const void* A, const qg_layout* Adesc,
                   const void* U, const qg_layout* Udesc,
                   const void* B, const qg_layout* Bdesc,
                   const void* V, const qg_layout* Vdesc,
                   float beta,
                   const void* C, const qg_layout* Cdesc,
                   void* D, const qg_layout* Ddesc,
                   hipStream_t stream);
size_t qg_noalloc_barriers_size(void);
size_t qg_noalloc_partials_size(void);

/* qg_run of a split-K or data-parallel plan that also records where the
 * time of the launch goes (measurement; the pages' tuning is by measurement
 * -- Interface page, Description). The plan, the kernel and its result are
 * those of qg_run (the same bits); in addition the first thread of the
 * workgroup running unit u writes eight 64-bit values to stamps[8u .. 8u+7]
 * (device memory, 8-byte aligned). A split-K unit is (tile t, chunk s),
 * u = t * splits + s; a data-parallel unit is tile u. The values: the
 * constant 100 MHz clock at the unit's start [0], at the end of its
 * mainloop [1], after it published its partial tile [2] (data-parallel: =
 * [1]), after the unit that completed the tile read the partial tiles back
 * and summed them (all its waves) [3] (0 in the other split-K units;
 * data-parallel: = [1]), after the completing unit's stores finished [4]
 * (= [2] in the split-K units that do not complete their tile), 1 in a unit
 * that completes its tile (every data-parallel unit) and 0 otherwise [5],
 * and the shader clock at the start [6] and end [7]. *units receives the
 * number of units of the plan (also when the call fails for a short buffer);
 * units_cap is the capacity of `stamps` in units. Returns
 * QG_ERR_UNSUPPORTED when the resolved plan is neither split-K nor
 * data-parallel (stream-K, grouped, batched), for QG_POLICY_MEASURE and for
 * an empty problem, and QG_ERR_INVALID_ARG for a missing, misaligned or
 * short `stamps`; otherwise as qg_run. */
int qg_run_timed(qg_handle* h, const qg_operation* op, float alpha,
                 const void* A, const qg_layout* Adesc,
                 const void* U, const qg_layout* Udesc,
                 const void* B, const qg_layout* Bdesc,
                 const void* V, const qg_layout* Vdesc,
                 float beta,
                 const void* C, const qg_layout* Cdesc,
                 void* D, const qg_layout* Ddesc,
                 const qg_workspace* ws, hipStream_t stream,
                 uint64_t* stamps, int64_t units_cap, int64_t* units);

/* What qg_run would launch for these arguments, without launching (no
 * device access, no measuring). `desc` receives a NUL-terminated text line
 * "kernel=<name> schedule=<dp|splitk|streamk|grouped> split=<s> programs=<p>
 * tiles=<t> grid=<g> partials=<bytes> barriers=<bytes> bm=<rows> bn=<cols>
 * bk=<k per iteration>"; `cap` is its size. */
int qg_plan(qg_handle* h, const qg_operation* op,
            const qg_layout* Adesc, const qg_layout* Udesc,
            const qg_layout* Bdesc, const qg_layout* Vdesc,
            const qg_layout* Cdesc, const qg_layout* Ddesc,
            float alpha, float beta, const qg_workspace* ws,
            char* desc, size_t cap);

/* ---- dispatch cache ("Export/Import", "GetTuningSeq") ---------------------- */
/* Serialises the dispatch cache as versioned text. With buf == NULL (or cap
 * too small) *len receives the size needed (including the final NUL) and the
 * call returns 0 (NULL buf) or QG_ERR_BUFFER_SMALL. */
int qg_export(qg_handle* h, char* buf, size_t cap, size_t* len);
/* Merges cache text produced by qg_export. All-or-nothing: on any error
 * (QG_ERR_FORMAT) the cache is left unchanged. Entries for another GPU
 * architecture are rejected with QG_ERR_FORMAT. */
int qg_import(qg_handle* h, const char* buf, size_t len);
/* Batch-size (M) tuning sequence: writes min(cap, total) values, *count = total. */
int qg_get_tuning_seq(qg_handle* h, int* out, int cap, int* count);
/* Number of cache entries (for tests and tools). */
int qg_cache_size(qg_handle* h, int* count);

/* ---- registry introspection --------------------------------------------- */
int qg_kernel_count(void);
/* Name of registry entry `index`, or NULL when out of range. */
const char* qg_kernel_name(int index);

/* ---- schedule introspection ---------------------------------------------- */
/* The stream-K division that QG_SCHED_STREAMK runs for `tiles` output tiles
 * of `iters` k-iterations each on `programs` programs (the work-sharing idea
 * of the TileLang tutorial page "gemm_variants.py", gemm_streamk; the split
 * itself is this library's: whole tiles round-robin first, then the last
 * P + T % P tiles' k-iterations (all tiles when T < P; none when P divides T)
 * in P contiguous balanced ranges, program p owning
 * [floor(p W / P), floor((p + 1) W / P)) of their W iterations).
 * qg_streamk_units writes, for every program in order, its work units as rows
 * of five int32 (program, tile, k_begin, k_end, slot) in execution order;
 * slot is the partials-workspace slot of a partial piece, -1 for a whole tile
 * stored directly. At most `cap` rows are written; *count receives the total
 * (QG_ERR_BUFFER_SMALL when it exceeds cap). Host-only, computed by the same
 * code the kernels run. */
int qg_streamk_units(int tiles, int iters, int programs, int32_t* rows, int cap, int* count);
/* The order in which the workgroup completing shared tile `tile` sums its
 * partial pieces: the slots of the owning programs' pieces in k order
 * (*count = 0 for a tile taken whole). Same conventions as above. */
int qg_streamk_fixup(int tiles, int iters, int programs, int tile, int32_t* slots, int cap, int* count);

/* Static text for a status code. */
const char* qg_status_str(int status);
/* Library version string. */
const char* qg_version(void);

#ifdef __cplusplus
}
#endif

#endif /* QGEMM_H */
