/*
 * qgemm.h -- C ABI of the MI355X (gfx950) quantized-weight GEMM library.
 *
 * The library computes C[M,N] = A[M,K] * dequant(Wq)[K,N] for small-to-medium
 * batches (M = 1..128 is the design range; larger M is accepted), the
 * mixed-precision auto-regressive linear layer of the MARLIN paper (abstract:
 * weights compressed to about 4 bits per element, batched decode with 1..128
 * parallel clients, memory-bound up to batch 16..32). Four weight formats,
 * a general-grid 4-bit variant (qgemm_w4g) and a bit-plane W_b A8 format
 * (qgemm_bitplane_*), both below:
 *
 *   W4A16  fp16 activations; unsigned 4-bit codes q (0..15) with an implicit
 *          zero point 8 and one fp16 scale s per group of 128 consecutive k of
 *          one output column: W[k,n] = (q[k,n] - 8) * s[k/128, n].
 *   W4A8   int8 activations with one fp16 scale per row (token); signed int4
 *          weights q (-8..7) with an int8 scale per group of 128 k and an fp16
 *          scale per output column (the W4A8 setting of the OdysseyLLM /
 *          FastGEMM abstract): acc[m,n] = sum_k A[m,k] * q[k,n] * s_g[k/128,n]
 *          exactly in int32, C[m,n] = fp16(acc * a_scale[m] * s_c[n]).
 *   W2W4   mixed 2/4-bit groups (the "Enabling Fast 2-bit LLM on GPUs" page,
 *          abstract: only a small fraction of large-range groups keep 4 bits,
 *          stored with memory alignment in mind): per group of 128 k of one
 *          column either 4-bit codes (zero 8) or 2-bit codes (zero 2), one fp16
 *          scale per group, a host bitmap marking the 4-bit groups.
 *   W4A16_SP24  W4A16 with 2:4 structured sparsity along K (the MARLIN
 *          abstract's sparse extension): in every run of 4 consecutive k
 *          (k = 4j .. 4j+3) of a column at most two codes differ from the zero
 *          point 8; the blob keeps only those two codes and their positions
 *          (3 bits per weight with the metadata) and the GEMM runs on the gfx950
 *          sparse matrix instruction.
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers unless the name ends in _host.
 *     The caller allocates and owns every buffer and keeps it alive until the
 *     work queued on `stream` has finished. The library never allocates or
 *     frees memory.
 *   - `stream` is a hipStream_t (NULL = the default stream). Calls only enqueue
 *     work; results are valid after the caller synchronizes the stream. A fault
 *     inside a kernel surfaces at that synchronization, not as a return code.
 *   - Matrices are row-major with a leading dimension in elements (lda, ldc).
 *   - Return value: QGEMM_OK (0) or a negative qgemm_status. Arguments are fully
 *     validated before any HIP call; a call that fails validation enqueues
 *     nothing and writes nothing. No C++ exception crosses this boundary.
 *   - Shapes: K > 0 a multiple of 128, N > 0 a multiple of 64, K and N at most
 *     2^20, K*N at most 2^32 (2 GiB of 4-bit codes), 0 <= M <= 65535 (M == 0
 *     returns QGEMM_OK without launching anything). A shape for which no launch
 *     configuration fits the 160 KB of LDS of a workgroup is refused with
 *     QGEMM_ERR_SHAPE (the planner finds one for every shape above; the check
 *     guards forced plans and future formats).
 *   - Plans are sized for the current device's compute-unit count (queried
 *     once per device and cached; 256, the MI355X count, when no device is
 *     visible), so query workspace sizes and plans with the device current
 *     that will run the call.
 *   - Pointers: 16-byte aligned; lda, ldc multiples of 8 (fp16) or 16 (int8).
 *   - Concurrent calls that share one workspace race; give each stream its own.
 */
#ifndef QGEMM_H
#define QGEMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum qgemm_status {
  QGEMM_OK = 0,
  QGEMM_ERR_NULL = -1,      /* a required pointer is NULL */
  QGEMM_ERR_SHAPE = -2,     /* K, N or M outside the accepted range */
  QGEMM_ERR_ALIGN = -3,     /* pointer or leading dimension misaligned / too small */
  QGEMM_ERR_WORKSPACE = -4, /* workspace smaller than qgemm_workspace_bytes() */
  QGEMM_ERR_FORMAT = -5,    /* unknown format id */
  QGEMM_ERR_RANGE = -6,     /* an argument value outside its documented range */
  QGEMM_ERR_ALIAS = -7,     /* output overlaps an input */
  QGEMM_ERR_HIP = -8,       /* a HIP runtime call failed (see qgemm_last_error) */
  QGEMM_ERR_DEVICE = -9,    /* current device is not a gfx950 GPU */
  QGEMM_ERR_SIZE = -10      /* blob size does not match qgemm_packed_bytes() */
} qgemm_status;

typedef enum qgemm_fmt {
  QGEMM_FMT_W4A16 = 1,
  QGEMM_FMT_W4A8 = 2,
  QGEMM_FMT_W2W4 = 3,
  QGEMM_FMT_W4G = 4,  /* general grid: only through the qgemm_w4g_* entry points */
  QGEMM_FMT_W4A16_SP24 = 5,
  QGEMM_FMT_BITPLANE = 6  /* bit-plane W_b A8: only through the qgemm_bitplane_* entry points */
} qgemm_fmt;

/* Activation (and scale, output) type of the general-grid 4-bit GEMM. */
typedef enum qgemm_dtype {
  QGEMM_DT_F16 = 1,   /* IEEE binary16 */
  QGEMM_DT_BF16 = 2   /* bfloat16 (upper half of binary32) */
} qgemm_dtype;

/* Human-readable name of a status code (static string, never NULL). */
const char* qgemm_status_str(int status);

/* Text describing the last QGEMM_ERR_HIP / QGEMM_ERR_DEVICE of the calling
 * thread ("" if none). Valid until the thread's next library call. */
const char* qgemm_last_error(void);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int qgemm_version(void);

/*
 * Size in bytes of the repacked weight blob for (fmt, K, N).
 * For QGEMM_FMT_W2W4 the size depends on how many groups are 4-bit, so
 * bitmap_host (uint32[K/128][ceil(N/32)], HOST memory, bit n%32 of word
 * [g][n/32] set = group (g, n) is 4-bit) is required; it is ignored (may be
 * NULL) for the other formats. Bits for columns >= N must be 0 (QGEMM_ERR_RANGE).
 */
int qgemm_packed_bytes(int fmt, int64_t K, int64_t N, const uint32_t* bitmap_host,
                       size_t* bytes);

/*
 * Workspace bytes one GEMM call of this shape needs (0 when the plan does not
 * split K). Layout: a fixed 64 KiB region of per-tile arrival counters, then the
 * split-K partial sums. The workspace must be filled with zero bytes ONCE before
 * its first use; every completed call leaves the counter region zero again, so
 * one workspace can be reused by any sequence of calls (of any shapes and
 * formats) on one stream without clearing. A larger workspace is always
 * accepted. A call interrupted before completion leaves it undefined: zero it
 * again.
 */
int qgemm_workspace_bytes(int fmt, int64_t M, int64_t K, int64_t N, size_t* bytes);

/*
 * Offline weight preprocessing (the arbitrary-precision Tensor Core page's
 * abstract reorganises the matrices ahead of time into a layout suited to the
 * later computation): rewrites canonical codes and scales into the blob the GEMM
 * kernels stream, laid out in gfx950 MFMA operand order (one 1 KB, fully
 * coalesced wave load per 16 columns x 128 k for the 4-bit formats).
 *
 *   W4A16: codes        uint32[K/8][N], nibble j of word [r][n] = code of
 *                       k = 8r + j (0..15)
 *          group_scales fp16[K/128][N]; chan_scales and bitmap_host unused.
 *   W4A8:  codes        uint32[K/8][N], two's-complement int4 nibbles (-8..7)
 *          group_scales int8[K/128][N] (any int8 value)
 *          chan_scales  fp16[N]
 *   W2W4:  codes        uint8[K][N], one code per byte; 0..15 for 4-bit groups,
 *                       0..3 for 2-bit groups (higher bits of 2-bit-group codes
 *                       are ignored)
 *          group_scales fp16[K/128][N]
 *          bitmap_host  HOST uint32[K/128][ceil(N/32)] (see qgemm_packed_bytes)
 *   W4A16_SP24: codes    uint32[K/8][N] dense, as W4A16, pruned weights holding
 *                        code 8; a run of 4 consecutive k with more than two
 *                        other codes is QGEMM_ERR_RANGE (the repack then
 *                        synchronizes `stream` once to read its check)
 *          group_scales fp16[K/128][N]
 *
 * packed must hold exactly qgemm_packed_bytes() bytes (QGEMM_ERR_SIZE
 * otherwise) and must not overlap the inputs. W4A16 and W4A8 repacks are fully
 * asynchronous (W4A16_SP24: see above). The W2W4 repack uploads a small per-tile offset table computed
 * on the host from bitmap_host and synchronizes `stream` once before returning.
 */
int qgemm_repack(int fmt, int64_t K, int64_t N, const void* codes, const void* group_scales,
                 const void* chan_scales, const uint32_t* bitmap_host, void* packed,
                 size_t packed_bytes, void* stream);

/*
 * W4A16 GEMM: C[M,N] (fp16, row-major, leading dimension ldc >= N) =
 * A[M,K] (fp16, lda >= K) * dequant(packed) with fp32 accumulation and one
 * round-to-nearest-even conversion of each output to fp16. packed is a
 * QGEMM_FMT_W4A16 blob of shape (K, N). workspace: see qgemm_workspace_bytes.
 * Results are deterministic (bit-identical run to run).
 */
int qgemm_w4a16(const void* A, int64_t lda, const void* packed, void* C, int64_t ldc,
                int64_t M, int64_t K, int64_t N, void* workspace, size_t workspace_bytes,
                void* stream);

/*
 * W4A8 GEMM: A int8[M][lda], a_scale fp16[M], packed a QGEMM_FMT_W4A8 blob.
 * acc[m,n] = sum_k A[m,k] * q[k,n] * s_g[k/128,n] is computed exactly in int32
 * (K <= 16384 guarantees no overflow for any int8 inputs; larger K is
 * QGEMM_ERR_SHAPE). C fp16[M][ldc] = fp16(float(acc) * a_scale[m] * s_c[n]).
 * acc_out (nullable) receives the int32 accumulators, int32[M][N] dense.
 */
int qgemm_w4a8(const void* A, int64_t lda, const void* a_scale, const void* packed, void* C,
               int64_t ldc, int32_t* acc_out, int64_t M, int64_t K, int64_t N,
               void* workspace, size_t workspace_bytes, void* stream);

/*
 * 2:4 sparse W4A16 GEMM: like qgemm_w4a16 but packed is a QGEMM_FMT_W4A16_SP24
 * blob; the result equals qgemm_w4a16's on the dense codes (pruned weights
 * are exactly zero).
 */
int qgemm_w4a16_sp24(const void* A, int64_t lda, const void* packed, void* C, int64_t ldc,
                     int64_t M, int64_t K, int64_t N, void* workspace, size_t workspace_bytes,
                     void* stream);

/*
 * Mixed 2/4-bit GEMM: like qgemm_w4a16 but packed is a QGEMM_FMT_W2W4 blob; each
 * group dequantizes with zero point 8 (4-bit) or 2 (2-bit) as recorded in it.
 */
int qgemm_w2w4_mixed(const void* A, int64_t lda, const void* packed, void* C, int64_t ldc,
                     int64_t M, int64_t K, int64_t N, void* workspace, size_t workspace_bytes,
                     void* stream);

/*
 * Per-token dynamic int8 quantization of fp16 activations, producing the A and
 * a_scale operands of qgemm_w4a8 (the Atom review's method section adapts the
 * activation quantization parameters to each activation matrix at inference
 * time; the OdysseyLLM abstract's W4A8 GEMM takes int8 activations). Symmetric
 * absmax per row m of A fp16[M][lda]:
 *   a_scale[m] = fp16(amax_m / 127), amax_m = max_k |A[m,k]| (fp32 division,
 *                round to nearest even),
 *   A_q[m,k]   = clamp(rint(A[m,k] / a_scale[m]), -127, 127) (fp32, half to
 *                even); a row with a_scale[m] == 0 becomes zeros.
 * A_q int8[M][ldq] and a_scale fp16[M] are device outputs owned by the caller.
 * Shapes: 0 < K <= 2^20 a multiple of 8, 0 <= M <= 65535 (M == 0: no launch).
 * Alignment: A and A_q 16 bytes, a_scale 2 bytes, lda >= K a multiple of 8,
 * ldq >= K a multiple of 16 (so A_q feeds qgemm_w4a8 directly). Outputs must
 * not overlap A or each other (QGEMM_ERR_ALIAS). Elements of A must be finite.
 */
int qgemm_quantize_a8(const void* A, int64_t lda, int64_t M, int64_t K, void* A_q, int64_t ldq,
                      void* a_scale, void* stream);

/*
 * 4-bit weights on a general quantization grid. The 2-bit page's abstract and
 * the Atom review's method section quantize weights by groups without fixing
 * the group length, and asymmetric grids keep a zero point per group:
 *
 *   W[k,n] = (q[k,n] - z[g,n]) * s[g,n],  g = k / group_size,
 *
 * with unsigned 4-bit codes q, group_size 64 or a multiple of 128 that divides
 * K (group_size == K gives one scale per column), z a stored zero point 0..15
 * per (group, column) or, without stored zero points, the constant 8, and
 * activations A, scales s and output C all of one type (act_dtype,
 * QGEMM_DT_F16 or QGEMM_DT_BF16). Accumulation is fp32; each output is
 * rounded once (to nearest even) to act_dtype. Shapes and alignment as for
 * qgemm_w4a16; an invalid group_size or act_dtype is QGEMM_ERR_RANGE.
 *
 * qgemm_w4g_packed_bytes: blob size (has_zeros 0 or 1).
 * qgemm_w4g_workspace_bytes: workspace for a call of this shape with any grid
 *   and activation type (otherwise the contract of qgemm_workspace_bytes).
 * qgemm_w4g_repack: codes uint32[K/8][N] (as W4A16), scales 16-bit
 *   [K/group_size][N] in the activation type (copied bit for bit), zeros
 *   uint8[K/group_size][N] or NULL (implicit 8; only the low 4 bits of each
 *   stored value are used). packed must hold exactly qgemm_w4g_packed_bytes()
 *   bytes with has_zeros = (zeros != NULL). Asynchronous on `stream`.
 * qgemm_w4g: the GEMM; group_size and has_zeros must be those the blob was
 *   repacked with (they are not recorded in it), act_dtype the type of A, of
 *   the scales given to the repack and of C (C is act_dtype[M][ldc]).
 */
int qgemm_w4g_packed_bytes(int64_t K, int64_t N, int32_t group_size, int32_t has_zeros,
                           size_t* bytes);
int qgemm_w4g_workspace_bytes(int64_t M, int64_t K, int64_t N, size_t* bytes);
int qgemm_w4g_repack(int64_t K, int64_t N, int32_t group_size, const void* codes,
                     const void* scales, const void* zeros, void* packed, size_t packed_bytes,
                     void* stream);
int qgemm_w4g(const void* A, int64_t lda, const void* packed, void* C, int64_t ldc, int64_t M,
              int64_t K, int64_t N, int32_t group_size, int32_t has_zeros, int32_t act_dtype,
              void* workspace, size_t workspace_bytes, void* stream);

/*
 * Bit-plane W_b A8 GEMM, b = 1..8 bits per weight (the arbitrary-precision
 * Tensor Core page's abstract: a symmetric bipolar-INT weight format whose
 * matrices are decomposed at the bit level and recovered after the products).
 * A weight with stored bits u_i (code U = sum_i 2^i u_i) has the value
 *   w = sum_i 2^i (2 u_i - 1) = 2U - (2^b - 1),
 * the odd integers -(2^b - 1) .. 2^b - 1; each output column has one fp16
 * scale s_c[n]. Activations are int8 with a per-row fp16 scale (as
 * qgemm_w4a8; qgemm_quantize_a8 produces them):
 *   acc[m,n] = sum_k A[m,k] * w[k,n]   (exact int32; K <= 65536, else
 *              QGEMM_ERR_SHAPE, keeps |acc| < 2^31 for every input)
 *   C[m,n]   = fp16(float(acc) * a_scale[m] * s_c[n]).
 * The blob holds the b bit planes (b/8 bytes per weight) and the channel
 * scales. bits outside 1..8 is QGEMM_ERR_RANGE.
 *
 * qgemm_bitplane_packed_bytes / _workspace_bytes: sizes (workspace contract
 *   as qgemm_workspace_bytes).
 * qgemm_bitplane_repack: codes uint8[K][N] holding U (only the low `bits`
 *   bits of each byte are used), chan_scales fp16[N]; packed must hold exactly
 *   qgemm_bitplane_packed_bytes() bytes. Asynchronous on `stream`.
 * qgemm_bitplane_a8: A int8[M][lda] (lda a multiple of 16), a_scale fp16[M],
 *   C fp16[M][ldc], acc_out (nullable) int32[M][N] dense; `bits` must be the
 *   value the blob was repacked with (it is not recorded in the blob).
 */
int qgemm_bitplane_packed_bytes(int64_t K, int64_t N, int32_t bits, size_t* bytes);
int qgemm_bitplane_workspace_bytes(int64_t M, int64_t K, int64_t N, int32_t bits, size_t* bytes);
int qgemm_bitplane_repack(int64_t K, int64_t N, int32_t bits, const void* codes, const void* chan_scales,
                          void* packed, size_t packed_bytes, void* stream);
int qgemm_bitplane_a8(const void* A, int64_t lda, const void* a_scale, const void* packed, void* C,
                      int64_t ldc, int32_t* acc_out, int64_t M, int64_t K, int64_t N, int32_t bits,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * qgemm_w4a16 for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc. Same
 * arguments, kernels, plans and results as qgemm_w4a16 minus the workspace:
 * the split-K arrival counters and partial sums live in a fixed 32 MiB device
 * array of this library (one per GPU, held until the process ends; its
 * address is looked up once per device). The call allocates and frees
 * nothing; the caller still provides A, the blob and C.
 *   - A call whose plan needs more than 32 MiB of split-K scratch (only forced
 *     plans: every automatic W4A16 plan needs at most 16 MiB + 64 KiB) returns
 *     QGEMM_ERR_WORKSPACE before any launch; other errors as qgemm_w4a16.
 *   - The first call on a device queues a clear of the array's counters on
 *     `stream` before its GEMM; every completed call leaves them zero again.
 *   - All calls on one GPU share its array: calls that can overlap (on
 *     different streams, or concurrent graph replays) race and give wrong
 *     results. Serialize them, or use qgemm_w4a16 with one workspace each.
 */
int qgemm_w4a16_noalloc(const void* A, int64_t lda, const void* packed, void* C, int64_t ldc, int64_t M,
                        int64_t K, int64_t N, void* stream);

/*
 * Work decomposition used for a call of this shape (for tests and tuning).
 * Fills out10[0..9] = {kernel id (1 streaming, 2 wide, 3 streaming general-grid
 * kernel with per-lane grid entries; 1 there stages them in LDS), 16-row blocks per tile,
 * 16-column blocks per wave (kernel 2: the tile width in 64-column units, 4
 * or 2), waves per workgroup,
 * k-splits across workgroups, groups per k-split, m-tiles, n-tiles,
 * workgroups, waves}. fmt may also be QGEMM_FMT_W4G: the plan for group length
 * 128 with zero points and fp16 activations (qgemm_w4g_plan gives it for any
 * grid and type). Host-only: its only HIP calls are the cached device-property
 * queries.
 */
int qgemm_plan(int fmt, int64_t M, int64_t K, int64_t N, int64_t* out10);

/*
 * The work decomposition of a call of any format (fmt QGEMM_FMT_BITPLANE uses
 * `bits`, QGEMM_FMT_W4G uses `group_size`, `has_zeros` and `act_dtype`; the
 * others ignore them) with the launch's resources: out12[0..9] as qgemm_plan, out12[10] =
 * workspace bytes the call needs, out12[11] = dynamic LDS bytes per workgroup
 * the launch requests (at most 160 KB - 256). QGEMM_ERR_SHAPE when no launch
 * shape fits; argument rules as for the format's GEMM entry point. Host-only:
 * its only HIP calls are the cached device-property queries.
 */
int qgemm_plan_info(int fmt, int64_t M, int64_t K, int64_t N, int32_t bits, int32_t group_size,
                    int32_t has_zeros, int32_t act_dtype, int64_t* out12);

/*
 * The work decomposition of a bit-plane W_b A8 call (qgemm_bitplane_a8) of
 * this shape and bit width, in the layout of qgemm_plan. bits outside 1..8:
 * QGEMM_ERR_RANGE; shape rules as for qgemm_bitplane_a8. Host-only (cached
 * device-property queries only).
 */
int qgemm_bitplane_plan(int64_t M, int64_t K, int64_t N, int32_t bits, int64_t* out10);

/*
 * The work decomposition of a general-grid call (qgemm_w4g) of this shape,
 * grid and activation type, in the layout of qgemm_plan; the grid sets the
 * size of the grid entries that the kernel can stage in LDS, and fp16 calls
 * with N a multiple of 256 may run on the wide kernel (kernel id 2), so both
 * enter the choice. An invalid group_size, has_zeros or act_dtype:
 * QGEMM_ERR_RANGE; shape rules as for qgemm_w4g. Host-only (cached
 * device-property queries only).
 */
int qgemm_w4g_plan(int64_t M, int64_t K, int64_t N, int32_t group_size, int32_t has_zeros,
                   int32_t act_dtype, int64_t* out10);

/*
 * Override the automatic plan for later calls of this process: kernel (1 =
 * streaming kernel for every format, 2 = wide kernel for W4A16 and for the
 * general grid with fp16 activations, N a multiple of 256, 3 = general-grid
 * streaming kernel with per-lane grid entries; other cases keep kernel 1),
 * nb: 16-column blocks per wave of kernel 1 (1 or 2; 4 is taken as 2), or the
 * tile width of kernel 2 in 64-column units (4: 256 columns, 2: 128 columns
 * as two K-parts of 4 waves, which fixes 8 waves; 1: automatic), waves per
 * workgroup (kernel 1: 4, 8 or 16; kernel 2 with 256 columns: 16 runs two
 * K-parts of 8 waves, 4 or 8 one part of 8) and
 * k-splits across workgroups (1..4096); 0 keeps the automatic choice for that
 * field. Values a shape cannot use are clamped (no more K-parts than groups).
 * For tests of the split-K reductions and for tuning sweeps; affects
 * qgemm_workspace_bytes and qgemm_plan too. Not thread-safe against concurrent
 * GEMM calls.
 */
int qgemm_set_plan_override(int kernel, int nb_per_wave, int waves_per_workgroup, int k_splits);

#ifdef __cplusplus
}
#endif

#endif /* QGEMM_H */
