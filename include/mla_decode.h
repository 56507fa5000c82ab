/*
 * mla_decode.h -- C ABI of the MI355X (gfx950) absorbed-MLA split-KV decode library.
 *
 * Source pages: "Kimi K3 on AMD Instinct MI355X: vLLM serving ... on AgentX" (AMD blog
 * post).  What the library computes follows:
 *   - section 4 "MLA: AITER assembly long-context decode": a decode query of an MLA
 *     layer reads the layer's whole compressed KV history; query heads attend
 *     independently, so 12 heads may be padded to 16 without changing any real head;
 *     the history is split into partitions processed by different workgroups of one
 *     GPU and their results are combined, with the KV storage left as it is;
 *   - section 1 "Cache", DCP8 paragraph: under decode context parallelism each GPU
 *     holds a slice of the positions and returns, per head, a partial answer that
 *     carries its softmax normalisation; partial answers are merged with softmax
 *     weights;
 *   - section 1, payload estimate: one cached position of one layer is a 576-value
 *     latent (576 bytes in FP8);
 *   - section 5 (verification positions) and section 6 (draft depth): several draft
 *     tokens of a request are verified at once.
 *
 * Arithmetic.  For request r with L = seq_lens[r] cached positions, query token t of
 * T = q_len (the last T cached positions are the T query tokens), and head h:
 *     n      = causal ? L - T + t + 1 : L        (visible positions 0 .. n-1)
 *     s_j    = softmax_scale * sum_{d<576} q[r,t,h,d] * x_r[j,d]
 *     O      = sum_j exp(s_j) * x_r[j, 0:512] / sum_j exp(s_j)
 *     LSE    = ln sum_j exp(s_j)                 (natural log, of the scaled scores)
 * where x_r[j,:] is the latent of position j (K = all 576 columns, V = the first 512).
 * An empty visible set gives O = 0 and LSE = -inf.
 *
 * Memory.  The caller owns every buffer.  Device buffers are plain device pointers
 * (hipMalloc / torch CUDA tensors).  The library allocates no device memory and never
 * keeps a pointer past a call (the scratch of mla_decode_splitkv_noalloc is a static
 * device array of the library's code object, not an allocation).  A plan is host memory
 * owned by the library (mla_plan_create / mla_plan_destroy).
 *
 * Streams.  `stream` is a hipStream_t passed as void* (NULL = the null stream).  All
 * device work is enqueued on it; no call synchronises the host with the device.
 *
 * Errors.  Every entry point returns a status; nothing throws or aborts across the
 * ABI.  Argument, shape, dtype, alignment and size checks run on the host before any
 * work is enqueued; on an error nothing is enqueued and no output is touched.
 * mla_last_error() gives a message for the last failing call of the calling thread.
 * Launch failures return MLA_ERR_DEVICE.  Block-table contents are not checked on
 * the decode path (that would need a device synchronisation); mla_block_table_check
 * is the host-side check.  A page id outside [0, num_pages) met on the device is not
 * dereferenced: the affected rows come out as NaN instead.
 */
#ifndef MLA_DECODE_H
#define MLA_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MLA_OK = 0,
  MLA_ERR_INVALID_ARGUMENT = 1,
  MLA_ERR_UNSUPPORTED = 2,
  MLA_ERR_WORKSPACE_TOO_SMALL = 3,
  MLA_ERR_DEVICE = 4
} mla_status;

typedef enum {
  MLA_BF16 = 0,       /* bfloat16 */
  MLA_FP8_E4M3FN = 1, /* OCP FP8 E4M3FN: bias 7, max 448, no inf, S.1111.111 = NaN */
  MLA_FP32 = 2        /* IEEE binary32 */
} mla_dtype;

/* Latent width: the key of a position uses all MLA_D_LATENT values of its row, the
 * value the first MLA_D_V (section 1 payload estimate: 576 values per position). */
#define MLA_D_LATENT 576
#define MLA_D_V 512
/* Supported page size (positions per page). */
#define MLA_PAGE_SIZE 64

/*
 * Paged latent KV of one layer.  All pointers are caller-owned device memory.
 *   pool        [num_pages][page_size][576] elements of kv_dtype, row-major, 16-byte
 *               aligned.  Position j of request r lives at
 *               pool[block_table[r*max_pages_per_seq + j/page_size]][j%page_size][:].
 *               Pages are only read; several requests may share a page.
 *   kv_dtype    MLA_BF16 or MLA_FP8_E4M3FN.
 *   kv_scale    FP8 dequantisation factor (value = code * kv_scale), finite and > 0;
 *               must be exactly 1.0f for MLA_BF16.
 *   block_table int32 [batch][max_pages_per_seq], physical page ids.  Only the first
 *               ceil(seq_lens[r]/page_size) entries of row r are read.
 *   seq_lens    int32 [batch], cached positions per request including its q_len query
 *               tokens.  Must equal the host copy the plan was made from: for batch <= 64
 *               the partial stage works from the plan's copy and compares each request's
 *               device length with it, and a request that differs comes out as NaN rows
 *               (its partial answers too); above 64 requests both stages read the device
 *               lengths, and a total page count that differs from the plan's makes every
 *               row NaN.
 */
typedef struct {
  const void* pool;
  int64_t num_pages;
  int32_t page_size;
  int32_t kv_dtype; /* mla_dtype */
  float kv_scale;
  const int32_t* block_table;
  int32_t max_pages_per_seq;
  const int32_t* seq_lens;
} mla_paged_kv;

/*
 * Decode problem shape.
 *   batch         requests (>= 1)
 *   q_len         query tokens per request, T >= 1 (T > 1: multi-token verification)
 *   num_heads     real query heads H >= 1; rows are padded to a multiple of 16 inside
 *                 the kernel (padding rows are never loaded or written).  Limit:
 *                 q_len * ceil(H/16) <= 64.
 *   softmax_scale scale applied to q.k (e.g. 1/sqrt(192)), finite and > 0
 *   causal        1: token t sees positions 0 .. L-T+t; 0: every token sees all L
 *   num_splits    history partitions per request: 0 = automatic (pages balanced over
 *                 all compute units, one partial per piece), k >= 1 = k near-equal
 *                 page-aligned contiguous pieces per request (16 is the policy the
 *                 pages describe for the AITER assembly path, 1 the one-workgroup-
 *                 per-request policy of the older path)
 * The partial answers between the two stages are kept in fp32 in the workspace.
 */
typedef struct {
  int32_t batch;
  int32_t q_len;
  int32_t num_heads;
  float softmax_scale;
  int32_t causal;
  int32_t num_splits;
} mla_decode_shape;

typedef struct mla_plan mla_plan; /* opaque, host memory */

/*
 * Plan a decode step: choose the partition of every request's history into
 * workgroup tasks (section 4: partitions are workgroup tasks on one GPU; section
 * "What to optimise next": count the independent work so that all compute units
 * are busy).  A plan depends only on the shape, the host copy of seq_lens, the KV
 * dtype and the compute-unit count, so one plan serves every layer of a decode step.
 *   seq_lens_host  int32 [batch] host memory, each >= q_len with causal = 1, else >= 1
 *   page_size      must be MLA_PAGE_SIZE
 *   num_cus        compute units to fill; 0 = query the current device
 *   plan           out: new plan, release with mla_plan_destroy
 *   workspace_bytes out: device workspace size mla_decode_splitkv needs with it
 * Residency experiment (Kimi K3 on MI355X, "Technical notes": reserve unused LDS to
 * cross an occupancy threshold with the same kernel binary, then compare times): when
 * the environment variable MLA_LDS_RESERVE holds a byte count at plan creation, every
 * merge workgroup of the plan's decodes reserves that much unused LDS (clamped to
 * [0, 131072]; results are unchanged, only how many merge workgroups a compute unit
 * holds at once).  Unset, no LDS is reserved.
 */
mla_status mla_plan_create(const mla_decode_shape* shape, const int32_t* seq_lens_host,
                           int32_t page_size, int32_t kv_dtype, int32_t num_cus,
                           mla_plan** plan, size_t* workspace_bytes);
void mla_plan_destroy(mla_plan* plan);
/* Work units of the partial stage (history ranges; each unit's pieces are the
 * entries of mla_plan_get_work with that unit index), and partial slots in the workspace. */
int32_t mla_plan_num_units(const mla_plan* plan);
int32_t mla_plan_num_parts(const mla_plan* plan);
/* Workgroups per work unit: the 16-row blocks of the problem (q_len * ceil(num_heads/16))
 * are dealt to that many workgroups, two per workgroup from two row blocks on (an odd
 * count is padded with one row block that is computed and discarded). */
int32_t mla_plan_row_groups(const mla_plan* plan);
/*
 * Optional FP8 matrix-core form of q.k for an FP8 pool (Kimi K3 on MI355X, section 1
 * "Cache": the latents are stored in FP8; the same section's DCP8 paragraph: one shard
 * holds all 96 heads).  enable = 1: the partial stage feeds the pool's E4M3FN codes to
 * the FP8 matrix cores as they are, and each query row as two E4M3FN vectors hi + lo
 * after scaling the row by a power of two (hi + lo equals every bf16 query element
 * times that power exactly, except elements below 2^-9 of the row's largest magnitude,
 * which keep an error below 2^-17 of it).  The value side is unchanged.  Off by default.
 * Needs kv_dtype = MLA_FP8_E4M3FN and q_len * ceil(num_heads/16) >= 2; otherwise
 * MLA_ERR_UNSUPPORTED (the plan is left unchanged).  enable must be 0 or 1
 * (MLA_ERR_INVALID_ARGUMENT).
 */
mla_status mla_plan_set_fp8_qk(mla_plan* plan, int32_t enable);
/*
 * Host copy of the work list, for inspection: 5 int32 per piece
 * (workgroup, request, first page, end page (exclusive), partial slot), in workgroup
 * order.  Writes at most `capacity` pieces; returns the number of pieces, or -1 on a
 * bad argument.
 */
int32_t mla_plan_get_work(const mla_plan* plan, int32_t* out, int32_t capacity);

/*
 * Split-KV decode of one MLA layer.
 *   q          bf16 [batch][q_len][num_heads][576], 16-byte aligned
 *   kv         paged latent KV (kv->kv_dtype must match the plan's)
 *   workspace  device scratch of at least the plan's workspace_bytes, 256-byte
 *              aligned.  It holds the partial answers between the two stages and needs
 *              no initialisation.
 *   out        [batch][q_len][num_heads][512] of out_dtype (MLA_BF16, rounded to
 *              nearest even, or MLA_FP32), 16-byte aligned, or NULL
 *   out_lse    fp32 [batch][q_len][num_heads] natural-log LSE, or NULL.  With it the
 *              result is a DCP shard's partial answer (section 1): merge shards with
 *              mla_merge_lse.
 *   hidden     NULL (the shape's causal flag decides what each token sees), or device
 *              int32 [batch][q_len], 4-byte aligned, read during this call only: token t
 *              of request r then attends to the first seq_lens[r] - hidden[r][t]
 *              positions of its history (values below 0 count as 0; seq_lens[r] or more
 *              hides everything, and that row's answer is empty: LSE = -inf, O = 0).
 *              This replaces the causal pattern (causal is hidden = q_len - 1 - t), so a
 *              decode-context-parallel shard whose local history ends with some of the
 *              draft tokens masks exactly the drafts each token may not see (section 1
 *              "Cache", DCP8 paragraph, and the multi-token verification it extends to).
 * The two stages run as two kernels back to back on `stream`.  With out == NULL and
 * out_lse == NULL only the partial stage runs and the partials stay in the workspace:
 * at byte 0, fp32 O [rows][16][num_parts][32] (row = token * num_heads + head; the 512
 * columns in 16 chunks of 32, each chunk's parts contiguous); then, at the next 256-byte
 * boundary, fp32 LSE [rows][num_parts].  The parts of request r are the slots that
 * mla_plan_get_work lists for it.
 * Calls that share a workspace must be ordered on one stream.
 */
mla_status mla_decode_splitkv(const mla_plan* plan, const void* q, const mla_paged_kv* kv,
                              void* workspace, size_t workspace_bytes, void* out,
                              int32_t out_dtype, float* out_lse, const int32_t* hidden,
                              void* stream);

/*
 * Split-KV decode that allocates nothing, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * mla_decode_splitkv with the partial answers kept in a scratch array the library holds,
 * one per GPU (MLA_NOALLOC_SCRATCH_BYTES each, kept until the process ends), instead of
 * a caller's workspace.  Arguments and results are those of mla_decode_splitkv, except
 * that out and out_lse may not both be NULL (MLA_ERR_INVALID_ARGUMENT).  A plan whose
 * workspace_bytes exceed MLA_NOALLOC_SCRATCH_BYTES is refused (MLA_ERR_UNSUPPORTED,
 * nothing enqueued).  Every call on one GPU uses that GPU's one scratch array, which
 * keeps the last call's partial answers (nothing in it needs to start cleared): calls
 * ordered on one stream are fine, calls that overlap on one GPU (several streams, or
 * host threads without ordering) race and must not be made.  The first call on a device
 * looks up the array's address there (hipGetSymbolAddress; no allocation).
 */
#define MLA_NOALLOC_SCRATCH_BYTES (32u << 20)
mla_status mla_decode_splitkv_noalloc(const mla_plan* plan, const void* q, const mla_paged_kv* kv,
                                      void* out, int32_t out_dtype, float* out_lse,
                                      const int32_t* hidden, void* stream);

/*
 * Merge partial answers that carry their LSE (section 1, DCP8 paragraph; section 4,
 * combining partitions).  For every row:
 *   M = max_p LSE_p;  a_p = exp(LSE_p - M);
 *   O = sum_p a_p O_p / sum_p a_p;  LSE = M + ln sum_p a_p
 * Rows whose parts are all -inf give O = 0, LSE = -inf.
 *   part_o    [num_parts][rows][512] of part_dtype (MLA_BF16 or MLA_FP32), 16-byte aligned
 *   part_lse  fp32 [num_parts][rows]
 *   out       [rows][512] of out_dtype (MLA_BF16 or MLA_FP32), or NULL
 *   out_lse   fp32 [rows], or NULL
 */
mla_status mla_merge_lse(const void* part_o, int32_t part_dtype, const float* part_lse,
                         int32_t num_parts, int64_t rows, void* out, int32_t out_dtype,
                         float* out_lse, void* stream);

/*
 * Append the q_len new tokens' latents of every request to the paged cache of one layer
 * (section 1 "Cache": one 576-value latent per cached position and layer, stored in
 * FP8, growing by the new tokens of every step; the model side hands them over in BF16).
 *   pool        [num_pages][page_size][576] of kv_dtype, device memory, 16-byte aligned;
 *               written in place (only the new positions' rows)
 *   kv_dtype    MLA_BF16: the bf16 bits are copied.  MLA_FP8_E4M3FN: each value x is
 *               stored as the E4M3FN code nearest to fp32(x) / kv_scale (an fp32
 *               division), ties to the even code, magnitudes past 448 saturating to
 *               +-448, NaN to a NaN code
 *   kv_scale    as in mla_paged_kv (finite > 0 for FP8, exactly 1 for bf16)
 *   block_table, max_pages_per_seq, seq_lens: as in mla_paged_kv, device memory;
 *               seq_lens[r] counts the new tokens, so token t of request r goes to
 *               position seq_lens[r] - q_len + t
 *   latents     bf16 [batch][q_len][576], device memory, 16-byte aligned
 * A new position below 0, past the block-table row, or whose page id is outside
 * [0, num_pages), is skipped on the device (nothing is written for it).  Enqueued on
 * `stream`; a decode that reads the new positions must be ordered after it.
 */
mla_status mla_kv_append(void* pool, int64_t num_pages, int32_t page_size, int32_t kv_dtype,
                         float kv_scale, const int32_t* block_table, int32_t max_pages_per_seq,
                         const int32_t* seq_lens, const void* latents, int32_t batch,
                         int32_t q_len, void* stream);

/*
 * Host-side block-table check: every page a request reads (the first
 * ceil(seq_lens[r]/page_size) entries of its row) is in [0, num_pages), and
 * ceil(seq_lens[r]/page_size) <= max_pages_per_seq.  Host pointers.
 */
mla_status mla_block_table_check(const int32_t* block_table_host, int32_t batch,
                                 int32_t max_pages_per_seq, const int32_t* seq_lens_host,
                                 int32_t page_size, int64_t num_pages);

/*
 * Bandwidth reference, for measurement only (the post's roofline is the 8 TB/s HBM figure
 * of its MI355X specification table, and "What to optimise next" asks for measured
 * limits): one kernel that reads every byte of [buf, buf + bytes) once and does nothing
 * else, so its time is the floor any single launch that streams the same bytes can
 * reach on this device.
 *   mode 0  plain 128-bit vector loads into registers (4,096 workgroups, grid-stride)
 *   mode 1  128-bit direct copies into LDS, 144 KiB per workgroup: the copy the partial
 *           stage issues for its pages, without the attention arithmetic
 *   mode 2  an empty kernel (one workgroup): the cost of a launch; buf, bytes and sink
 *           are ignored
 *   buf     device memory, 16-byte aligned; bytes a multiple of 1024
 *   sink    device uint32, 4-byte aligned; written only if a checksum of the data hits
 *           one fixed 96-bit pattern (so in practice never)
 * Enqueued on `stream`.  Errors: MLA_ERR_INVALID_ARGUMENT for a bad mode, pointer,
 * alignment or size; MLA_ERR_DEVICE if the launch fails.
 */
mla_status mla_read_reference(const void* buf, size_t bytes, int32_t mode, uint32_t* sink, void* stream);

/* Bytes of one page: page_size * 576 * element size; 0 for an unsupported dtype. */
size_t mla_page_bytes(int32_t page_size, int32_t kv_dtype);
const char* mla_status_str(mla_status status);
/* Message for the last failing call on this thread ("" if none). */
const char* mla_last_error(void);
const char* mla_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MLA_DECODE_H */
