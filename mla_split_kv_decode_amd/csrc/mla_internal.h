// Internal definitions shared by the host library and the gfx950 kernels.
//
// Work decomposition (Kimi K3 on MI355X, section 4 "MLA": the history of a request is
// split into partitions that different workgroups process, and their results are
// combined; section "What to optimise next": count the independent work so every
// compute unit gets some).
//
// Pages are the unit of work.  Request r owns pages_r = ceil(L_r / 64) pages (clamped
// to the block-table row length), and the requests' pages are laid end to end on a
// global axis g = pre_r + local page, pre_r = sum_{s<r} pages_s, P = sum_r pages_r.
//
//  * SPLIT_BALANCED (num_splits = 0): W work units, W <= P.  Unit w takes global pages
//    [floor(w P / W), floor((w+1) P / W)), which may span several requests.  Each
//    (unit, request) overlap is one piece with its own partial answer, stored in slot
//    w + r.  Along the global axis both w and r only grow, so no two pieces share a
//    slot, and the pieces of request r occupy the contiguous slot range
//    [wg_of(pre_r) + r, wg_of(pre_r + pages_r - 1) + r].  Slots: W + B - 1.
//  * SPLIT_FIXED (num_splits = S >= 1): W = B * S units; unit w = r S + s takes the
//    request's local pages [floor(s pages_r / S), floor((s+1) pages_r / S)) and slot w.
//    A piece may be empty (pages_r < S); it then stores LSE = -inf and O = 0.
//
// A unit runs as row_groups workgroups, each computing the unit's pieces for its own
// row blocks (16 query rows each), i.e. its own rows of every slot.
//
// Both the host planner (for inspection and sizing) and the device kernels evaluate the
// same closed forms below, from seq_lens; the device never needs an uploaded work list.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define MLA_HD __host__ __device__ __forceinline__
#else
#define MLA_HD inline
#endif

namespace mla {

constexpr int kPage = 64;          // positions per page
constexpr int kDLatent = 576;      // latent width (key = all columns)
constexpr int kDV = 512;           // value width (first columns of the latent)
constexpr int kRowsPerBlock = 16;  // MFMA rows: heads are padded to a multiple of 16
constexpr int kMaxRowBlocks = 64;  // q_len * ceil(heads / 16) limit of one call

enum SplitMode : int32_t { SPLIT_BALANCED = 0, SPLIT_FIXED = 1 };

// Partial answers between the two stages, in the workspace (slots = the plan's parts):
//   O   [rows][kDV / kMergeCols chunks][slots][kMergeCols] fp32
//   LSE [rows][slots] fp32
// rows = q_len * num_heads, token-major then head; request r's pieces use its own slot
// range.  A merge unit (row, column chunk) of a request thus reads one contiguous block.
constexpr int kMergeCols = 32;
constexpr int kMergeChunks = kDV / kMergeCols;  // 16

// Pages request r reads, from its length and the block-table row length.
MLA_HD int32_t pages_of(int32_t seq_len, int32_t max_pages) {
  int32_t p = seq_len > 0 ? (seq_len + kPage - 1) / kPage : 0;
  return p < max_pages ? p : max_pages;
}

// floor(x / y) for 0 <= x < 2^52, 0 < y: a double-precision estimate corrected to the
// exact quotient with integer multiplies (a 64-bit integer division is a long software
// sequence on the GPU).
MLA_HD int64_t div_floor(int64_t x, int64_t y) {
  int64_t q = (int64_t)((double)x / (double)y);
  if (q * y > x) --q;
  if ((q + 1) * y <= x) ++q;
  return q;
}

// floor(x / y) as above, with plain 32-bit division when the operands fit (the usual case).
MLA_HD int64_t div_floor_fast(int64_t x, int64_t y) {
  if (x >= 0 && x <= 0xFFFFFFFFll && y > 0 && y <= 0xFFFFFFFFll) return (int64_t)((uint32_t)x / (uint32_t)y);
  return div_floor(x, y);
}

// First global page of unit w under SPLIT_BALANCED.
MLA_HD int64_t balanced_start(int64_t w, int64_t P, int64_t W) { return div_floor_fast(w * P, W); }

// Unit holding global page g under SPLIT_BALANCED (largest w with start(w) <= g).
MLA_HD int64_t balanced_wg_of(int64_t g, int64_t P, int64_t W) { return div_floor_fast((g + 1) * W - 1, P); }

MLA_HD int32_t fixed_page_begin(int32_t s, int32_t pages, int32_t S) {
  return (int32_t)(((int64_t)s * pages) / S);
}

// The plan's host copy of the lengths, in the kernel arguments when the batch is small
// enough, so that neither kernel waits for a device load of seq_lens before its first
// real loads.  The partial stage still reads the device seq_lens, under its page copies,
// and a request whose device length differs from the plan's gives NaN pieces, which the
// merge carries to the request's rows.
constexpr int kArgBatch = 64;
struct PlanArgs {
  int32_t n;                    // requests described here (0: derive from device seq_lens)
  int32_t len[kArgBatch];       // seq_lens of the plan
  int32_t pre[kArgBatch + 1];   // pre[r] = sum_{s<r} ceil(len[s] / kPage)
};

// Blocks of a partial-stage launch: W units times the row groups, rounded up to whole
// groups of eight units when there are several row groups (block b serves unit
// 8 (b / 8 / G) + b % 8, row group (b / 8) % G; see the kernel).
MLA_HD int64_t partial_grid(int64_t W, int32_t G) { return G == 1 ? W : (W + 7) / 8 * 8 * G; }

// Launch parameters of the partial-attention kernel.
struct PartialParams {
  const uint16_t* q;          // bf16 [B][T][H][576]
  const uint8_t* pool;        // [num_pages][64][576] of the KV element type
  const int32_t* block_table; // [B][max_pages]
  const int32_t* seq_lens;    // [B]
  float* part_o;              // fp32 partial O (layout above)
  float* part_lse;            // fp32 [rows][slots]
  int64_t num_pages;
  int32_t max_pages;
  int32_t batch, q_len, num_heads, head_groups, rows;  // rows = T * H
  int32_t rbw;        // row blocks per workgroup (1 or 2)
  int32_t row_groups; // workgroups per work unit: q_len * head_groups / rbw
  int32_t causal;
  int32_t mode;       // SplitMode
  int32_t num_wg;     // W work units
  int32_t num_splits; // S (SPLIT_FIXED)
  int32_t num_slots;  // slot stride of the partial layout
  int64_t total_pages; // P from the plan's host copy of seq_lens (SPLIT_BALANCED)
  float score_scale;  // softmax_scale * log2(e) * kv_scale: scores in log2 units
  float v_scale;      // kv_scale applied to the value rows (1 for bf16)
  PlanArgs plan;
  const int32_t* hidden;  // null, or [B][T]: token t of request r does not see the last
                          // hidden[r][t] positions (replaces the causal pattern)
  int32_t nt_parts;       // fp32 parts stored non-temporal (kNtPartBytes)
  int32_t stream_pages;   // one-row-group kernels: page copies with the non-temporal hint
};

// A layer's KV above this size is streamed past the caches (non-temporal page copies): the
// memory-side cache (256 MB) could not keep the 24 layers' pools between decode steps.
constexpr int64_t kStreamKvBytes = int64_t(8) << 20;

// Partial answers go out with non-temporal stores when they are a large share of the
// partial kernel's traffic: at least this many bytes and an eighth of the KV bytes (no
// write-allocate in L2 and no dirty lines to write back when the kernel ends; long32k
// and the 96-head DCP shard, 17-21%).  Smaller shares (ragged, verification, short
// histories: under 2%, or under 1 MB) are left in the caches for the merge.
constexpr int64_t kNtPartBytes = int64_t(4) << 20;

// Launch parameters of the LSE merge kernel.
enum MergeMode : int32_t { MERGE_GENERIC = 0, MERGE_DECODE = 1 };

struct MergeParams {
  const void* part_o;     // MERGE_GENERIC: [num_parts][rows][512]; MERGE_DECODE: layout above
  const float* part_lse;  // MERGE_GENERIC: [num_parts][rows]; MERGE_DECODE: [rows][slots]
  void* out;              // [groups * rows][512] or null
  float* out_lse;         // [groups * rows] or null
  int64_t rows;           // output rows per group (decode: T*H real rows)
  int32_t out_bf16;       // out element type: 1 bf16, 0 fp32
  // MERGE_GENERIC: slots [0, num_parts) for every row, groups = 1
  int32_t num_parts;
  // MERGE_DECODE: groups = batch, slot ranges from the split closed forms
  const int32_t* seq_lens;
  int32_t batch, max_pages, split_mode, num_wg, num_splits, num_slots;
  int64_t total_pages;    // P of the plan (SPLIT_BALANCED)
  PlanArgs plan;
};

}  // namespace mla
