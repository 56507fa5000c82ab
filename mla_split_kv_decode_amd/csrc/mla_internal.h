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
//  * SPLIT_BALANCED (num_splits = 0): W workgroups, W <= P.  Workgroup w takes global
//    pages [floor(w P / W), floor((w+1) P / W)), which may span several requests.  Each
//    (workgroup, request) overlap is one piece with its own partial answer, stored in
//    slot w + r.  Along the global axis both w and r only grow, so no two pieces share
//    a slot, and the pieces of request r occupy the contiguous slot range
//    [wg_of(pre_r) + r, wg_of(pre_r + pages_r - 1) + r].  Slots: W + B - 1.
//  * SPLIT_FIXED (num_splits = S >= 1): W = B * S workgroups; workgroup w = r S + s takes
//    the request's local pages [floor(s pages_r / S), floor((s+1) pages_r / S)) and slot
//    w.  A piece may be empty (pages_r < S); it then stores LSE = -inf and O = 0.
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
constexpr int kMaxRowBlocks = 8;   // q_len * ceil(heads / 16) limit of one workgroup

enum SplitMode : int32_t { SPLIT_BALANCED = 0, SPLIT_FIXED = 1 };

// Control words at the end of the workspace (fused launch): [0] barrier arrivals,
// [1] barrier generation, [2] marker that the words were initialised.
constexpr int kCtrlWords = 4;
constexpr int kCtrlMagicWord = 2;
constexpr uint32_t kCtrlMagic = 0x4D4C4131u;
constexpr size_t kCtrlBytes = 256;

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

// First global page of workgroup w under SPLIT_BALANCED.
MLA_HD int64_t balanced_start(int64_t w, int64_t P, int64_t W) { return div_floor(w * P, W); }

// Workgroup holding global page g under SPLIT_BALANCED (largest w with start(w) <= g).
MLA_HD int64_t balanced_wg_of(int64_t g, int64_t P, int64_t W) { return div_floor((g + 1) * W - 1, P); }

MLA_HD int32_t fixed_page_begin(int32_t s, int32_t pages, int32_t S) {
  return (int32_t)(((int64_t)s * pages) / S);
}

// Launch parameters of the partial-attention kernel.
struct PartialParams {
  const uint16_t* q;          // bf16 [B][T][H][576]
  const uint8_t* pool;        // [num_pages][64][576] of the KV element type
  const int32_t* block_table; // [B][max_pages]
  const int32_t* seq_lens;    // [B]
  float* part_o;              // fp32 [slots][T*H][512]
  float* part_lse;            // fp32 [slots][T*H]
  int64_t num_pages;
  int32_t max_pages;
  int32_t batch, q_len, num_heads, head_groups, rows;  // rows = T * H
  int32_t causal;
  int32_t mode;       // SplitMode
  int32_t num_wg;     // W
  int32_t num_splits; // S (SPLIT_FIXED)
  int64_t total_pages; // P from the plan's host copy of seq_lens (SPLIT_BALANCED)
  float score_scale;  // softmax_scale * log2(e) * kv_scale: scores in log2 units
  float v_scale;      // kv_scale applied to the value rows (1 for bf16)
};

// Launch parameters of the LSE merge kernel.
enum MergeMode : int32_t { MERGE_GENERIC = 0, MERGE_DECODE = 1 };

struct MergeParams {
  const void* part_o;     // [slots][part_rows][512] fp32 or bf16
  const float* part_lse;  // [slots][part_rows]
  void* out;              // [groups * rows][512] or null
  float* out_lse;         // [groups * rows] or null
  int64_t rows;           // output rows per group (decode: T*H real rows)
  int64_t part_rows;      // row stride of one slot
  int32_t part_bf16;      // part_o element type: 1 bf16, 0 fp32
  int32_t out_bf16;       // out element type: 1 bf16, 0 fp32
  int32_t mode;           // MergeMode
  // MERGE_GENERIC: slots [0, num_parts) for every row, groups = 1
  int32_t num_parts;
  // MERGE_DECODE: groups = batch, slot ranges from the split closed forms
  const int32_t* seq_lens;
  int32_t batch, max_pages, split_mode, num_wg, num_splits;
  int64_t total_pages;    // P of the plan (SPLIT_BALANCED)
};

}  // namespace mla
