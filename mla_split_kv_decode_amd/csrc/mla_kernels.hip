// gfx950 kernels of absorbed-MLA split-KV decode.
//
// Stage 1, mla_partial_kernel: one workgroup per piece list (see mla_internal.h).  For
// each piece (request, page range) it streams the latent pages into LDS and computes,
// for every query row of the request, the softmax-attention partial answer over the
// piece: O_p (normalised, fp32) and LSE_p.  Kimi K3 on MI355X, section 4 "MLA": the
// history is split into partitions handled by separate workgroups; section 1 "Cache",
// DCP8 paragraph: a partial answer carries its normalisation so pieces can be merged.
//
// Stage 2, mla_merge_kernel: the LSE-weighted merge of the partial answers of each row.
//
// Data movement.  A page (64 positions x 576 latent values) is copied from HBM straight
// into an LDS tile with global_load_lds_dwordx4 (no staging registers); two tiles per
// workgroup, so the next page streams in while the current one is consumed, and a piece
// of two pages has its whole history in flight at once.  Within a tile each 16-byte
// chunk of a row sits at an XOR-swizzled column so that the MFMA operand reads below hit
// distinct LDS banks; the DMA fills the tile in contiguous 1 KiB blocks and each lane
// fetches the global chunk that belongs at its slot.
//
// Matrix layout (all on the 16x16 MFMA grid, wave64):
//  * rows   : 16 query rows = 16 heads of one query token ("row block"); heads past the
//             real count are zero rows (section 4: padding heads leaves real heads
//             unchanged) that are never loaded or written.
//  * QK^T   : S^T[pos][row] = sum_k K[pos][k] Q[row][k] with v_mfma_f32_16x16x32_bf16,
//             A = 16 positions x 32 latent columns read from the LDS tile, B = the row
//             block's queries, kept in registers for the whole piece.
//  * PV     : O^T[col][row] += sum_pos V^T[col][pos] P^T[pos][row].  The S^T accumulator
//             layout (lane = row, 4 consecutive positions per lane) is already the B
//             layout of the next MFMA, so P never leaves registers (or, when several
//             waves share a row block, takes one small LDS exchange).  V^T is read from
//             the same LDS tile with the gfx950 transposing LDS reads (ds_read_b64_tr_b16
//             for bf16, ds_read_b64_tr_b8 for FP8), so each latent byte leaves HBM once.
//  * softmax: online, in log2 units; the row max is a 2-step cross-lane reduction and,
//             across waves of one row block, an LDS exchange.
#include <hip/hip_runtime.h>

#include "mla_internal.h"

// m0 is set inside the page-copy asm, the only user of m0 in these kernels
#pragma clang diagnostic ignored "-Winline-asm"

namespace mla {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;
typedef __attribute__((address_space(3))) void lds_void;

constexpr float kLn2 = 0.69314718055994531f;
constexpr float kLog2e = 1.44269504088896341f;
constexpr float kNegInf = -__builtin_inff();

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_fast(float x) { return __builtin_amdgcn_logf(x); }

// Wait until at most N vector-memory operations of this wave are outstanding (they
// complete in issue order).  gfx9 encoding: vmcnt in bits 3:0 and 15:14; expcnt and
// lgkmcnt fields at their maxima (no wait on them).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}

// Workgroup barrier for LDS traffic only: this wave's LDS operations complete, then the
// rendezvous.  Unlike __syncthreads() it does not wait for outstanding global loads, so
// page copies into the other tile stay in flight across it.  The empty asm statements
// keep the compiler from moving memory accesses across the barrier.
__device__ __forceinline__ void barrier_lds() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt, expcnt at their maxima
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// LDS reads of the small cross-wave exchange buffers, issued as inline assembly: the
// compiler cannot tell these buffers from the page tiles being filled by copies still in
// flight and would otherwise wait for all of them first.  Each call completes its reads
// (lgkmcnt(0)) before returning.  `off` is the LDS byte address.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
template <int G>
__device__ __forceinline__ float lds_max_of(const float* p, float init) {
  // max of p[0], p[16], ..., p[16 (G-1)] and init
  float v[4];
  if constexpr (G == 4) {
    asm volatile("ds_read_b32 %0, %4\n\tds_read_b32 %1, %4 offset:64\n\t"
                 "ds_read_b32 %2, %4 offset:128\n\tds_read_b32 %3, %4 offset:192\n\t"
                 "s_waitcnt lgkmcnt(0)"
                 : "=v"(v[0]), "=v"(v[1]), "=v"(v[2]), "=v"(v[3]) : "v"(lds_addr(p)));
    return fmaxf(fmaxf(fmaxf(init, v[0]), fmaxf(v[1], v[2])), v[3]);
  } else {
    static_assert(G == 2, "exchange width");
    asm volatile("ds_read_b32 %0, %2\n\tds_read_b32 %1, %2 offset:64\n\ts_waitcnt lgkmcnt(0)"
                 : "=v"(v[0]), "=v"(v[1]) : "v"(lds_addr(p)));
    return fmaxf(fmaxf(init, v[0]), v[1]);
  }
}
template <int G>
__device__ __forceinline__ float lds_sum_of(const float* p) {
  float v[4];
  if constexpr (G == 4) {
    asm volatile("ds_read_b32 %0, %4\n\tds_read_b32 %1, %4 offset:64\n\t"
                 "ds_read_b32 %2, %4 offset:128\n\tds_read_b32 %3, %4 offset:192\n\t"
                 "s_waitcnt lgkmcnt(0)"
                 : "=v"(v[0]), "=v"(v[1]), "=v"(v[2]), "=v"(v[3]) : "v"(lds_addr(p)));
    return ((v[0] + v[1]) + v[2]) + v[3];
  } else {
    static_assert(G == 2, "exchange width");
    asm volatile("ds_read_b32 %0, %2\n\tds_read_b32 %1, %2 offset:64\n\ts_waitcnt lgkmcnt(0)"
                 : "=v"(v[0]), "=v"(v[1]) : "v"(lds_addr(p)));
    return v[0] + v[1];
  }
}
// two 16-byte reads 1 KiB apart (the two 32-position P^T chunks of a row block)
__device__ __forceinline__ void lds_read_pair_b128(const void* p, i32x4& a, i32x4& b) {
  asm volatile("ds_read_b128 %0, %2\n\tds_read_b128 %1, %2 offset:1024\n\ts_waitcnt lgkmcnt(0)"
               : "=v"(a), "=v"(b) : "v"(lds_addr(p)));
}

// A load of one int32 through the vector memory path.  Uniform loads would otherwise be
// scalar loads, which the compiler waits for at once (they share a counter with LDS
// traffic); the zero added here is opaque to it, so the load stays a vector load that it
// tracks and waits for only where the value is used.
__device__ __forceinline__ int32_t vector_load_i32(const int32_t* p) {
  int32_t z;
  asm volatile("v_mov_b32 %0, 0" : "=v"(z));
  return p[z];
}

// Eight FP8 E4M3FN codes (little-endian bytes of `raw`) -> eight bf16, exactly.
__device__ __forceinline__ bf16x8 fp8x8_to_bf16x8(i32x2 raw) {
  bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw[0], 1.0f, false);
  bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw[0], 1.0f, true);
  bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw[1], 1.0f, false);
  bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw[1], 1.0f, true);
  return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

template <bool FP8>
struct TileGeom {
  static constexpr int kElem = FP8 ? 1 : 2;
  static constexpr int kRowBytes = kDLatent * kElem;     // one latent, in HBM and in LDS
  static constexpr int kChunksPerRow = kRowBytes / 16;   // 72 (bf16) or 36 (fp8)
  static constexpr int kPageBytes = kPage * kRowBytes;   // one page = one LDS tile
  static constexpr int kDmaOps = kPageBytes / 1024;      // 1 KiB wave-wide DMA blocks

  // LDS column of 16-byte chunk c of `row`: chunks are permuted within aligned groups
  // (8 for bf16, 4 for fp8) by an XOR with a row-dependent key.  An involution.
  // bf16: rows 2 apart fall on the same banks (1152-byte rows), so their keys must move
  // the 32-byte chunk pairs the transposing V^T reads take, not just swap within a pair;
  // over 16 rows the key is a bijection on even and on odd rows, which keeps the K
  // operand reads (one chunk of 16 rows) conflict-free as well.
  __device__ static constexpr int key16(int row) {
    return (((row >> 1) & 3) << 1) | ((row >> 3) & 1);
  }
  __device__ static __forceinline__ int swz(int row, int c) {
    if constexpr (FP8) return (c & ~3) | ((c & 3) ^ ((row >> 2) & 3));
    else return (c & ~7) | ((c & 7) ^ key16(row));
  }
  __device__ static __forceinline__ int offset(int row, int chunk) {
    return row * kRowBytes + swz(row, chunk) * 16;
  }
  // Byte offset of slot s (16 bytes) of a page in HBM that the copy puts at LDS slot s.
  __device__ static __forceinline__ int dma_src_offset(int s) {
    const int row = s / kChunksPerRow, cs = s - row * kChunksPerRow;
    return row * kRowBytes + swz(row, cs) * 16;
  }
};

// Per-lane LDS addressing of the MFMA operands.  The swizzle key of every row a lane
// reads is the same for all its reads, so each operand address is a per-lane base plus a
// compile-time offset (an instruction immediate).
//
// K (A operand of QK^T), 16x32 block of sub-tile pt and k-step kk:
//   kbase[kk & 1] + pt * 16 * kRowBytes + kstep(kk)
// V^T (A operand of PV), 32-position chunk c, half hh (positions +16), column tile ct of
// this wave: vbase[ct & 3] + c * 32 * kRowBytes + hh * 16 * kRowBytes + vstep(ct)
template <bool FP8>
struct OperandAddr {
  using TG = TileGeom<FP8>;
  int kbase[2];
  int vbase[4];
  __device__ __forceinline__ OperandAddr(int lrow, int lgrp, int wave_col_tile0) {
    if constexpr (FP8) {
      // K: row 16pt+lrow, chunk 2kk + (lgrp>>1), byte 8(lgrp&1); key (lrow>>2)&3
      const int key = (lrow >> 2) & 3;
#pragma unroll
      for (int e = 0; e < 2; ++e)
        kbase[e] = lrow * TG::kRowBytes + 16 * ((2 * e + (lgrp >> 1)) ^ key) + 8 * (lgrp & 1);
      // V^T (tr8): lane (lgrp, lrow = 2ii + h) reads row 32c + 16(ii>>2) + 4 lgrp + (ii&3),
      // chunk n = wave_col_tile0 + ct, byte 8h; key = lgrp
      const int ii = lrow >> 1, h = lrow & 1;
      const int row = 16 * (ii >> 2) + 4 * lgrp + (ii & 3);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        vbase[j] = row * TG::kRowBytes + 16 * (4 * (wave_col_tile0 >> 2) + (j ^ lgrp)) + 8 * h;
    } else {
      // K: row 16pt+lrow, chunk 4kk + lgrp; key key16(lrow)
      const int key = TG::key16(lrow);
#pragma unroll
      for (int e = 0; e < 2; ++e) kbase[e] = lrow * TG::kRowBytes + 16 * ((4 * e + lgrp) ^ key);
      // V^T (tr16): row 32c + 16hh + 4 lgrp + (lrow>>2), chunk 2n + ((lrow&3)>>1) with
      // n = wave_col_tile0 + ct, byte 8(lrow&1); key key16 of the row
      const int key_v = TG::key16(4 * lgrp + (lrow >> 2));
      const int row = 4 * lgrp + (lrow >> 2);
      const int b = (lrow & 3) >> 1;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        vbase[j] = row * TG::kRowBytes + 16 * (8 * (wave_col_tile0 >> 2) + ((2 * j + b) ^ key_v)) +
                   8 * (lrow & 1);
    }
  }
  __device__ static constexpr int kstep(int kk) { return (FP8 ? 64 : 128) * (kk >> 1); }
  // kbase[e] computed from e (for k-steps whose parity is known only at run time)
  __device__ static __forceinline__ int kbase_of(int lrow, int lgrp, int e) {
    if constexpr (FP8)
      return lrow * TG::kRowBytes + 16 * ((2 * e + (lgrp >> 1)) ^ ((lrow >> 2) & 3)) + 8 * (lgrp & 1);
    else
      return lrow * TG::kRowBytes + 16 * ((4 * e + lgrp) ^ TG::key16(lrow));
  }
  __device__ static constexpr int vstep(int ct) { return (FP8 ? 64 : 128) * (ct >> 2); }
};

// Copy one page from HBM into an LDS tile.  The tile is kDmaOps blocks of 1 KiB; block k
// is written by one wave-wide global_load_lds_dwordx4 in which lane l fills 16-byte slot
// 64k + l.  Every wave issues exactly kPer operations (blocks past the end repeat the
// last block: identical bytes to the identical place), so the per-wave count of
// outstanding operations per page is a compile-time constant.  Rows at or past
// `valid_rows` (the unwritten tail of a request's last page) are filled from the last
// valid row instead: their scores are masked, so only their finiteness matters (a zero
// softmax weight times a NaN left in the pool would still be NaN).
template <bool FP8, int NW>
struct PageCopy {
  using TG = TileGeom<FP8>;
  static constexpr int kPer = (TG::kDmaOps + NW - 1) / NW;
  int src_off[kPer];  // this lane's source offsets within a page, one per operation
  int wave, lane;
  __device__ __forceinline__ PageCopy(int wave_, int lane_) : wave(wave_), lane(lane_) {
#pragma unroll
    for (int j = 0; j < kPer; ++j) src_off[j] = TG::dma_src_offset(block(j) * 64 + lane);
  }
  __device__ __forceinline__ int block(int j) const {
    const int k = wave + NW * j;
    return k < TG::kDmaOps ? k : TG::kDmaOps - 1;
  }
  // The copies are issued as inline assembly so that the compiler neither delays LDS
  // reads of the other tiles behind them nor counts them: every wait on them is explicit
  // (wait_vmcnt), and they complete in issue order with the other vector-memory ops.
  __device__ __forceinline__ void operator()(unsigned char* tile, const unsigned char* src,
                                             int valid_rows) const {
    const uint32_t base = lds_addr(tile);
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      int off = src_off[j];
      if (valid_rows < kPage) {
        const int row = (block(j) * 64 + lane) / TG::kChunksPerRow;
        if (row >= valid_rows) off -= (row - (valid_rows - 1)) * TG::kRowBytes;
      }
      const uint32_t dst = __builtin_amdgcn_readfirstlane(base + block(j) * 1024);
      asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
                   :: "s"(dst), "v"(off), "s"(src) : "memory", "m0");
    }
  }
};

// Copy the queries of a workgroup's RB row blocks (request r) into an LDS staging area of
// RB x 16 rows of 576 bf16, laid out like a bf16 page tile (same chunk swizzle), so one
// HBM read serves every wave that shares a row block.  Row i of row block rb is head
// 16 hg + i of token t (rb = t * head_groups + hg); a padding head repeats the last real
// head (its results are discarded).  Same operation-count rule as PageCopy.
template <int NW, int RB>
struct QueryCopy {
  using TG = TileGeom<false>;
  static constexpr int kBlocks = RB * kRowsPerBlock * TG::kRowBytes / 1024;
  static constexpr int kPer = (kBlocks + NW - 1) / NW;
  int wave, lane;
  __device__ __forceinline__ QueryCopy(int wave_, int lane_) : wave(wave_), lane(lane_) {}
  __device__ __forceinline__ void operator()(unsigned char* stage, const uint16_t* q_req,
                                             int num_heads, int head_groups) const {
    const uint32_t base = lds_addr(stage);
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      int k = wave + NW * j;
      k = k < kBlocks ? k : kBlocks - 1;
      const int s = k * 64 + lane;
      const int row = s / TG::kChunksPerRow, cs = s - row * TG::kChunksPerRow;
      const int rb = row / kRowsPerBlock, i = row - rb * kRowsPerBlock;
      const int t = rb / head_groups, hg = rb - t * head_groups;
      const int head = min(hg * kRowsPerBlock + i, num_heads - 1);
      const int off = (t * num_heads + head) * TG::kRowBytes + TG::swz(row, cs) * 16;
      const uint32_t dst = __builtin_amdgcn_readfirstlane(base + k * 1024);
      asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
                   :: "s"(dst), "v"(off), "s"(q_req) : "memory", "m0");
    }
  }
};

// Wait until at most n * PER of this wave's vector-memory operations are outstanding,
// n in [0, NMAX] known only at run time (s_waitcnt takes an immediate).
template <int PER, int NMAX>
__device__ __forceinline__ void wait_pages(int n) {
  static_assert(NMAX <= 4, "wait cases");
  if (NMAX >= 4 && n >= 4) wait_vmcnt<(NMAX >= 4 ? 4 * PER : 0)>();
  else if (NMAX >= 3 && n == 3) wait_vmcnt<(NMAX >= 3 ? 3 * PER : 0)>();
  else if (NMAX >= 2 && n == 2) wait_vmcnt<(NMAX >= 2 ? 2 * PER : 0)>();
  else if (NMAX >= 1 && n == 1) wait_vmcnt<PER>();
  else wait_vmcnt<0>();
}

// Shape of the partial-attention workgroup.  RB row blocks of 16 query rows; G waves
// share a row block (they split its positions for QK^T and its output columns for PV);
// NG groups of RB * G waves run in lockstep on consecutive pages, each group on its own
// page, and combine their answers at the end of a piece.
template <bool FP8, int G_, int RB_, int NG_>
struct PartialCfg {
  static constexpr int G = G_, RB = RB_, NG = NG_;
  using TG = TileGeom<FP8>;
  static constexpr int WPG = RB * G;                // waves per group
  static constexpr int NW = NG * WPG;               // waves per workgroup
  static constexpr int NST = 4 / G;                 // 16-position sub-tiles of a page per wave
  static constexpr int CT = 32 / G;                 // 16-column output tiles per wave
  static constexpr int kTiles = FP8 ? 4 : 2;        // page tiles in LDS (147,456 bytes)
  static constexpr int kSIF = kTiles / NG;          // steps (NG pages each) in flight
  static constexpr int kPer = PageCopy<FP8, NW>::kPer;
  // queries go through LDS when several waves need the same row block
  static constexpr bool kQLds = G > 1 || NG > 1;
  static constexpr int kQPer = kQLds ? QueryCopy<NW, RB>::kPer : 0;
  static constexpr int kQTiles =
      kQLds ? (QueryCopy<NW, RB>::kBlocks * 1024 + TG::kPageBytes - 1) / TG::kPageBytes : 0;
  static constexpr int kXBytes = G > 1 ? NG * RB * 2 * 64 * 16 : 16;  // P exchange
  static_assert(G == 1 || G == 2 || G == 4, "waves per row block");
  static_assert(RB >= 1 && RB <= kMaxRowBlocks && NW <= 16, "workgroup shape");
  static_assert(kTiles % NG == 0 && kQTiles < kTiles, "tile plan");
  static_assert(kPer * kTiles + kQPer <= 63, "outstanding operations exceed vmcnt");
  static_assert(NG == 1 || G > 1, "the group combine relies on the denominator barrier");
};

// Every scalar argument a partial-stage prologue needs, fetched in one batch: the compiler
// would otherwise load some fields lazily inside branches, one memory round trip each,
// before the first page copy can be issued.
struct HotArgs {
  int heads, hgroups, mode, nwg, nsplits, plan_n, len0, maxp, batch, qlen, causal, nslots, pbf16;
  int64_t total, npages;
  float sscale, vscale;
  __device__ __forceinline__ explicit HotArgs(const PartialParams& p)
      : heads(p.num_heads), hgroups(p.head_groups), mode(p.mode), nwg(p.num_wg),
        nsplits(p.num_splits), plan_n(p.plan.n), len0(p.plan.len[0]), maxp(p.max_pages),
        batch(p.batch), qlen(p.q_len), causal(p.causal), nslots(p.num_slots), pbf16(p.part_bf16),
        total(p.total_pages), npages(p.num_pages), sscale(p.score_scale), vscale(p.v_scale) {
    asm volatile("" ::"s"(heads), "s"(hgroups), "s"(mode), "s"(nwg), "s"(nsplits), "s"(plan_n),
                 "s"(len0), "s"(maxp), "s"(batch), "s"(qlen), "s"(causal), "s"(nslots), "s"(pbf16),
                 "s"(total), "s"(npages), "s"(sscale), "s"(vscale));
  }
};

// The pieces of workgroup blockIdx.x (mla_internal.h): run(r, first page, end page, slot, L)
// for each, from the plan's lengths in the arguments when present, else from seq_lens.
template <class F>
__device__ __forceinline__ void for_each_piece(const PartialParams& p, const HotArgs& a,
                                               const int32_t* __restrict__ seq_lens, F&& run_piece) {
  const int64_t w = blockIdx.x;
  const bool use_plan = a.plan_n > 0;
  if (a.mode == SPLIT_FIXED) {
    const int S = a.nsplits;
    const int r = (int)(w / S), sp = (int)(w - (int64_t)r * S);
    const int L = use_plan ? (a.plan_n == 1 ? a.len0 : p.plan.len[r]) : max(seq_lens[r], 0);
    const int pages = pages_of(L, a.maxp);
    run_piece(r, fixed_page_begin(sp, pages, S), fixed_page_begin(sp + 1, pages, S), w, L);
  } else if (a.plan_n == 1) {  // one request: its pages are the whole page axis
    const int64_t gb = balanced_start(w, a.total, a.nwg), ge = balanced_start(w + 1, a.total, a.nwg);
    run_piece(0, (int)gb, (int)ge, w, a.len0);
  } else if (use_plan) {
    const int64_t P = a.total;
    const int64_t gb = balanced_start(w, P, a.nwg), ge = balanced_start(w + 1, P, a.nwg);
    for (int r = 0; r < a.plan_n; ++r) {
      const int64_t pre = p.plan.pre[r], nxt = p.plan.pre[r + 1];
      if (nxt <= gb) continue;
      if (pre >= ge) break;
      const int L = p.plan.len[r];
      const int64_t lo = gb > pre ? gb : pre, hi = ge < nxt ? ge : nxt;
      run_piece(r, (int)(lo - pre), (int)(hi - pre), w + r, L);
    }
  } else {
    int64_t P = 0;
    for (int r = 0; r < a.batch; ++r) P += pages_of(seq_lens[r], a.maxp);
    // Device lengths that disagree with the plan's: no piece is computed and the merge
    // writes NaN (the split below would not match the merge's slot ranges).
    if (P == 0 || P != a.total) return;
    const int64_t gb = balanced_start(w, P, a.nwg), ge = balanced_start(w + 1, P, a.nwg);
    int64_t pre = 0;
    for (int r = 0; r < a.batch && pre < ge; ++r) {
      const int L = max(seq_lens[r], 0);
      const int pr = pages_of(L, a.maxp);
      const int64_t lo = gb > pre ? gb : pre;
      const int64_t hi = ge < pre + pr ? ge : pre + pr;
      if (lo < hi) run_piece(r, (int)(lo - pre), (int)(hi - pre), w + r, L);
      pre += pr;
    }
  }
}

// Partial answer of one row of one piece to the workspace layout of mla_internal.h:
// four consecutive columns starting at `col`.
__device__ __forceinline__ void store_partial(void* part_o, bool bf16, int64_t orow, int col,
                                              int nslots, int64_t slot, f32x4 v) {
  const int64_t idx = ((orow * kMergeChunks + (col >> 5)) * nslots + slot) * kMergeCols + (col & 31);
  if (bf16)
    *(bf16x4*)((__bf16*)part_o + idx) = bf16x4{(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
  else
    *(f32x4*)((float*)part_o + idx) = v;
}

template <class C>
struct PartialSmem {
  using TG = typename C::TG;
  __attribute__((aligned(1024))) unsigned char tiles[C::kTiles * TG::kPageBytes];
  __attribute__((aligned(16))) unsigned char pbuf[C::kXBytes];  // P of a step
  float red[C::NW * 16];   // row maxima of a step
  float red2[C::NW * 16];  // row denominators of the epilogue
  float xch[C::NG * C::RB * 16 * 2];
};

// Stage 1 for workgroup blockIdx.x: every piece it owns, partial answers to the workspace.
// The device pointers are separate __restrict__ arguments: read-only, never aliased by
// the output stores, so uniform reads (lengths, page ids) become scalar loads.
template <bool FP8, class C>
__device__ __forceinline__ void partial_phase(
    const PartialParams& p, const uint16_t* __restrict__ q_ptr, const uint8_t* __restrict__ pool,
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ seq_lens,
    void* __restrict__ part_o, float* __restrict__ part_lse, PartialSmem<C>& sm) {
  using TG = TileGeom<FP8>;
  using Copy = PageCopy<FP8, C::NW>;
  constexpr int G = C::G, RB = C::RB, NG = C::NG, WPG = C::WPG, NST = C::NST, CT = C::CT;
  constexpr int kTiles = C::kTiles, kSIF = C::kSIF, kPer = C::kPer;
  constexpr int kEarlyTiles = kTiles - C::kQTiles;  // tiles not used to stage the queries

  const HotArgs args(p);
  const int a_heads = args.heads, a_hgroups = args.hgroups, a_maxp = args.maxp;
  const int a_qlen = args.qlen, a_causal = args.causal, a_nslots = args.nslots, a_pbf16 = args.pbf16;
  const int64_t a_npages = args.npages;
  const float a_sscale = args.sscale, a_vscale = args.vscale;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int lrow = lane & 15, lgrp = lane >> 4;
  const int grp = wave / WPG, wig = wave - grp * WPG;  // group, wave in group
  const int rb = wig / G, g = wig - (wig / G) * G;
  const int t = rb / a_hgroups, hg = rb - t * a_hgroups;
  const int head = hg * kRowsPerBlock + lrow;
  const bool head_ok = head < a_heads;
  const Copy copy(wave, lane);
  const OperandAddr<FP8> addr(lrow, lgrp, g * CT);
  unsigned char* const tiles = sm.tiles;
  unsigned char* const pbuf = sm.pbuf;
  float* const red = sm.red;

  // One piece: request r of length L, local pages [pb, pe), partial slot `slot`.  With
  // the plan's lengths in the arguments no device length is read here (a pending load of
  // it would be waited for at the first page copy's inline assembly): the merge stage
  // compares the device lengths with the plan's.
  auto run_piece = [&](int r, int pb, int pe, int64_t slot, int L) {
    const int limit = a_causal ? L - a_qlen + t + 1 : L;  // visible: position < limit
    const int32_t* trow = block_table + (int64_t)r * a_maxp;
    const int n = pe - pb;                   // pages of the piece
    const int nsteps = (n + NG - 1) / NG;    // step s: page s * NG + group
    bool bad = false;

    // A page id outside the pool is never dereferenced: the copy reads page 0 instead
    // (keeping the per-wave operation count) and the piece's result becomes NaN.
    auto issue = [&](int s, int gi) {
      const int i = s * NG + gi;
      if (i >= n) return;
      const int lp = pb + i;
      int32_t id = trow[lp];
      if ((uint64_t)(int64_t)id >= (uint64_t)a_npages) {
        bad = true;
        id = 0;
      }
      const int valid_rows = min(kPage, L - lp * kPage);
      copy(tiles + ((s % kSIF) * NG + gi) * TG::kPageBytes, pool + (int64_t)id * TG::kPageBytes,
           valid_rows);
    };

    // ---- queries and the first pages
    i32x4 qf[kDLatent / 32];
    const uint16_t* q_req = q_ptr + (int64_t)r * a_qlen * a_heads * kDLatent;
    if constexpr (C::kQLds) {
      unsigned char* stage = tiles + kEarlyTiles * TG::kPageBytes;
      QueryCopy<C::NW, RB>(wave, lane)(stage, q_req, a_heads, a_hgroups);
      int early = 0;
#pragma unroll
      for (int ti = 0; ti < kEarlyTiles; ++ti) {
        issue(ti / NG, ti % NG);
        early += (ti < n) ? 1 : 0;
      }
      wait_pages<kPer, kEarlyTiles>(early);  // the query copies are older: all landed
      barrier_lds();
      const OperandAddr<false> qa(lrow, lgrp, 0);
      const unsigned char* qb = stage + rb * kRowsPerBlock * TileGeom<false>::kRowBytes;
#pragma unroll
      for (int kk = 0; kk < kDLatent / 32; ++kk)
        qf[kk] = *(const i32x4*)(qb + qa.kbase[kk & 1] + OperandAddr<false>::kstep(kk));
      barrier_lds();  // the staging tiles are free again
#pragma unroll
      for (int ti = kEarlyTiles; ti < kTiles; ++ti) issue(ti / NG, ti % NG);
    } else {
      // One wave per row block: the page copies go out first, then the queries as
      // ordinary loads.  The compiler waits for those at the next inline assembly (the
      // first step's wait), so that step also waits for the prefetched pages; later steps
      // are unaffected.  A padding row repeats the last real head.
#pragma unroll
      for (int ti = 0; ti < kTiles; ++ti) issue(ti / NG, ti % NG);
      const int hq = head_ok ? head : a_heads - 1;
      const uint16_t* qrow = q_req + ((int64_t)t * a_heads + hq) * kDLatent + lgrp * 8;
#pragma unroll
      for (int kk = 0; kk < kDLatent / 32; ++kk) qf[kk] = *(const i32x4*)(qrow + kk * 32);
    }

    float m = kNegInf;   // running max of this lane's row (log2 units)
    float lsum = 0.f;    // this lane's share of the running denominator
    f32x4 acc[CT];
#pragma unroll
    for (int i = 0; i < CT; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int s = 0; s < nsteps; ++s) {
      // pages of steps s+1 .. s+kSIF-1 were issued after this step's: let them fly
      wait_pages<kPer, (kSIF - 1) * NG>(min(n, (s + kSIF) * NG) - min(n, (s + 1) * NG));
      barrier_lds();  // every wave's copies of this step have landed
      const int i = s * NG + grp;
      const bool has = i < n;  // uniform in the group
      const unsigned char* tile = tiles + ((s % kSIF) * NG + grp) * TG::kPageBytes;
      const int lp = pb + i;

      // ---- S^T = K Q^T for this wave's sub-tiles, scale, mask, tile max.  When registers
      // allow (a wave with at most 8 output column tiles), the V^T operands of the first
      // PV chunk are read right after the QK^T MFMAs are issued: they do not depend on the
      // softmax, so those transposing LDS reads run under the MFMAs and the exchanges.
      constexpr int kEarly = CT <= 8 ? 1 : 0;  // PV chunks whose operands are read early
      f32x4 sv[NST];
      bf16x8 va[2][CT];
      auto read_v = [&](int c) {
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          const unsigned char* va0 =
              tile + c * 32 * TG::kRowBytes + addr.vbase[ct & 3] + OperandAddr<FP8>::vstep(ct);
          if constexpr (FP8) {
            va[c][ct] = fp8x8_to_bf16x8(__builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)va0));
          } else {
            const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)va0);
            const bf16x4 hi =
                __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(va0 + 16 * TG::kRowBytes));
            va[c][ct] = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          }
        }
      };
      float mx = kNegInf;
      if (has) {
#pragma unroll
        for (int u = 0; u < NST; ++u) {
          const unsigned char* kt = tile + (g * NST + u) * 16 * TG::kRowBytes;
          bf16x8 kf[kDLatent / 32];
#pragma unroll
          for (int kk = 0; kk < kDLatent / 32; ++kk) {
            const unsigned char* ka = kt + addr.kbase[kk & 1] + OperandAddr<FP8>::kstep(kk);
            if constexpr (FP8) kf[kk] = fp8x8_to_bf16x8(*(const i32x2*)ka);
            else kf[kk] = *(const bf16x8*)ka;
          }
          // one accumulation chain in k-step order (dependent MFMAs forward their
          // accumulator), so that each MFMA consumes the oldest outstanding K read
          f32x4 a0 = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kk = 0; kk < kDLatent / 32; ++kk)
            a0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[kk], __builtin_bit_cast(bf16x8, qf[kk]),
                                                         a0, 0, 0, 0);
          sv[u] = a0;
          if constexpr (kEarly > 0) read_v(0);  // kEarly implies one sub-tile per wave
          if constexpr (!FP8) {
            // Instruction order of the sub-tile: six K reads ahead, then one MFMA per
            // read, so LDS latency hides under the MFMAs; the early V^T reads go between
            // the last six MFMAs.  (Left alone, the scheduler keeps only one or two reads
            // ahead and each MFMA waits for its operand.)
            __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
#pragma unroll
            for (int i = 0; i < 12; ++i) {
              __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
              __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
            if constexpr (kEarly > 0) {
              static_assert(NST == 1 && 2 * CT == 16, "early V^T reads: one chunk, 16 reads");
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
              }
#pragma unroll
              for (int i = 0; i < 2; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
              }
            } else {
              __builtin_amdgcn_sched_group_barrier(0x008, 6, 0);
            }
          }
        }
        const int pos0 = lp * kPage;
#pragma unroll
        for (int u = 0; u < NST; ++u) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int j = pos0 + (g * NST + u) * 16 + lgrp * 4 + e;
            const float v = j < limit ? sv[u][e] * a_sscale : kNegInf;
            sv[u][e] = v;
            mx = fmaxf(mx, v);
          }
        }
      } else {
#pragma unroll
        for (int u = 0; u < NST; ++u) sv[u] = f32x4{kNegInf, kNegInf, kNegInf, kNegInf};
      }
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      if constexpr (G > 1) {
        if (lgrp == 0) red[(grp * WPG + rb * G + g) * 16 + lrow] = mx;
        barrier_lds();
        mx = lds_max_of<G>(&red[(grp * WPG + rb * G) * 16 + lrow], mx);
      }

      // ---- online softmax update
      const float m_new = fmaxf(m, mx);
      const float msub = m_new == kNegInf ? 0.f : m_new;
      const float alpha = exp2_fast(m - msub);  // m = -inf -> 0
      m = m_new;
      float ps = 0.f;
      bf16x8 pf[2];
#pragma unroll
      for (int u = 0; u < NST; ++u) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float pv = exp2_fast(sv[u][e] - msub);
          sv[u][e] = pv;
          ps += pv;
        }
      }
      lsum = lsum * alpha + ps;
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) acc[ct] *= alpha;

      // ---- P^T as the B operand of the PV MFMA: slots 0-3 = positions 4*lgrp+0..3 of
      // the chunk's first 16-position sub-tile, slots 4-7 = the same of its second.
      if constexpr (G == 1) {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          pf[c] = bf16x8{(__bf16)sv[2 * c][0], (__bf16)sv[2 * c][1], (__bf16)sv[2 * c][2],
                         (__bf16)sv[2 * c][3], (__bf16)sv[2 * c + 1][0], (__bf16)sv[2 * c + 1][1],
                         (__bf16)sv[2 * c + 1][2], (__bf16)sv[2 * c + 1][3]};
        }
      } else {
        unsigned char* pb_rb = pbuf + (grp * RB + rb) * 2 * 64 * 16;
#pragma unroll
        for (int u = 0; u < NST; ++u) {
          const int pt = g * NST + u;
          bf16x4 v = bf16x4{(__bf16)sv[u][0], (__bf16)sv[u][1], (__bf16)sv[u][2], (__bf16)sv[u][3]};
          *(bf16x4*)(pb_rb + ((pt >> 1) * 64 + lane) * 16 + (pt & 1) * 8) = v;
        }
        barrier_lds();
        i32x4 p0, p1;
        lds_read_pair_b128(pb_rb + lane * 16, p0, p1);
        pf[0] = __builtin_bit_cast(bf16x8, p0);
        pf[1] = __builtin_bit_cast(bf16x8, p1);
      }

      // ---- O^T += V^T P^T over the page's two 32-position chunks
      if (has) {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          if (c >= kEarly) read_v(c);
#pragma unroll
          for (int ct = 0; ct < CT; ++ct)
            acc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[c][ct], pf[c], acc[ct], 0, 0, 0);
        }
      }

      // The next copies into this step's tiles wait until every wave is done with them.
      // Without copies (the last steps) no barrier is needed: the exchange buffers of the
      // next step are written only after its own first barrier, and the epilogue uses
      // buffers of its own (the group combine reuses the tiles only after the
      // denominator barrier, by which every wave has finished its last V^T reads).
      if ((s + kSIF) * NG < n) {
        barrier_lds();
#pragma unroll
        for (int gi = 0; gi < NG; ++gi) issue(s + kSIF, gi);
      }
    }

    // ---- epilogue: partial answers go to [row][32-column chunk][slot][32] (bf16 or fp32)
    const int64_t orow = (int64_t)t * a_heads + head;
    auto store_o = [&](int ct, f32x4 v) {
      store_partial(part_o, a_pbf16, orow, g * CT * 16 + ct * 16 + lgrp * 4, a_nslots, slot, v);
    };
    // the group's full row denominator
    float ls = lsum;
    ls += __shfl_xor(ls, 16);
    ls += __shfl_xor(ls, 32);
    if constexpr (G > 1) {
      if (lgrp == 0) sm.red2[(grp * WPG + rb * G + g) * 16 + lrow] = ls;
      barrier_lds();
      ls = lds_sum_of<G>(&sm.red2[(grp * WPG + rb * G) * 16 + lrow]);
    }
    if constexpr (NG == 1) {
      const bool empty = m == kNegInf;
      float oscale = empty ? 0.f : a_vscale / ls;
      float lse = empty ? kNegInf : (m + log2_fast(ls)) * kLn2;
      if (bad) {
        oscale = __builtin_nanf("");
        lse = __builtin_nanf("");
      }
      if (head_ok) {
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) store_o(ct, acc[ct] * oscale);
        if (g == 0 && lgrp == 0) part_lse[orow * a_nslots + slot] = lse;
      }
    } else {
      // ---- the two groups combine: (m, l) through LDS, then each wave keeps half of its
      // output columns and receives its partner's (same row block and columns, other
      // group) copy of that half through the now idle page tiles.
      static_assert(NG == 2 && CT % 2 == 0, "group combine");
      constexpr int H2 = CT / 2;
      float* xm = sm.xch + ((grp * RB + rb) * 16 + lrow) * 2;
      if (g == 0 && lgrp == 0) {
        xm[0] = m;
        xm[1] = ls;
      }
      float* xa = (float*)tiles;  // [wave][H2][64 lanes][4]
#pragma unroll
      for (int c = 0; c < H2; ++c) {
        const f32x4 v = grp == 0 ? acc[H2 + c] : acc[c];
        *(f32x4*)(xa + ((wave * H2 + c) * 64 + lane) * 4) = v;
      }
      barrier_lds();
      const float* xo = sm.xch + (((1 - grp) * RB + rb) * 16 + lrow) * 2;
      const float m_o = xo[0], l_o = xo[1];
      const float M = fmaxf(m, m_o);
      const float Msub = M == kNegInf ? 0.f : M;
      const float a_s = exp2_fast(m - Msub), a_o = exp2_fast(m_o - Msub);
      const float Lsum = a_s * ls + a_o * l_o;
      const bool empty = M == kNegInf;
      float oscale = empty ? 0.f : a_vscale / Lsum;
      float lse = empty ? kNegInf : (M + log2_fast(Lsum)) * kLn2;
      if (bad) {
        oscale = __builtin_nanf("");
        lse = __builtin_nanf("");
      }
      const int partner = (1 - grp) * WPG + wig;
      const float* xp = xa + (partner * H2 * 64 + lane) * 4;
      if (head_ok) {
        if (grp == 0) {
#pragma unroll
          for (int c = 0; c < H2; ++c) {
            const f32x4 o = *(const f32x4*)(xp + c * 64 * 4);
            store_o(c, (acc[c] * a_s + o * a_o) * oscale);
          }
          if (g == 0 && lgrp == 0) part_lse[orow * a_nslots + slot] = lse;
        } else {
#pragma unroll
          for (int c = 0; c < H2; ++c) {
            const f32x4 o = *(const f32x4*)(xp + c * 64 * 4);
            store_o(H2 + c, (acc[H2 + c] * a_s + o * a_o) * oscale);
          }
        }
      }
    }
    barrier_lds();  // tiles and exchange buffers are reused by the next piece
  };

  for_each_piece(p, args, seq_lens, run_piece);
}


// ------------------------------------------------------------------- K-split partial stage
//
// One row block of 16 query rows (one query token, up to 16 heads), eight waves per
// workgroup, all on the same page.  In QK^T wave w computes the partial scores of the
// 16-position sub-tile u = w & 3 over half kh = w >> 2 of the latent (nine of the 18
// k-steps of 32 columns); the two halves are added through LDS.  In PV wave w produces
// output columns [64 w, 64 w + 64) over the page's 64 positions.  One softmax state for the
// whole workgroup, pages double-buffered (FP8: four in flight), and a page is processed as
// soon as it has landed, so once the stream ends only the last page's work remains.
template <bool FP8>
struct KSplitCfg {
  using TG = TileGeom<FP8>;
  static constexpr int NW = 8;
  static constexpr int kTiles = FP8 ? 4 : 2;
  static constexpr int kPer = PageCopy<FP8, NW>::kPer;
  static constexpr int KS = kDLatent / 32 / 2;  // k-steps per half: 9
  static constexpr int CT = 4;                  // 16-column output tiles per wave
  static constexpr int kQTiles =
      (QueryCopy<NW, 1>::kBlocks * 1024 + TG::kPageBytes - 1) / TG::kPageBytes;
  static_assert(kPer * kTiles + QueryCopy<NW, 1>::kPer <= 63, "outstanding operations exceed vmcnt");
  static_assert(kQTiles < kTiles, "tile plan");
};

template <bool FP8>
struct KSplitSmem {
  using C = KSplitCfg<FP8>;
  __attribute__((aligned(1024))) unsigned char tiles[C::kTiles * C::TG::kPageBytes];
  f32x4 sx[4][64];                                               // k-half 1 partial scores
  __attribute__((aligned(16))) unsigned char pbuf[2 * 64 * 16];  // P^T of the page, bf16
  float red[4 * 16];                                             // row maxima of the sub-tiles
  float red2[4 * 16];                                            // row denominators (epilogue)
};

template <bool FP8>
__device__ __forceinline__ void partial_ks(
    const PartialParams& p, const uint16_t* __restrict__ q_ptr, const uint8_t* __restrict__ pool,
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ seq_lens,
    void* __restrict__ part_o, float* __restrict__ part_lse, KSplitSmem<FP8>& sm) {
  using C = KSplitCfg<FP8>;
  using TG = TileGeom<FP8>;
  constexpr int kTiles = C::kTiles, kPer = C::kPer, CT = C::CT, KS = C::KS;
  constexpr int kEarlyTiles = kTiles - C::kQTiles;  // tiles not used to stage the queries
  const HotArgs args(p);

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int lrow = lane & 15, lgrp = lane >> 4;
  const int u = wave & 3, kh = wave >> 2;  // sub-tile, k-half
  const int head = lrow;                   // one token: rows are the heads
  const bool head_ok = head < args.heads;
  const PageCopy<FP8, C::NW> copy(wave, lane);
  const OperandAddr<FP8> addr(lrow, lgrp, 4 * wave);  // V^T: output column tiles 4w .. 4w+3
  unsigned char* const tiles = sm.tiles;

  auto run_piece = [&](int r, int pb, int pe, int64_t slot, int L) {
    const int32_t* trow = block_table + (int64_t)r * args.maxp;
    const int n = pe - pb;
    bool bad = false;
    // page i of the piece into tile i % kTiles; an id outside the pool is never
    // dereferenced (page 0 is copied instead, the piece becomes NaN)
    auto issue = [&](int i) {
      if (i >= n) return;
      const int lp = pb + i;
      int32_t id = trow[lp];
      if ((uint64_t)(int64_t)id >= (uint64_t)args.npages) {
        bad = true;
        id = 0;
      }
      copy(tiles + (i % kTiles) * TG::kPageBytes, pool + (int64_t)id * TG::kPageBytes,
           min(kPage, L - lp * kPage));
    };

    // ---- queries through LDS (one HBM read per workgroup), then the first pages
    unsigned char* stage = tiles + kEarlyTiles * TG::kPageBytes;
    QueryCopy<C::NW, 1>(wave, lane)(stage, q_ptr + (int64_t)r * args.heads * kDLatent, args.heads, 1);
    int early = 0;
#pragma unroll
    for (int ti = 0; ti < kEarlyTiles; ++ti) {
      issue(ti);
      early += ti < n ? 1 : 0;
    }
    wait_pages<kPer, kEarlyTiles>(early);  // the query copies are older: all landed
    barrier_lds();
    i32x4 qf[KS];  // this wave's half of the queries
    {
#pragma unroll
      for (int j = 0; j < KS; ++j) {
        const int kk = kh * KS + j;  // depends on the wave: offsets computed, not indexed
        const int kb = OperandAddr<false>::kbase_of(lrow, lgrp, kk & 1);
        qf[j] = *(const i32x4*)(stage + kb + OperandAddr<false>::kstep(kk));
      }
    }
    barrier_lds();  // the staging tiles are free again
#pragma unroll
    for (int ti = kEarlyTiles; ti < kTiles; ++ti) issue(ti);

    float m = kNegInf;  // running row max (log2 units), the same in every wave
    float lsum = 0.f;   // k-half 0 waves: this lane's share of its sub-tile's denominator
    f32x4 acc[CT];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) acc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int i = 0; i < n; ++i) {
      // pages i+1 .. i+kTiles-1 were issued after page i: let them fly
      wait_pages<kPer, kTiles - 1>(min(n, i + kTiles) - (i + 1));
      barrier_lds();  // every wave's copies of page i have landed
      const unsigned char* tile = tiles + (i % kTiles) * TG::kPageBytes;
      const int lp = pb + i;

      // ---- partial S^T of sub-tile u over this wave's k-half, then the V^T operands of
      // this wave's output columns (both 32-position chunks; they do not depend on the
      // softmax, so these transposing reads run under the MFMAs and the exchanges)
      const unsigned char* kt = tile + u * 16 * TG::kRowBytes;
      bf16x8 kf[KS];
#pragma unroll
      for (int j = 0; j < KS; ++j) {
        const int kk = kh * KS + j;
        const unsigned char* ka =
            kt + OperandAddr<FP8>::kbase_of(lrow, lgrp, kk & 1) + OperandAddr<FP8>::kstep(kk);
        if constexpr (FP8) kf[j] = fp8x8_to_bf16x8(*(const i32x2*)ka);
        else kf[j] = *(const bf16x8*)ka;
      }
      f32x4 sp = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < KS; ++j)
        sp = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[j], __builtin_bit_cast(bf16x8, qf[j]), sp, 0, 0, 0);
      bf16x8 va[2][CT];
#pragma unroll
      for (int c = 0; c < 2; ++c) {
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          const unsigned char* va0 = tile + c * 32 * TG::kRowBytes + addr.vbase[ct] + OperandAddr<FP8>::vstep(ct);
          if constexpr (FP8) {
            va[c][ct] = fp8x8_to_bf16x8(__builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)va0));
          } else {
            const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)va0);
            const bf16x4 hi =
                __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(va0 + 16 * TG::kRowBytes));
            va[c][ct] = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          }
        }
      }
      if constexpr (!FP8) {
        // instruction order: six K reads ahead of the MFMAs, then one MFMA per remaining
        // read; the sixteen V^T reads go between the last six MFMAs
        __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
#pragma unroll
        for (int j = 0; j < 3; ++j) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
      }

      // ---- the k-halves meet: half 1 hands its partial scores to half 0, which scales,
      // masks and takes its sub-tile's row max
      if (kh == 1) sm.sx[u][lane] = sp;
      barrier_lds();
      f32x4 sv = f32x4{kNegInf, kNegInf, kNegInf, kNegInf};
      if (kh == 0) {
        const f32x4 other = sm.sx[u][lane];
        float mx = kNegInf;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int j = lp * kPage + u * 16 + lgrp * 4 + e;
          const float v = j < L ? (sp[e] + other[e]) * args.sscale : kNegInf;
          sv[e] = v;
          mx = fmaxf(mx, v);
        }
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        if (lgrp == 0) sm.red[u * 16 + lrow] = mx;
      }
      barrier_lds();
      const float mx = lds_max_of<4>(&sm.red[lrow], kNegInf);

      // ---- online softmax update; half 0 builds P^T of its sub-tile for every wave
      const float m_new = fmaxf(m, mx);
      const float msub = m_new == kNegInf ? 0.f : m_new;
      const float alpha = exp2_fast(m - msub);  // m = -inf -> 0
      m = m_new;
      if (kh == 0) {
        float ps = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sv[e] = exp2_fast(sv[e] - msub);
          ps += sv[e];
        }
        lsum = lsum * alpha + ps;
        *(bf16x4*)(sm.pbuf + ((u >> 1) * 64 + lane) * 16 + (u & 1) * 8) =
            bf16x4{(__bf16)sv[0], (__bf16)sv[1], (__bf16)sv[2], (__bf16)sv[3]};
      }
      barrier_lds();
      i32x4 p0, p1;
      lds_read_pair_b128(sm.pbuf + lane * 16, p0, p1);
      const bf16x8 pf[2] = {__builtin_bit_cast(bf16x8, p0), __builtin_bit_cast(bf16x8, p1)};

      // ---- O^T += V^T P^T for this wave's 64 columns
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) acc[ct] *= alpha;
#pragma unroll
      for (int c = 0; c < 2; ++c) {
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
          acc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[c][ct], pf[c], acc[ct], 0, 0, 0);
      }

      // the next copy into this tile waits until every wave is done with it
      if (i + kTiles < n) {
        barrier_lds();
        issue(i + kTiles);
      }
    }

    // ---- epilogue: the row denominator from the four k-half 0 waves, normalise, store
    float ls = lsum;
    ls += __shfl_xor(ls, 16);
    ls += __shfl_xor(ls, 32);
    if (kh == 0 && lgrp == 0) sm.red2[u * 16 + lrow] = ls;
    barrier_lds();
    ls = lds_sum_of<4>(&sm.red2[lrow]);
    const bool empty = m == kNegInf;
    float oscale = empty ? 0.f : args.vscale / ls;
    float lse = empty ? kNegInf : (m + log2_fast(ls)) * kLn2;
    if (bad) {
      oscale = __builtin_nanf("");
      lse = __builtin_nanf("");
    }
    if (head_ok) {
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
        store_partial(part_o, args.pbf16, head, 64 * wave + 16 * ct + 4 * lgrp, args.nslots, slot,
                      acc[ct] * oscale);
      if (wave == 0 && lgrp == 0) part_lse[(int64_t)head * args.nslots + slot] = lse;
    }
    barrier_lds();  // tiles and exchange buffers are reused by the next piece
  };

  for_each_piece(p, args, seq_lens, run_piece);
}

// ------------------------------------------------------------------- merge
//
// A merge unit is (output row, 32-column chunk).  Thread (slot lane sl, column piece cp)
// owns 16 bytes of each of slots s0 + sl, s0 + sl + SPP, ...: 8 columns of bf16 parts or
// 4 of fp32 parts.  A round of 256 slots per unit has all its loads (O pieces and LSEs)
// in flight together, so a merge of up to 256 parts costs one memory round trip.

constexpr int kMergeThreads = 256;
constexpr int kMergeWaves = kMergeThreads / 64;

__device__ __forceinline__ float nan_max(float a, float b) {
  // a NaN LSE (a piece that met a bad page id) must reach the output
  return a != a ? a : (b != b ? b : fmaxf(a, b));
}

template <bool PART_BF16>
struct MergeGeom {
  static constexpr int kCPT = PART_BF16 ? 8 : 4;          // columns per thread
  static constexpr int kTPS = kMergeCols / kCPT;          // threads per slot
  static constexpr int kSPP = kMergeThreads / kTPS;       // slots per pass
  static constexpr int kPasses = 256 / kSPP;              // passes per round of 256 slots
};

template <bool PART_BF16>
__device__ __forceinline__ void load_piece(const void* base, int64_t idx, float (&v)[MergeGeom<PART_BF16>::kCPT]) {
  if constexpr (PART_BF16) {
    const bf16x8 b = *(const bf16x8*)((const __bf16*)base + idx);
#pragma unroll
    for (int c = 0; c < 8; ++c) v[c] = (float)b[c];
  } else {
    const f32x4 f = *(const f32x4*)((const float*)base + idx);
#pragma unroll
    for (int c = 0; c < 4; ++c) v[c] = f[c];
  }
}

template <bool PART_BF16, bool OUT_BF16, bool DECODE>
__global__ __launch_bounds__(kMergeThreads) void mla_merge_kernel(MergeParams p) {
  using MG = MergeGeom<PART_BF16>;
  constexpr int kCPT = MG::kCPT, kTPS = MG::kTPS, kSPP = MG::kSPP, kPasses = MG::kPasses;
  __shared__ float sm_m[kMergeWaves];
  __shared__ float sm_acc[kMergeWaves][kTPS][kCPT];
  __shared__ float sm_den[kMergeWaves];

  // scalar arguments of the prologue in one batch (see partial_phase)
  const int64_t a_rows = p.rows, a_total = p.total_pages;
  const int a_nwg = p.num_wg, a_nsplits = p.num_splits, a_mode = p.split_mode, a_plan_n = p.plan.n;
  const int a_nparts = p.num_parts, a_nslots = p.num_slots, a_len0 = p.plan.len[0];
  asm volatile("" ::"s"(a_rows), "s"(a_total), "s"(a_nwg), "s"(a_nsplits), "s"(a_mode), "s"(a_plan_n),
               "s"(a_nparts), "s"(a_nslots), "s"(a_len0));

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int sl = tid / kTPS, cp = tid - (tid / kTPS) * kTPS;
  const int64_t unit = blockIdx.x;
  const int64_t orow = unit / kMergeChunks;
  const int chunk = (int)(unit - orow * kMergeChunks);
  const int64_t grp = (int64_t)((uint32_t)orow / (uint32_t)a_rows);  // rows * groups < 2^31
  const int64_t row = orow - grp * a_rows;

  // slot range [s0, s1) of this group.  Under SPLIT_BALANCED every workgroup owns at
  // least one page (W <= P), so every slot in the range holds a piece.
  int64_t s0 = 0, s1 = 0;
  bool inconsistent = false;
  // plan path: the device length (a vector load, waited for only where it is compared,
  // after the partial answers have been loaded) must equal the plan's
  int dev_len = 0, plan_len = 0;
  if constexpr (!DECODE) {
    s1 = a_nparts;
  } else if (a_plan_n == 1) {  // one request
    dev_len = vector_load_i32(p.seq_lens);
    plan_len = a_len0;
    s1 = a_mode == SPLIT_FIXED ? a_nsplits : a_nwg;
  } else if (a_plan_n > 0) {
    // slot range from the plan's lengths; the device length is only compared with it
    dev_len = vector_load_i32(p.seq_lens + grp);
    plan_len = p.plan.len[grp];
    if (a_mode == SPLIT_FIXED) {
      s0 = grp * a_nsplits;
      s1 = s0 + a_nsplits;
    } else {
      const int64_t pre = p.plan.pre[grp], pr = p.plan.pre[grp + 1] - pre;
      s0 = balanced_wg_of(pre, a_total, a_nwg) + grp;
      s1 = balanced_wg_of(pre + pr - 1, a_total, a_nwg) + grp + 1;
    }
  } else if (a_mode == SPLIT_FIXED) {
    s0 = grp * a_nsplits;
    s1 = s0 + a_nsplits;
  } else {
    int64_t P = 0, pre = 0, pr = 0;
    for (int r = 0; r < p.batch; ++r) {
      const int pg = pages_of(p.seq_lens[r], p.max_pages);
      if (r < grp) pre += pg;
      if (r == grp) pr = pg;
      P += pg;
    }
    inconsistent = P != p.total_pages;
    if (pr > 0 && !inconsistent) {
      s0 = balanced_wg_of(pre, P, p.num_wg) + grp;
      s1 = balanced_wg_of(pre + pr - 1, P, p.num_wg) + grp + 1;
    }
  }
  const int64_t col = (int64_t)chunk * kMergeCols + cp * kCPT;
  auto o_index = [&](int64_t s) -> int64_t {
    if constexpr (DECODE) return ((row * kMergeChunks + chunk) * a_nslots + s) * kMergeCols + cp * kCPT;
    else return (s * a_rows + row) * kDV + col;
  };
  auto lse_index = [&](int64_t s) -> int64_t {
    if constexpr (DECODE) return row * a_nslots + s;
    else return s * a_rows + row;
  };

  // first round: loads of O and LSE together
  float o[kPasses][kCPT];
  float l[kPasses];
#pragma unroll
  for (int k = 0; k < kPasses; ++k) {
    const int64_t s = s0 + sl + kSPP * k;
    const bool ok = s < s1;
    l[k] = ok ? p.part_lse[lse_index(s)] : kNegInf;
    if (ok) load_piece<PART_BF16>(p.part_o, o_index(s), o[k]);
    else {
#pragma unroll
      for (int c = 0; c < kCPT; ++c) o[k][c] = 0.f;
    }
  }
  // M over all slots (later rounds: LSEs only)
  float mx = kNegInf;
  inconsistent = inconsistent || dev_len != plan_len;
#pragma unroll
  for (int k = 0; k < kPasses; ++k) mx = nan_max(mx, l[k]);
  for (int64_t s = s0 + 256 + tid; s < s1; s += kMergeThreads) mx = nan_max(mx, p.part_lse[lse_index(s)]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) mx = nan_max(mx, __shfl_xor(mx, off));
  if (lane == 0) sm_m[wave] = mx;
  __syncthreads();
  float M = sm_m[0];
#pragma unroll
  for (int wv = 1; wv < kMergeWaves; ++wv) M = nan_max(M, sm_m[wv]);

  float acc[kCPT];
#pragma unroll
  for (int c = 0; c < kCPT; ++c) acc[c] = 0.f;
  float den = 0.f;
  if (M != kNegInf) {
#pragma unroll
    for (int k = 0; k < kPasses; ++k) {
      const float a = exp2_fast((l[k] - M) * kLog2e);  // empty slots: exp2(-inf) = 0
#pragma unroll
      for (int c = 0; c < kCPT; ++c) acc[c] += a * o[k][c];
      den += a;
    }
    for (int64_t base = s0 + 256; base < s1; base += 256) {
#pragma unroll
      for (int k = 0; k < kPasses; ++k) {
        const int64_t s = base + sl + kSPP * k;
        if (s >= s1) continue;
        const float a = exp2_fast((p.part_lse[lse_index(s)] - M) * kLog2e);
        float v[kCPT];
        load_piece<PART_BF16>(p.part_o, o_index(s), v);
#pragma unroll
        for (int c = 0; c < kCPT; ++c) acc[c] += a * v[c];
        den += a;
      }
    }
  }
  // sum over the slot lanes: lanes cp + kTPS k of a wave, then the waves.  Every thread of
  // a slot lane holds the same weights, so the denominator is summed over slot lanes only.
#pragma unroll
  for (int off = kTPS; off < 64; off <<= 1) {
#pragma unroll
    for (int c = 0; c < kCPT; ++c) acc[c] += __shfl_xor(acc[c], off);
    den += __shfl_xor(den, off);
  }
  if (lane < kTPS) {
#pragma unroll
    for (int c = 0; c < kCPT; ++c) sm_acc[wave][lane][c] = acc[c];
    if (lane == 0) sm_den[wave] = den;
  }
  __syncthreads();
  if (tid < kTPS) {
    float v[kCPT];
    float d = sm_den[0];
#pragma unroll
    for (int c = 0; c < kCPT; ++c) v[c] = sm_acc[0][tid][c];
#pragma unroll
    for (int wv = 1; wv < kMergeWaves; ++wv) {
#pragma unroll
      for (int c = 0; c < kCPT; ++c) v[c] += sm_acc[wv][tid][c];
      d += sm_den[wv];
    }
    const bool empty = M == kNegInf && !inconsistent;
    const float inv = 1.0f / d;
#pragma unroll
    for (int c = 0; c < kCPT; ++c) {
      v[c] = empty ? 0.f : v[c] * inv;
      if (inconsistent) v[c] = __builtin_nanf("");
    }
    if (p.out) {
      const int64_t off = orow * kDV + col;
      if constexpr (OUT_BF16) {
#pragma unroll
        for (int c = 0; c < kCPT; c += 4)
          *(bf16x4*)((__bf16*)p.out + off + c) =
              bf16x4{(__bf16)v[c], (__bf16)v[c + 1], (__bf16)v[c + 2], (__bf16)v[c + 3]};
      } else {
#pragma unroll
        for (int c = 0; c < kCPT; c += 4)
          *(f32x4*)((float*)p.out + off + c) = f32x4{v[c], v[c + 1], v[c + 2], v[c + 3]};
      }
    }
    if (p.out_lse && chunk == 0 && tid == 0) {
      p.out_lse[orow] =
          inconsistent ? __builtin_nanf("") : (empty ? kNegInf : M + log2_fast(d) * kLn2);
    }
  }
}

// ------------------------------------------------------------------- kernels

// The workgroup shape for RB row blocks (see PartialCfg): one row block uses two groups
// of 4 waves, two row blocks two groups of 2 waves per row block, so the four SIMDs each
// run two waves; larger counts use one wave (two for three blocks) per row block.
template <bool FP8, int RB>
struct CfgFor;
template <bool FP8> struct CfgFor<FP8, 2> { using type = PartialCfg<FP8, 2, 2, 2>; };
template <bool FP8> struct CfgFor<FP8, 3> { using type = PartialCfg<FP8, 2, 3, 1>; };
template <bool FP8> struct CfgFor<FP8, 4> { using type = PartialCfg<FP8, 1, 4, 1>; };
template <bool FP8> struct CfgFor<FP8, 5> { using type = PartialCfg<FP8, 1, 5, 1>; };
template <bool FP8> struct CfgFor<FP8, 6> { using type = PartialCfg<FP8, 1, 6, 1>; };
template <bool FP8> struct CfgFor<FP8, 7> { using type = PartialCfg<FP8, 1, 7, 1>; };
template <bool FP8> struct CfgFor<FP8, 8> { using type = PartialCfg<FP8, 1, 8, 1>; };

// LDS (the page tiles) caps residency at one workgroup per compute unit; the register
// budget is what that workgroup's waves per SIMD allow.
template <bool FP8, class C>
__global__ __launch_bounds__(C::NW * 64)
__attribute__((amdgpu_waves_per_eu((C::NW + 3) / 4, (C::NW + 3) / 4))) void mla_partial_kernel(
    PartialParams p, const uint16_t* __restrict__ q_ptr, const uint8_t* __restrict__ pool,
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ seq_lens,
    void* __restrict__ part_o, float* __restrict__ part_lse) {
  __shared__ PartialSmem<C> sm;
  partial_phase<FP8, C>(p, q_ptr, pool, block_table, seq_lens, part_o, part_lse, sm);
}


// One row block (one token, up to 16 heads): the K-split workgroup of eight waves.
template <bool FP8>
__global__ __launch_bounds__(KSplitCfg<FP8>::NW * 64)
__attribute__((amdgpu_waves_per_eu(2, 2))) void mla_partial_ks_kernel(
    PartialParams p, const uint16_t* __restrict__ q_ptr, const uint8_t* __restrict__ pool,
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ seq_lens,
    void* __restrict__ part_o, float* __restrict__ part_lse) {
  __shared__ KSplitSmem<FP8> sm;
  partial_ks<FP8>(p, q_ptr, pool, block_table, seq_lens, part_o, part_lse, sm);
}

// ------------------------------------------------------------------ launchers

namespace {

template <bool FP8, class C>
hipError_t launch_partial_t(const PartialParams& p, hipStream_t stream) {
  hipLaunchKernelGGL((mla_partial_kernel<FP8, C>), dim3(p.num_wg), dim3(C::NW * 64), 0, stream, p,
                     p.q, p.pool, p.block_table, p.seq_lens, p.part_o, p.part_lse);
  return hipGetLastError();
}

template <bool FP8>
hipError_t launch_partial_ks(const PartialParams& p, hipStream_t stream) {
  hipLaunchKernelGGL((mla_partial_ks_kernel<FP8>), dim3(p.num_wg), dim3(KSplitCfg<FP8>::NW * 64), 0,
                     stream, p, p.q, p.pool, p.block_table, p.seq_lens, p.part_o, p.part_lse);
  return hipGetLastError();
}

// row blocks 2 .. 8 (one row block takes the K-split kernel)
template <bool FP8, template <bool, class> class F, class... A>
auto by_row_blocks(int rb, A&&... a) {
  switch (rb) {
    case 2: return F<FP8, typename CfgFor<FP8, 2>::type>::run(a...);
    case 3: return F<FP8, typename CfgFor<FP8, 3>::type>::run(a...);
    case 4: return F<FP8, typename CfgFor<FP8, 4>::type>::run(a...);
    case 5: return F<FP8, typename CfgFor<FP8, 5>::type>::run(a...);
    case 6: return F<FP8, typename CfgFor<FP8, 6>::type>::run(a...);
    case 7: return F<FP8, typename CfgFor<FP8, 7>::type>::run(a...);
    default: return F<FP8, typename CfgFor<FP8, 8>::type>::run(a...);
  }
}

template <bool FP8, class C>
struct PartialLaunch {
  static hipError_t run(const PartialParams& p, hipStream_t s) { return launch_partial_t<FP8, C>(p, s); }
};
template <bool FP8, class C>
struct PartialLds {
  static size_t run() { return sizeof(PartialSmem<C>); }
};

}  // namespace

// LDS bytes of one partial-stage workgroup, for the planner's residency estimate.
size_t partial_lds_size(bool fp8, int row_blocks) {
  if (row_blocks < 1 || row_blocks > kMaxRowBlocks) return 0;
  if (row_blocks == 1) return fp8 ? sizeof(KSplitSmem<true>) : sizeof(KSplitSmem<false>);
  return fp8 ? by_row_blocks<true, PartialLds>(row_blocks) : by_row_blocks<false, PartialLds>(row_blocks);
}

hipError_t launch_partial(const PartialParams& p, bool fp8, hipStream_t stream) {
  const int rb = p.q_len * p.head_groups;
  if (rb < 1 || rb > kMaxRowBlocks) return hipErrorInvalidValue;
  if (rb == 1) return fp8 ? launch_partial_ks<true>(p, stream) : launch_partial_ks<false>(p, stream);
  return fp8 ? by_row_blocks<true, PartialLaunch>(rb, p, stream)
             : by_row_blocks<false, PartialLaunch>(rb, p, stream);
}

hipError_t launch_merge(const MergeParams& p, bool part_bf16, bool decode, int64_t total_rows,
                        hipStream_t stream) {
  const dim3 grid((unsigned)(total_rows * kMergeChunks));
  const int sel = (part_bf16 ? 4 : 0) + (p.out_bf16 ? 2 : 0) + (decode ? 1 : 0);
  switch (sel) {
#define MLA_MERGE_CASE(S, A, B, D) \
    case S: hipLaunchKernelGGL((mla_merge_kernel<A, B, D>), grid, dim3(kMergeThreads), 0, stream, p); break;
    MLA_MERGE_CASE(0, false, false, false)
    MLA_MERGE_CASE(1, false, false, true)
    MLA_MERGE_CASE(2, false, true, false)
    MLA_MERGE_CASE(3, false, true, true)
    MLA_MERGE_CASE(4, true, false, false)
    MLA_MERGE_CASE(5, true, false, true)
    MLA_MERGE_CASE(6, true, true, false)
    MLA_MERGE_CASE(7, true, true, true)
#undef MLA_MERGE_CASE
  }
  return hipGetLastError();
}

}  // namespace mla
