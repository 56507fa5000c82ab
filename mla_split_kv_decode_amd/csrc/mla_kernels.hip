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
  __device__ static __forceinline__ int swz(int row, int c) {
    if constexpr (FP8) return (c & ~3) | ((c & 3) ^ ((row >> 2) & 3));
    else return (c & ~7) | ((c & 7) ^ ((row >> 1) & 7));
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
      // K: row 16pt+lrow, chunk 4kk + lgrp; key (lrow>>1)&7
      const int key = (lrow >> 1) & 7;
#pragma unroll
      for (int e = 0; e < 2; ++e) kbase[e] = lrow * TG::kRowBytes + 16 * ((4 * e + lgrp) ^ key);
      // V^T (tr16): row 32c + 16hh + 4 lgrp + (lrow>>2), chunk 2n + ((lrow&3)>>1) with
      // n = wave_col_tile0 + ct, byte 8(lrow&1); key (2 lgrp + (lrow>>3)) & 7
      const int key_v = (2 * lgrp + (lrow >> 3)) & 7;
      const int row = 4 * lgrp + (lrow >> 2);
      const int b = (lrow & 3) >> 1;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        vbase[j] = row * TG::kRowBytes + 16 * (8 * (wave_col_tile0 >> 2) + ((2 * j + b) ^ key_v)) +
                   8 * (lrow & 1);
    }
  }
  __device__ static constexpr int kstep(int kk) { return (FP8 ? 64 : 128) * (kk >> 1); }
  __device__ static constexpr int vstep(int ct) { return (FP8 ? 64 : 128) * (ct >> 2); }
};

// Copy one page from HBM into an LDS tile.  The tile is kDmaOps blocks of 1 KiB; block k
// is written by one wave-wide global_load_lds_dwordx4 in which lane l fills 16-byte slot
// 64k + l.  Every wave issues exactly kPer operations (blocks past the end repeat the
// last block: identical bytes to the identical place), so the per-wave count of
// outstanding operations per page is a compile-time constant.
template <bool FP8, int NW>
struct PageCopy {
  using TG = TileGeom<FP8>;
  static constexpr int kPer = (TG::kDmaOps + NW - 1) / NW;
  int src_off[kPer];  // this lane's source offsets within a page, one per operation
  int wave;
  __device__ __forceinline__ PageCopy(int wave_, int lane) : wave(wave_) {
#pragma unroll
    for (int j = 0; j < kPer; ++j) src_off[j] = TG::dma_src_offset(block(j) * 64 + lane);
  }
  __device__ __forceinline__ int block(int j) const {
    const int k = wave + NW * j;
    return k < TG::kDmaOps ? k : TG::kDmaOps - 1;
  }
  // The copies are issued as inline assembly so that the compiler neither delays LDS
  // reads of the other tile behind them nor counts them: every wait on them is explicit
  // (wait_vmcnt), and they complete in issue order with the other vector-memory ops.
  __device__ __forceinline__ void operator()(unsigned char* tile, const unsigned char* src) const {
    const uint32_t base = lds_addr(tile);
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const uint32_t dst = __builtin_amdgcn_readfirstlane(base + block(j) * 1024);
      asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
                   :: "s"(dst), "v"(src_off[j]), "s"(src) : "memory", "m0");
    }
  }
};

// Stage 1 for workgroup blockIdx.x: every piece it owns, partial answers to the workspace.
// The device pointers are separate __restrict__ arguments: read-only, never aliased by
// the output stores, so uniform reads (lengths, page ids) become scalar loads.
template <bool FP8, int G, int NW>
__device__ __forceinline__ void partial_phase(
    const PartialParams& p, const uint16_t* __restrict__ q_ptr, const uint8_t* __restrict__ pool,
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ seq_lens,
    float* __restrict__ part_o, float* __restrict__ part_lse, unsigned char* tile0,
    unsigned char* tile1, unsigned char* pbuf, float* red) {
  using TG = TileGeom<FP8>;
  using Copy = PageCopy<FP8, NW>;
  constexpr int RB = NW / G;                        // row blocks of the workgroup
  constexpr int NST = 4 / G;                        // 16-position sub-tiles of a page per wave
  constexpr int CT = 32 / G;                        // 16-column output tiles per wave
  constexpr int kPer = Copy::kPer;                  // copy operations per wave per page
  static_assert(RB * G == NW && RB <= kMaxRowBlocks, "wave layout");

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int lrow = lane & 15, lgrp = lane >> 4;
  const int rb = wave / G, g = wave - (wave / G) * G;
  const int t = rb / p.head_groups, hg = rb - t * p.head_groups;
  const int head = hg * kRowsPerBlock + lrow;
  const bool head_ok = head < p.num_heads;
  const Copy copy(wave, lane);
  const OperandAddr<FP8> addr(lrow, lgrp, g * CT);

  // One piece: request r, local pages [pb, pe), partial slot `slot`.
  auto run_piece = [&](int r, int pb, int pe, int64_t slot) {
    const int L = max(seq_lens[r], 0);
    const int limit = p.causal ? L - p.q_len + t + 1 : L;  // visible: position < limit
    const int32_t* trow = block_table + (int64_t)r * p.max_pages;
    const int npages = pe - pb;
    bool bad = false;

    // A page id outside the pool is never dereferenced: the copy reads page 0 instead
    // (keeping the per-wave operation count) and the piece's result becomes NaN.
    auto page_src = [&](int lp) -> const unsigned char* {
      int32_t id = trow[lp];
      if ((uint64_t)(int64_t)id >= (uint64_t)p.num_pages) {
        bad = true;
        id = 0;
      }
      return pool + (int64_t)id * TG::kPageBytes;
    };

    // Queries: ordinary loads issued before the page copies.  The compiler tracks them,
    // and since it does not see the copies, its wait before their first use drains the
    // copies too: both first pages have landed when the first page is consumed.  In
    // exchange the queries never queue behind the page stream.  A padding row repeats
    // the last real head: its outputs are discarded and rows are independent in every
    // step, so its content does not matter.
    i32x4 qf[kDLatent / 32];
    {
      const int hq = head_ok ? head : p.num_heads - 1;
      const uint16_t* qrow =
          q_ptr + (((int64_t)r * p.q_len + t) * p.num_heads + hq) * kDLatent + lgrp * 8;
#pragma unroll
      for (int kk = 0; kk < kDLatent / 32; ++kk) qf[kk] = *(const i32x4*)(qrow + kk * 32);
    }
    asm volatile("" ::: "memory");  // the query loads are issued before the copies
    if (npages > 0) copy(tile0, page_src(pb));
    if (npages > 1) copy(tile1, page_src(pb + 1));

    float m = kNegInf;   // running max of this lane's row (log2 units)
    float lsum = 0.f;    // this lane's share of the running denominator
    f32x4 acc[CT];
#pragma unroll
    for (int i = 0; i < CT; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto process = [&](unsigned char* tile, int i) {
      // this wave's copies of page i (and everything older) done, then everyone's
      if (i + 1 < npages) wait_vmcnt<kPer>();
      else wait_vmcnt<0>();
      barrier_lds();
      const int lp = pb + i;
      const int valid_rows = max(min(kPage, L - lp * kPage), 0);
      if (valid_rows < kPage) {  // rows past the end hold poison: zero them (P = 0 there)
        for (int idx = tid; idx < (kPage - valid_rows) * TG::kChunksPerRow; idx += NW * 64) {
          const int row = valid_rows + idx / TG::kChunksPerRow;
          const int col = idx % TG::kChunksPerRow;
          *(i32x4*)(tile + row * TG::kRowBytes + col * 16) = i32x4{0, 0, 0, 0};
        }
        barrier_lds();
      }

      // ---- S^T = K Q^T for this wave's sub-tiles
      f32x4 s[NST];
#pragma unroll
      for (int u = 0; u < NST; ++u) {
        const unsigned char* kt = tile + (g * NST + u) * 16 * TG::kRowBytes;
        // all K operands of the sub-tile in flight before the first MFMA
        bf16x8 kf[kDLatent / 32];
#pragma unroll
        for (int kk = 0; kk < kDLatent / 32; ++kk) {
          const unsigned char* ka = kt + addr.kbase[kk & 1] + OperandAddr<FP8>::kstep(kk);
          if constexpr (FP8) kf[kk] = fp8x8_to_bf16x8(*(const i32x2*)ka);
          else kf[kk] = *(const bf16x8*)ka;
        }
        __builtin_amdgcn_sched_barrier(0);  // keep every read ahead of the MFMAs
        // two independent accumulation chains (even / odd k-steps)
        f32x4 a0 = f32x4{0.f, 0.f, 0.f, 0.f}, a1 = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < kDLatent / 32; kk += 2) {
          a0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[kk], __builtin_bit_cast(bf16x8, qf[kk]),
                                                       a0, 0, 0, 0);
          a1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              kf[kk + 1], __builtin_bit_cast(bf16x8, qf[kk + 1]), a1, 0, 0, 0);
        }
        s[u] = a0 + a1;
      }

      // ---- scale, mask, tile max
      const int pos0 = lp * kPage;
      float mx = kNegInf;
#pragma unroll
      for (int u = 0; u < NST; ++u) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int j = pos0 + (g * NST + u) * 16 + lgrp * 4 + e;
          const float v = j < limit ? s[u][e] * p.score_scale : kNegInf;
          s[u][e] = v;
          mx = fmaxf(mx, v);
        }
      }
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      if constexpr (G > 1) {
        if (lgrp == 0) red[(rb * G + g) * 16 + lrow] = mx;
        barrier_lds();
        mx = lds_max_of<G>(&red[rb * G * 16 + lrow], mx);
      }

      // ---- online softmax update
      const float m_new = fmaxf(m, mx);
      const float msub = m_new == kNegInf ? 0.f : m_new;
      const float alpha = exp2_fast(m - msub);  // m = -inf -> 0
      m = m_new;
      float ps = 0.f;
#pragma unroll
      for (int u = 0; u < NST; ++u) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float pv = exp2_fast(s[u][e] - msub);
          s[u][e] = pv;
          ps += pv;
        }
      }
      lsum = lsum * alpha + ps;
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) acc[ct] *= alpha;

      // ---- P^T as the B operand of the PV MFMA: slots 0-3 = positions 4*lgrp+0..3 of
      // the chunk's first 16-position sub-tile, slots 4-7 = the same of its second.
      bf16x8 pf[2];
      if constexpr (G == 1) {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          pf[c] = bf16x8{(__bf16)s[2 * c][0], (__bf16)s[2 * c][1], (__bf16)s[2 * c][2],
                         (__bf16)s[2 * c][3], (__bf16)s[2 * c + 1][0], (__bf16)s[2 * c + 1][1],
                         (__bf16)s[2 * c + 1][2], (__bf16)s[2 * c + 1][3]};
        }
      } else {
#pragma unroll
        for (int u = 0; u < NST; ++u) {
          const int pt = g * NST + u;
          bf16x4 v = bf16x4{(__bf16)s[u][0], (__bf16)s[u][1], (__bf16)s[u][2], (__bf16)s[u][3]};
          *(bf16x4*)(pbuf + ((rb * 2 + (pt >> 1)) * 64 + lane) * 16 + (pt & 1) * 8) = v;
        }
        barrier_lds();
        i32x4 p0, p1;
        lds_read_pair_b128(pbuf + (rb * 2 * 64 + lane) * 16, p0, p1);
        pf[0] = __builtin_bit_cast(bf16x8, p0);
        pf[1] = __builtin_bit_cast(bf16x8, p1);
      }

      // ---- O^T += V^T P^T over the page's two 32-position chunks; each chunk's V^T
      // operands are read (transposing LDS reads) before its MFMAs are issued
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        bf16x8 va[CT];
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          const unsigned char* va0 =
              tile + c * 32 * TG::kRowBytes + addr.vbase[ct & 3] + OperandAddr<FP8>::vstep(ct);
          if constexpr (FP8) {
            va[ct] = fp8x8_to_bf16x8(__builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)va0));
          } else {
            const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)va0);
            const bf16x4 hi =
                __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(va0 + 16 * TG::kRowBytes));
            va[ct] = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          }
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
          acc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[ct], pf[c], acc[ct], 0, 0, 0);
      }

      barrier_lds();  // every wave is done with this tile
      if (i + 2 < npages) copy(tile, page_src(pb + i + 2));
    };

    for (int i = 0; i < npages; i += 2) {
      process(tile0, i);
      if (i + 1 < npages) process(tile1, i + 1);
    }

    // ---- epilogue: full row denominator, normalise, store the partial answer
    float ls = lsum;
    ls += __shfl_xor(ls, 16);
    ls += __shfl_xor(ls, 32);
    if constexpr (G > 1) {
      barrier_lds();
      if (lgrp == 0) red[(rb * G + g) * 16 + lrow] = ls;
      barrier_lds();
      ls = lds_sum_of<G>(&red[rb * G * 16 + lrow]);
    }
    const bool empty = m == kNegInf;
    float oscale = empty ? 0.f : p.v_scale / ls;
    float lse = empty ? kNegInf : (m + log2_fast(ls)) * kLn2;
    if (bad) {
      oscale = __builtin_nanf("");
      lse = __builtin_nanf("");
    }
    if (head_ok) {
      const int64_t orow = (int64_t)t * p.num_heads + head;
      float* dst = part_o + (slot * p.rows + orow) * kDV + g * CT * 16 + lgrp * 4;
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) *(f32x4*)(dst + ct * 16) = acc[ct] * oscale;
      if (g == 0 && lgrp == 0) part_lse[slot * p.rows + orow] = lse;
    }
    barrier_lds();  // tiles and exchange buffers are reused by the next piece
  };

  const int64_t w = blockIdx.x;
  if (p.mode == SPLIT_FIXED) {
    const int S = p.num_splits;
    const int r = (int)(w / S), sp = (int)(w - (int64_t)r * S);
    const int pages = pages_of(seq_lens[r], p.max_pages);
    run_piece(r, fixed_page_begin(sp, pages, S), fixed_page_begin(sp + 1, pages, S), w);
  } else {
    int64_t P = 0;
    for (int r = 0; r < p.batch; ++r) P += pages_of(seq_lens[r], p.max_pages);
    // Device lengths that disagree with the plan's: no piece is computed and the merge
    // writes NaN (the split below would not match the merge's slot ranges).
    if (P == 0 || P != p.total_pages) return;
    const int64_t gb = balanced_start(w, P, p.num_wg), ge = balanced_start(w + 1, P, p.num_wg);
    int64_t pre = 0;
    for (int r = 0; r < p.batch && pre < ge; ++r) {
      const int pr = pages_of(seq_lens[r], p.max_pages);
      const int64_t lo = gb > pre ? gb : pre;
      const int64_t hi = ge < pre + pr ? ge : pre + pr;
      if (lo < hi) run_piece(r, (int)(lo - pre), (int)(hi - pre), w + r);
      pre += pr;
    }
  }
}

// ------------------------------------------------------------------- merge
//
// A merge unit is (output row, 32-column chunk).  Thread (part lane pl, column quad cq)
// owns parts s0 + pl, s0 + pl + 32, ...; a round of 8 parts per lane (256 parts per unit)
// has all its loads (O quads and LSEs) in flight together, so a merge of up to 256 parts
// costs one memory round trip.

constexpr int kMergeCols = 32;
constexpr int kMergeThreads = 256;
constexpr int kMergeQuads = kMergeCols / 4;            // 8
constexpr int kMergeLanes = kMergeThreads / kMergeQuads;  // 32 part lanes
constexpr int kMergeUnroll = 8;                        // parts per lane per round
constexpr int kMergeRound = kMergeLanes * kMergeUnroll;   // 256
constexpr int kMergeChunks = kDV / kMergeCols;         // 16 units per output row

__device__ __forceinline__ float nan_max(float a, float b) {
  // a NaN LSE (a piece that met a bad page id) must reach the output
  return a != a ? a : (b != b ? b : fmaxf(a, b));
}

struct MergeScratch {
  float m[kMergeThreads / 64];
  f32x4 v[kMergeThreads / 64][kMergeQuads];
  float s[kMergeThreads / 64][kMergeQuads];
};

// Runs with any block of at least kMergeThreads threads; threads past kMergeThreads only
// take part in the barriers.
template <bool PART_BF16, bool OUT_BF16>
__device__ __forceinline__ void merge_unit(const MergeParams& p, int64_t unit, MergeScratch& sc,
                                           bool force_nan) {
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const bool active = tid < kMergeThreads;
  const int pl = tid >> 3, cq = tid & 7;
  const int64_t orow = unit / kMergeChunks;
  const int cchunk = (int)(unit - orow * kMergeChunks);
  const int64_t grp = (int64_t)((uint32_t)orow / (uint32_t)p.rows);  // rows * groups < 2^31
  const int64_t row = orow - grp * p.rows;

  // slot range [s0, s1) of this group.  Under SPLIT_BALANCED every workgroup owns at
  // least one page (W <= P), so every slot in the range holds a piece.
  int64_t s0 = 0, s1 = 0;
  bool inconsistent = force_nan;
  if (p.mode == MERGE_GENERIC) {
    s1 = p.num_parts;
  } else if (p.split_mode == SPLIT_FIXED) {
    s0 = grp * p.num_splits;
    s1 = s0 + p.num_splits;
  } else {
    int64_t P = 0, pre = 0, pr = 0;
    for (int r = 0; r < p.batch; ++r) {
      const int pg = pages_of(p.seq_lens[r], p.max_pages);
      if (r < grp) pre += pg;
      if (r == grp) pr = pg;
      P += pg;
    }
    inconsistent = inconsistent || P != p.total_pages;
    if (pr > 0 && !inconsistent) {
      s0 = balanced_wg_of(pre, P, p.num_wg) + grp;
      s1 = balanced_wg_of(pre + pr - 1, P, p.num_wg) + grp + 1;
    }
  }
  const int64_t col = cchunk * kMergeCols + cq * 4;
  auto load_o = [&](int64_t s) -> f32x4 {
    const int64_t off = (s * p.part_rows + row) * kDV + col;
    if constexpr (PART_BF16) {
      const bf16x4 b = *(const bf16x4*)((const __bf16*)p.part_o + off);
      return f32x4{(float)b[0], (float)b[1], (float)b[2], (float)b[3]};
    } else {
      return *(const f32x4*)((const float*)p.part_o + off);
    }
  };

  // first round: loads of O and LSE together
  f32x4 o[kMergeUnroll];
  float l[kMergeUnroll];
#pragma unroll
  for (int u = 0; u < kMergeUnroll; ++u) {
    const int64_t s = s0 + pl + kMergeLanes * u;
    const bool ok = active && s < s1;
    l[u] = ok ? p.part_lse[s * p.part_rows + row] : kNegInf;
    o[u] = ok ? load_o(s) : f32x4{0.f, 0.f, 0.f, 0.f};
  }
  // M over all parts (later rounds: LSEs only)
  float mx = kNegInf;
#pragma unroll
  for (int u = 0; u < kMergeUnroll; ++u) mx = nan_max(mx, l[u]);
  if (active)
    for (int64_t s = s0 + kMergeRound + tid; s < s1; s += kMergeThreads)
      mx = nan_max(mx, p.part_lse[s * p.part_rows + row]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) mx = nan_max(mx, __shfl_xor(mx, off));
  if (active && lane == 0) sc.m[wave] = mx;
  __syncthreads();
  float M = sc.m[0];
#pragma unroll
  for (int wv = 1; wv < kMergeThreads / 64; ++wv) M = nan_max(M, sc.m[wv]);

  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  float asum = 0.f;
  if (active && M != kNegInf) {
#pragma unroll
    for (int u = 0; u < kMergeUnroll; ++u) {
      const float a = exp2_fast((l[u] - M) * kLog2e);  // empty parts: exp2(-inf) = 0
      acc += a * o[u];
      asum += a;
    }
    for (int64_t base = s0 + kMergeRound; base < s1; base += kMergeRound) {
#pragma unroll
      for (int u = 0; u < kMergeUnroll; ++u) {
        const int64_t s = base + pl + kMergeLanes * u;
        if (s >= s1) continue;
        const float a = exp2_fast((p.part_lse[s * p.part_rows + row] - M) * kLog2e);
        acc += a * load_o(s);
        asum += a;
      }
    }
  }
  // sum over the part lanes: 8 per wave (lanes cq + 8k), then the waves
#pragma unroll
  for (int off = 8; off < 64; off <<= 1) {
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] += __shfl_xor(acc[e], off);
    asum += __shfl_xor(asum, off);
  }
  if (active && lane < kMergeQuads) {
    sc.v[wave][cq] = acc;
    sc.s[wave][cq] = asum;
  }
  __syncthreads();
  if (tid < kMergeQuads) {
    f32x4 v = sc.v[0][cq];
    float den = sc.s[0][cq];
#pragma unroll
    for (int wv = 1; wv < kMergeThreads / 64; ++wv) {
      v += sc.v[wv][cq];
      den += sc.s[wv][cq];
    }
    const bool empty = M == kNegInf && !inconsistent;
    f32x4 res = empty ? f32x4{0.f, 0.f, 0.f, 0.f} : v * (1.0f / den);
    if (inconsistent) res = f32x4{1.f, 1.f, 1.f, 1.f} * __builtin_nanf("");
    if (p.out) {
      const int64_t off = orow * kDV + col;
      if constexpr (OUT_BF16) {
        *(bf16x4*)((__bf16*)p.out + off) =
            bf16x4{(__bf16)res[0], (__bf16)res[1], (__bf16)res[2], (__bf16)res[3]};
      } else {
        *(f32x4*)((float*)p.out + off) = res;
      }
    }
    if (p.out_lse && cchunk == 0 && cq == 0) {
      p.out_lse[orow] =
          inconsistent ? __builtin_nanf("") : (empty ? kNegInf : M + log2_fast(den) * kLn2);
    }
  }
  __syncthreads();  // scratch is reused by the next unit
}

// ------------------------------------------------------------------- kernels

// LDS (two page tiles) caps residency at one or two workgroups per compute unit, so the
// kernels ask for no extra occupancy: the register budget is what the block size allows.
template <bool FP8, int G, int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(1, 1))) void mla_partial_kernel(
    PartialParams p, const uint16_t* __restrict__ q_ptr, const uint8_t* __restrict__ pool,
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ seq_lens,
    float* __restrict__ part_o, float* __restrict__ part_lse) {
  using TG = TileGeom<FP8>;
  constexpr int RB = NW / G;
  __shared__ __attribute__((aligned(1024))) unsigned char tile0[TG::kPageBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char tile1[TG::kPageBytes];
  __shared__ __attribute__((aligned(16))) unsigned char pbuf[G > 1 ? RB * 2 * 64 * 16 : 16];
  __shared__ float red[RB * G * 16];
  partial_phase<FP8, G, NW>(p, q_ptr, pool, block_table, seq_lens, part_o, part_lse, tile0, tile1,
                            pbuf, red);
}

// Both stages in one launch.  All workgroups are resident at once (the plan never asks for
// more than the compute units hold), so after the partial answers are written they meet
// at a device-wide barrier and then share the merge.  The barrier is a counter and a
// generation word in the workspace; the last arriver resets the counter and bumps the
// generation, which leaves the counter zero for the next call.  Waiting is bounded: a
// workgroup that gives up writes NaN instead of its merge results.
constexpr uint32_t kBarrierSpinLimit = 1u << 17;

template <bool FP8, int G, int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(1, 1))) void mla_fused_kernel(
    PartialParams p, MergeParams mp, const uint16_t* __restrict__ q_ptr,
    const uint8_t* __restrict__ pool, const int32_t* __restrict__ block_table,
    const int32_t* __restrict__ seq_lens, float* part_o, float* part_lse, uint32_t* ctrl) {
  using TG = TileGeom<FP8>;
  constexpr int RB = NW / G;
  __shared__ __attribute__((aligned(1024))) unsigned char tile0[TG::kPageBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char tile1[TG::kPageBytes];
  __shared__ __attribute__((aligned(16))) unsigned char pbuf[G > 1 ? RB * 2 * 64 * 16 : 16];
  __shared__ float red[RB * G * 16];
  __shared__ MergeScratch msc;
  __shared__ int timed_out;
  partial_phase<FP8, G, NW>(p, q_ptr, pool, block_table, seq_lens, part_o, part_lse, tile0, tile1,
                            pbuf, red);

  // ---- device-wide barrier
  __syncthreads();  // this workgroup's partial stores are complete
  if (threadIdx.x == 0) {
    // Without the marker the counters are not known to start at zero (workspace never
    // initialised, or a previous call gave up): nobody waits and every output is NaN.
    if (__hip_atomic_load(&ctrl[kCtrlMagicWord], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) !=
        kCtrlMagic) {
      timed_out = 1;
    } else {
    const uint32_t gen = __hip_atomic_load(&ctrl[1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");  // publish the partials device-wide
    const uint32_t arrived =
        __hip_atomic_fetch_add(&ctrl[0], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    int give_up = 0;
    if (arrived == gridDim.x - 1) {
      __hip_atomic_store(&ctrl[0], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_fetch_add(&ctrl[1], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
      uint32_t n = 0;
      while (__hip_atomic_load(&ctrl[1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == gen) {
        __builtin_amdgcn_s_sleep(1);
        if (++n == kBarrierSpinLimit) {
          give_up = 1;
          // the counters are now unreliable: later calls refuse to wait (NaN outputs)
          __hip_atomic_store(&ctrl[kCtrlMagicWord], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          break;
        }
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");  // see every workgroup's partials
    timed_out = give_up;
    }
  }
  __syncthreads();
  const bool force_nan = timed_out != 0;

  // ---- merge units, spread over the workgroups
  const int64_t units = (int64_t)mp.batch * mp.rows * kMergeChunks;
  for (int64_t u = blockIdx.x; u < units; u += gridDim.x) {
    if (mp.out_bf16) merge_unit<false, true>(mp, u, msc, force_nan);
    else merge_unit<false, false>(mp, u, msc, force_nan);
  }
}

template <bool PART_BF16, bool OUT_BF16>
__global__ __launch_bounds__(kMergeThreads) void mla_merge_kernel(MergeParams p) {
  __shared__ MergeScratch msc;
  merge_unit<PART_BF16, OUT_BF16>(p, blockIdx.x, msc, false);
}

// ------------------------------------------------------------------ launchers

namespace {

template <bool FP8, int G, int NW>
hipError_t launch_partial_t(const PartialParams& p, hipStream_t stream) {
  hipLaunchKernelGGL((mla_partial_kernel<FP8, G, NW>), dim3(p.num_wg), dim3(NW * 64), 0, stream, p,
                     p.q, p.pool, p.block_table, p.seq_lens, p.part_o, p.part_lse);
  return hipGetLastError();
}

// Workgroups of the fused kernel one device holds at once (cached per device).
template <bool FP8, int G, int NW>
int fused_capacity() {
  static int cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (cached[dev] == 0) {
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, mla_fused_kernel<FP8, G, NW>, NW * 64,
                                                     0) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return 0;
    cached[dev] = per_cu * cus > 0 ? per_cu * cus : -1;
  }
  return cached[dev] > 0 ? cached[dev] : 0;
}

template <bool FP8, int G, int NW>
hipError_t launch_fused_t(const PartialParams& p, const MergeParams& mp, uint32_t* ctrl,
                          hipStream_t stream, bool* launched) {
  *launched = false;
  if (p.num_wg > fused_capacity<FP8, G, NW>()) return hipSuccess;  // caller falls back
  hipLaunchKernelGGL((mla_fused_kernel<FP8, G, NW>), dim3(p.num_wg), dim3(NW * 64), 0, stream, p, mp,
                     p.q, p.pool, p.block_table, p.seq_lens, p.part_o, p.part_lse, ctrl);
  *launched = true;
  return hipGetLastError();
}

template <bool FP8>
hipError_t launch_partial_rb(const PartialParams& p, int rb, hipStream_t stream) {
  switch (rb) {
    case 1: return launch_partial_t<FP8, 4, 4>(p, stream);
    case 2: return launch_partial_t<FP8, 2, 4>(p, stream);
    case 3: return launch_partial_t<FP8, 2, 6>(p, stream);
    case 4: return launch_partial_t<FP8, 1, 4>(p, stream);
    case 5: return launch_partial_t<FP8, 1, 5>(p, stream);
    case 6: return launch_partial_t<FP8, 1, 6>(p, stream);
    case 7: return launch_partial_t<FP8, 1, 7>(p, stream);
    case 8: return launch_partial_t<FP8, 1, 8>(p, stream);
  }
  return hipErrorInvalidValue;
}

template <bool FP8>
hipError_t launch_fused_rb(const PartialParams& p, const MergeParams& mp, uint32_t* ctrl, int rb,
                           hipStream_t stream, bool* launched) {
  switch (rb) {
    case 1: return launch_fused_t<FP8, 4, 4>(p, mp, ctrl, stream, launched);
    case 2: return launch_fused_t<FP8, 2, 4>(p, mp, ctrl, stream, launched);
    case 3: return launch_fused_t<FP8, 2, 6>(p, mp, ctrl, stream, launched);
    case 4: return launch_fused_t<FP8, 1, 4>(p, mp, ctrl, stream, launched);
    case 5: return launch_fused_t<FP8, 1, 5>(p, mp, ctrl, stream, launched);
    case 6: return launch_fused_t<FP8, 1, 6>(p, mp, ctrl, stream, launched);
    case 7: return launch_fused_t<FP8, 1, 7>(p, mp, ctrl, stream, launched);
    case 8: return launch_fused_t<FP8, 1, 8>(p, mp, ctrl, stream, launched);
  }
  *launched = false;
  return hipErrorInvalidValue;
}

}  // namespace

// Waves per row block (G) for a row-block count: one row block needs 4 waves to keep
// the four SIMDs busy, so its positions and output columns are split over G waves.
int partial_waves_per_row_block(int row_blocks) {
  if (row_blocks == 1) return 4;
  if (row_blocks <= 3) return 2;
  return 1;
}

size_t partial_lds_size(bool fp8, int row_blocks) {
  const int G = partial_waves_per_row_block(row_blocks);
  const size_t tiles = 2 * (size_t)kPage * kDLatent * (fp8 ? 1 : 2);
  return tiles + (G > 1 ? row_blocks * 2 * 64 * 16 : 16) + row_blocks * G * 16 * 4 +
         sizeof(MergeScratch) + 16;
}

hipError_t launch_partial(const PartialParams& p, bool fp8, hipStream_t stream) {
  const int rb = p.q_len * p.head_groups;
  return fp8 ? launch_partial_rb<true>(p, rb, stream) : launch_partial_rb<false>(p, rb, stream);
}

// Both stages in one launch when every workgroup fits on the device at once; *launched
// reports whether it ran (otherwise the caller runs the two kernels).
hipError_t launch_fused(const PartialParams& p, const MergeParams& mp, uint32_t* ctrl, bool fp8,
                        hipStream_t stream, bool* launched) {
  const int rb = p.q_len * p.head_groups;
  return fp8 ? launch_fused_rb<true>(p, mp, ctrl, rb, stream, launched)
             : launch_fused_rb<false>(p, mp, ctrl, rb, stream, launched);
}

hipError_t launch_merge(const MergeParams& p, int64_t total_rows, hipStream_t stream) {
  const dim3 grid((unsigned)(total_rows * kMergeChunks));
  if (p.part_bf16) {
    if (p.out_bf16) hipLaunchKernelGGL((mla_merge_kernel<true, true>), grid, dim3(kMergeThreads), 0, stream, p);
    else hipLaunchKernelGGL((mla_merge_kernel<true, false>), grid, dim3(kMergeThreads), 0, stream, p);
  } else {
    if (p.out_bf16) hipLaunchKernelGGL((mla_merge_kernel<false, true>), grid, dim3(kMergeThreads), 0, stream, p);
    else hipLaunchKernelGGL((mla_merge_kernel<false, false>), grid, dim3(kMergeThreads), 0, stream, p);
  }
  return hipGetLastError();
}

// Initialise the workspace's control words: barrier counter and generation zero, the
// marker set (graph-safe: a kernel, not a memset node).
__global__ void mla_init_ctrl_kernel(uint32_t* w) {
  if (threadIdx.x < kCtrlWords) w[threadIdx.x] = threadIdx.x == kCtrlMagicWord ? kCtrlMagic : 0u;
}

hipError_t launch_init_ctrl(uint32_t* w, hipStream_t stream) {
  hipLaunchKernelGGL(mla_init_ctrl_kernel, dim3(1), dim3(64), 0, stream, w);
  return hipGetLastError();
}

}  // namespace mla
