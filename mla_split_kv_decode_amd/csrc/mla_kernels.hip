// gfx950 kernels of absorbed-MLA split-KV decode.
//
// Stage 1, mla_partial_kernel: work unit w (see mla_internal.h) runs as row_groups
// workgroups, each owning one or two row blocks of 16 query rows.  For each piece of the
// unit (request, page range) a workgroup streams the latent pages into LDS and computes,
// for its rows, the softmax-attention partial answer over the piece: O_p (normalised)
// and LSE_p.  Kimi K3 on MI355X, section 4 "MLA": the history is split into partitions
// handled by separate workgroups; section 1 "Cache", DCP8 paragraph: a partial answer
// carries its normalisation so pieces can be merged.
//
// Stage 2, mla_merge_kernel / mla_merge_rows_kernel: the LSE-weighted merge of the
// partial answers of each row.
//
// Data movement.  A page (64 positions x 576 latent values) is copied from HBM straight
// into an LDS tile with global_load_lds_dwordx4 (no staging registers); two bf16 tiles
// (four FP8 tiles) per workgroup, so the next pages stream in while the current one is
// consumed, and a piece of two pages has its whole history in flight at once.  The
// multi-row and FP8 kernels issue each copy in parts over the phases of a page (a CU
// accepts only about twenty copy operations before the issuing waves stall), and the
// FP8 two-row-block kernel works on two pages an iteration (one set of exchanges for
// both).  Within a
// tile each 16-byte chunk of a row sits at an XOR-swizzled column so that the MFMA
// operand reads below hit distinct LDS banks; the copy fills the tile in contiguous 1 KiB
// blocks and each lane fetches the global chunk that belongs at its slot.
//
// Matrix layout (all on the 16x16 MFMA grid, wave64):
//  * rows   : 16 query rows = 16 heads of one query token ("row block"); heads past the
//             real count repeat the last real head (section 4: padding heads leaves real
//             heads unchanged) and are never written.
//  * QK^T   : S^T[pos][row] = sum_k K[pos][k] Q[row][k] with v_mfma_f32_16x16x32_bf16,
//             A = 16 positions x 32 latent columns read from the LDS tile, B = the row
//             block's queries, kept in registers for the whole piece (on request, FP8
//             pools: v_mfma_f32_16x16x128_f8f6f4 on the codes and split-precision FP8
//             queries).
//  * PV     : O^T[col][row] += sum_pos V^T[col][pos] P^T[pos][row].  The S^T accumulator
//             layout (lane = row, 4 consecutive positions per lane) is already the B
//             layout of the next MFMA; P takes one small LDS exchange between the waves
//             that computed it and the waves that own the output columns.  V^T is read
//             from the same LDS tile with the gfx950 transposing LDS reads
//             (ds_read_b64_tr_b16 for bf16, ds_read_b64_tr_b8 for FP8), so each latent
//             byte leaves HBM once per workgroup.
//  * softmax: online, in log2 units, with an exact running max; the row max is a
//             cross-lane reduction (row swaps) and an LDS exchange between the waves.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "mla_internal.h"

// m0 is set inside the page-copy asm, the only user of m0 in these kernels
#pragma clang diagnostic ignored "-Winline-asm"

namespace mla {

// Timeline builds (-DMLA_TIMELINE=1, libmla_decode_timeline.so, read by bench.py --timeline):
// wave 0 of each workgroup stamps the device's 100 MHz real-time clock at fixed points of
// the decode (mla_timeline.h names them); the stamps of a workgroup's last piece are kept.
// The stamp waits for the wave's outstanding scalar loads, so the entry stamp comes first
// and no stamp sits between entry and the first copies of a piece.  In ordinary builds the
// macros are empty.
#ifdef MLA_TIMELINE
constexpr int kTlBlocks = 4096, kTlSlots = 8, kTlMergeBlocks = 16384, kTlMergeSlots = 4;
__device__ unsigned long long g_tl_partial[kTlBlocks * kTlSlots];
__device__ unsigned long long g_tl_merge[kTlMergeBlocks * kTlMergeSlots];
#define MLA_TL(k)                                                                              \
  do {                                                                                         \
    if (threadIdx.x == 0 && blockIdx.x < kTlBlocks)                                            \
      g_tl_partial[blockIdx.x * kTlSlots + (k)] = __builtin_amdgcn_s_memrealtime();            \
  } while (0)
#define MLA_TL_MERGE(k)                                                                        \
  do {                                                                                         \
    if (threadIdx.x == 0 && blockIdx.x < kTlMergeBlocks)                                       \
      g_tl_merge[blockIdx.x * kTlMergeSlots + (k)] = __builtin_amdgcn_s_memrealtime();         \
  } while (0)
#else
#define MLA_TL(k) \
  do {            \
  } while (0)
#define MLA_TL_MERGE(k) \
  do {                  \
  } while (0)
#endif

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
// Only for addresses the compiler can fold (a member of the workgroup's __shared__
// object at a constant offset): a run-time generic-to-LDS cast carries a null check on the
// shared aperture, which the gfx950 code generator can emit as an illegal instruction.
// Everything else takes integer LDS offsets from such a base.
// The outputs are early-clobber ("=&v"): the reads of a call share one address register,
// which must not double as the destination of an earlier read of the same call (a read
// that returns before a later one issues would replace the address).
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
template <int G>
__device__ __forceinline__ float lds_max_of(uint32_t off, float init) {
  // max of the floats at LDS byte offsets off, off + 64, ..., off + 64 (G-1), and init
  float v[4];
  if constexpr (G == 4) {
    asm volatile("ds_read_b32 %0, %4\n\tds_read_b32 %1, %4 offset:64\n\t"
                 "ds_read_b32 %2, %4 offset:128\n\tds_read_b32 %3, %4 offset:192\n\t"
                 "s_waitcnt lgkmcnt(0)"
                 : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]) : "v"(off));
    return fmaxf(fmaxf(fmaxf(init, v[0]), fmaxf(v[1], v[2])), v[3]);
  } else {
    static_assert(G == 2, "exchange width");
    asm volatile("ds_read_b32 %0, %2\n\tds_read_b32 %1, %2 offset:64\n\ts_waitcnt lgkmcnt(0)"
                 : "=&v"(v[0]), "=&v"(v[1]) : "v"(off));
    return fmaxf(fmaxf(init, v[0]), v[1]);
  }
}
// Row maxima of RB row blocks from the sub-tile exchange: row block j's four entries at
// off + 256 j + 64 u (u = sub-tile); both row blocks' eight reads in one round trip
template <int RB>
__device__ __forceinline__ void lds_row_maxima(uint32_t off, float (&mx)[RB]) {
  static_assert(RB == 1 || RB == 2, "row blocks");
  if constexpr (RB == 1) {
    mx[0] = lds_max_of<4>(off, kNegInf);
  } else {
    float v[4], w[4];
    asm volatile("ds_read_b32 %0, %8\n\tds_read_b32 %1, %8 offset:64\n\t"
                 "ds_read_b32 %2, %8 offset:128\n\tds_read_b32 %3, %8 offset:192\n\t"
                 "ds_read_b32 %4, %8 offset:256\n\tds_read_b32 %5, %8 offset:320\n\t"
                 "ds_read_b32 %6, %8 offset:384\n\tds_read_b32 %7, %8 offset:448\n\t"
                 "s_waitcnt lgkmcnt(0)"
                 : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(w[0]), "=&v"(w[1]), "=&v"(w[2]),
                   "=&v"(w[3])
                 : "v"(off));
    mx[0] = fmaxf(fmaxf(fmaxf(kNegInf, v[0]), fmaxf(v[1], v[2])), v[3]);
    mx[1] = fmaxf(fmaxf(fmaxf(kNegInf, w[0]), fmaxf(w[1], w[2])), w[3]);
  }
}
template <int G>
__device__ __forceinline__ float lds_sum_of(uint32_t off) {
  float v[4];
  if constexpr (G == 4) {
    asm volatile("ds_read_b32 %0, %4\n\tds_read_b32 %1, %4 offset:64\n\t"
                 "ds_read_b32 %2, %4 offset:128\n\tds_read_b32 %3, %4 offset:192\n\t"
                 "s_waitcnt lgkmcnt(0)"
                 : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]) : "v"(off));
    return ((v[0] + v[1]) + v[2]) + v[3];
  } else {
    static_assert(G == 2, "exchange width");
    asm volatile("ds_read_b32 %0, %2\n\tds_read_b32 %1, %2 offset:64\n\ts_waitcnt lgkmcnt(0)"
                 : "=&v"(v[0]), "=&v"(v[1]) : "v"(off));
    return v[0] + v[1];
  }
}
// lds_sum_of<4>(off), and the dword at off2 in the same round trip
__device__ __forceinline__ float lds_sum4_and_b32(uint32_t off, uint32_t off2, int32_t& u) {
  float v[4];
  asm volatile("ds_read_b32 %0, %5\n\tds_read_b32 %1, %5 offset:64\n\t"
               "ds_read_b32 %2, %5 offset:128\n\tds_read_b32 %3, %5 offset:192\n\t"
               "ds_read_b32 %4, %6\n\ts_waitcnt lgkmcnt(0)"
               : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(u) : "v"(off), "v"(off2));
  return ((v[0] + v[1]) + v[2]) + v[3];
}
// two consecutive dwords
template <int K>
__device__ __forceinline__ void lds_read_ids(uint32_t off, int32_t (&v)[K]) {
  static_assert(K == 2, "id count");
  asm volatile("ds_read_b32 %0, %2\n\tds_read_b32 %1, %2 offset:4\n\ts_waitcnt lgkmcnt(0)"
               : "=&v"(v[0]), "=&v"(v[1]) : "v"(off));
}
// two 16-byte reads 1 KiB apart (the two 32-position P^T chunks of a row block)
__device__ __forceinline__ void lds_read_pair_b128(uint32_t off, i32x4& a, i32x4& b) {
  asm volatile("ds_read_b128 %0, %2\n\tds_read_b128 %1, %2 offset:1024\n\ts_waitcnt lgkmcnt(0)"
               : "=&v"(a), "=&v"(b) : "v"(off));
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

// Max and sum of a value over the four lanes l, l ^ 16, l ^ 32, l ^ 48 (the four 16-lane
// rows of a wave): the gfx950 row-swap instructions exchange whole rows between two
// registers, so the larger (or the sum) of the two results combines each lane with its
// partner without an LDS round trip.
__device__ __forceinline__ float max_over_rows(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float sum_over_rows(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// x combined with op over the lanes lane ^ m for every power of two m in [LO, 64): DPP
// moves inside each 16-lane row (quad permutes for 1 and 2; rotates by 4 and 8, which on
// values already combined over the smaller offsets reach the same lanes as those xors),
// then the gfx950 row swaps across rows.  All lanes active; every lane gets the result.
template <int LO, class Op>
__device__ __forceinline__ float wave_combine(float x, Op op) {
  static_assert(LO == 1 || LO == 2 || LO == 4 || LO == 8 || LO == 16 || LO == 32, "offset");
  auto dpp = [](float v, auto ctrl) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), decltype(ctrl)::value, 0xF, 0xF, false));
  };
  if constexpr (LO <= 1) x = op(x, dpp(x, std::integral_constant<int, 0xB1>{}));   // quad_perm 1,0,3,2
  if constexpr (LO <= 2) x = op(x, dpp(x, std::integral_constant<int, 0x4E>{}));   // quad_perm 2,3,0,1
  if constexpr (LO <= 4) x = op(x, dpp(x, std::integral_constant<int, 0x124>{}));  // row_ror:4
  if constexpr (LO <= 8) x = op(x, dpp(x, std::integral_constant<int, 0x128>{}));  // row_ror:8
  if constexpr (LO <= 16) {
    auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = op(__uint_as_float(a[0]), __uint_as_float(a[1]));
  }
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return op(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Eight FP8 E4M3FN codes (little-endian bytes of `raw`) -> eight bf16, exactly.
__device__ __forceinline__ bf16x8 fp8x8_to_bf16x8(i32x2 raw) {
  bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw[0], 1.0f, false);
  bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw[0], 1.0f, true);
  bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw[1], 1.0f, false);
  bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw[1], 1.0f, true);
  return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

typedef int i32x8 __attribute__((ext_vector_type(8)));

// Eight bf16 values (the bits of q) times the power of two sc, |q sc| < 256, as two E4M3FN
// code vectors with hi + lo = q sc: hi is q sc rounded to nearest (even), lo the remainder
// (exact in fp32) rounded again.  A bf16 value has eight significant bits and hi keeps the
// top four, so the remainder is an integer multiple of q's last place of at most half of
// hi's, with at most four significant bits: lo is exact unless it falls below the E4M3FN
// normal range, i.e. hi + lo = q sc exactly for |q sc| >= 1/4 and to within 2^-10 below.
__device__ __forceinline__ void split_fp8x8(i32x4 q, float sc, i32x2& hi, i32x2& lo) {
  const bf16x8 v = __builtin_bit_cast(bf16x8, q);
  float x[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = (float)v[e] * sc;
#pragma unroll
  for (int w = 0; w < 2; ++w) {
    int h = __builtin_amdgcn_cvt_pk_fp8_f32(x[4 * w], x[4 * w + 1], 0, false);
    h = __builtin_amdgcn_cvt_pk_fp8_f32(x[4 * w + 2], x[4 * w + 3], h, true);
    const auto b0 = __builtin_amdgcn_cvt_pk_f32_fp8(h, false);
    const auto b1 = __builtin_amdgcn_cvt_pk_f32_fp8(h, true);
    int l = __builtin_amdgcn_cvt_pk_fp8_f32(x[4 * w] - b0[0], x[4 * w + 1] - b0[1], 0, false);
    l = __builtin_amdgcn_cvt_pk_fp8_f32(x[4 * w + 2] - b1[0], x[4 * w + 3] - b1[1], l, true);
    hi[w] = h;
    lo[w] = l;
  }
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
  // fp8: 576-byte rows 4 apart start on the same bank and so do rows 16 apart; the key
  // separates both within a 64-byte group (the transposing V^T reads take rows r and
  // r + 16 together)
  __device__ static constexpr int key8(int row) { return ((row >> 2) & 3) ^ (((row >> 4) & 1) << 1); }
  __device__ static __forceinline__ int swz(int row, int c) {
    if constexpr (FP8) return (c & ~3) | ((c & 3) ^ key8(row));
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
//   kbase_of(lrow, lgrp, kk & 1, pt) + pt * 16 * kRowBytes + kstep(kk)
// V^T (A operand of PV), 32-position chunk c, half hh (positions +16), column tile ct of
// this wave: vbase[ct & 3] + c * 32 * kRowBytes + hh * 16 * kRowBytes + vstep(ct)
template <bool FP8>
struct OperandAddr {
  using TG = TileGeom<FP8>;
  int kbase[2];  // kbase_of(lrow, lgrp, e, 0)
  int vbase[4];
  __device__ __forceinline__ OperandAddr(int lrow, int lgrp, int wave_col_tile0) {
    if constexpr (FP8) {
      const int kkey = TG::key8(lrow);
#pragma unroll
      for (int e = 0; e < 2; ++e)
        kbase[e] = lrow * TG::kRowBytes + 16 * ((2 * e + (lgrp >> 1)) ^ kkey) + 8 * (lgrp & 1);
      // V^T (tr8): lane (lgrp, lrow = 2ii + h) reads row 32c + 16(ii>>2) + 4 lgrp + (ii&3),
      // chunk n = wave_col_tile0 + ct, byte 8h; key8 of the row = lgrp ^ 2 ((ii>>2) & 1)
      const int ii = lrow >> 1, h = lrow & 1;
      const int row = 16 * (ii >> 2) + 4 * lgrp + (ii & 3);
      const int key = TG::key8(row);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        vbase[j] = row * TG::kRowBytes + 16 * (4 * (wave_col_tile0 >> 2) + (j ^ key)) + 8 * h;
    } else {
      const int kkey = TG::key16(lrow);
#pragma unroll
      for (int e = 0; e < 2; ++e) kbase[e] = lrow * TG::kRowBytes + 16 * ((4 * e + lgrp) ^ kkey);
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
  // K of sub-tile pt (rows 16 pt + lrow), k-step parity e:
  //   fp8: chunk 2kk + (lgrp>>1), byte 8(lgrp&1), key8 of the row (depends on pt's parity);
  //   bf16: chunk 4kk + lgrp, key16 of the row (the same for every pt)
  __device__ static __forceinline__ int kbase_of(int lrow, int lgrp, int e, int pt) {
    if constexpr (FP8)
      return lrow * TG::kRowBytes + 16 * ((2 * e + (lgrp >> 1)) ^ TG::key8(16 * pt + lrow)) + 8 * (lgrp & 1);
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
// STREAM (kernels of one-row-group plans): the copies carry the non-temporal hint.  A page
// that one workgroup alone reads is then not kept in the caches, so the small data every
// launch reuses (block table, queries, partial answers) stays resident: long32k 15.93 ->
// 15.45 us a layer-step, ragged 217 -> 194 us, two draft tokens over 131K positions
// (two row blocks) 212 -> 188 us (same-box A/B).  The plan asks for it only when a layer's
// KV is too large for the memory-side cache to keep the layers' pools between steps
// (tiny's 24 layers of 1.2 MB stay resident without the hint, 5.70 against 5.96 us);
// pages that several row groups read from their XCD's L2 keep the default policy (the
// hint cost dcp_fp8 and spec_verify 3% each).
template <bool FP8, int NW, bool STREAM = false>
struct PageCopy {
  using TG = TileGeom<FP8>;
  static constexpr int kPer = (TG::kDmaOps + NW - 1) / NW;
  int src_off[kPer];  // this lane's source offsets within a page, one per operation
  int wave, lane;
  bool stream;        // non-temporal copies (STREAM kernels only)
  __device__ __forceinline__ PageCopy(int wave_, int lane_, bool stream_ = false)
      : wave(wave_), lane(lane_), stream(stream_) {
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
  __device__ __forceinline__ void operator()(uint32_t base, const unsigned char* src,
                                             int valid_rows) const {
    part<0, kPer>(base, src, valid_rows);
  }
  // Operations J0 .. J1 - 1 of this wave's kPer (a copy may be issued in several parts).
  template <int J0, int J1>
  __device__ __forceinline__ void part(uint32_t base, const unsigned char* src, int valid_rows) const {
#pragma unroll
    for (int j = J0; j < (J1 < kPer ? J1 : kPer); ++j) {
      int off = src_off[j];
      if (valid_rows < kPage) {
        const int row = (block(j) * 64 + lane) / TG::kChunksPerRow;
        if (row >= valid_rows) off -= (row - (valid_rows - 1)) * TG::kRowBytes;
      }
      const uint32_t dst = __builtin_amdgcn_readfirstlane(base + block(j) * 1024);
      if (STREAM && stream)  // uniform
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2 nt"
                     :: "s"(dst), "v"(off), "s"(src) : "memory", "m0");
      else
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
                     :: "s"(dst), "v"(off), "s"(src) : "memory", "m0");
    }
  }
};

// Copy the queries of a workgroup's RB row blocks rb0 .. rb0 + RB - 1 (request r) into an
// LDS staging area of RB x 16 rows of 576 bf16, laid out like a bf16 page tile (same chunk
// swizzle), so one HBM read serves every wave that shares a row block.  Row i of row
// block rb is head 16 hg + i of token t (rb = t * head_groups + hg); a padding head
// repeats the last real head, and a padding row block (past rb_last) the last real row
// block (their results are discarded).  Same operation-count rule as PageCopy.
template <int NW, int RB>
struct QueryCopy {
  using TG = TileGeom<false>;
  static constexpr int kBlocks = RB * kRowsPerBlock * TG::kRowBytes / 1024;
  static constexpr int kPer = (kBlocks + NW - 1) / NW;
  int wave, lane;
  __device__ __forceinline__ QueryCopy(int wave_, int lane_) : wave(wave_), lane(lane_) {}
  __device__ __forceinline__ void operator()(uint32_t base, const uint16_t* q_req,
                                             int num_heads, int head_groups, int rb0,
                                             int rb_last) const {
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      int k = wave + NW * j;
      k = k < kBlocks ? k : kBlocks - 1;
      const int s = k * 64 + lane;
      const int row = s / TG::kChunksPerRow, cs = s - row * TG::kChunksPerRow;
      const int lrb = row / kRowsPerBlock, i = row - lrb * kRowsPerBlock;
      const int rb = min(rb0 + lrb, rb_last);  // a padding row block repeats the last
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

// The scalars of a partial-stage workgroup.  Everything a one-request plan needs before
// its first page copy (which pages, where the table, pool and queries are, the row-block
// shape, the pool's page count, the copy hint) arrives in the leading kernel arguments,
// which the library is built to have preloaded into SGPRs with the launch (fourteen
// dwords at most: small fields share a dword).  The rest come from the parameter block,
// whose loads run meanwhile and are settled (all of them at once, rather than one round
// trip per use inside a branch) once the first copies are out.
//   unit_pack  = row groups | split mode << 16 | plan_n << 17
//   shape_pack = heads | q_len << 16 | causal << 24 | stream << 25
//   npages     = the pool's page count, saturated at 2^32 - 1 (page ids are int32)
struct HotArgs {
  int heads, hgroups, rgroups, mode, nwg, plan_n, len0, maxp, qlen, causal, stream;
  uint32_t npages;
  int64_t total32;  // the plan's page total (plan_n > 0)
  // from the parameter block
  int nsplits, batch, nslots;
  int64_t total_dev;  // page total of the device lengths (plan_n = 0)
  float sscale, vscale;
  __device__ __forceinline__ HotArgs(const PartialParams& p, int nwg_, uint32_t unit_pack, int total32_, int len0_,
                                     int maxp_, uint32_t shape_pack, uint32_t npages_)
      : heads((int)(shape_pack & 0xFFFF)), hgroups((int)(((shape_pack & 0xFFFF) + kRowsPerBlock - 1) / kRowsPerBlock)),
        rgroups((int)(unit_pack & 0xFFFF)), mode((int)((unit_pack >> 16) & 1)), nwg(nwg_),
        plan_n((int)(unit_pack >> 17)), len0(len0_), maxp(maxp_), qlen((int)((shape_pack >> 16) & 0xFF)),
        causal((int)((shape_pack >> 24) & 1)), stream((int)((shape_pack >> 25) & 1)), npages(npages_),
        total32(total32_), nsplits(p.num_splits), batch(p.batch), nslots(p.num_slots),
        total_dev(p.total_pages), sscale(p.score_scale), vscale(p.v_scale) {}
  // a block-table entry outside the pool
  __device__ __forceinline__ bool bad_id(int32_t id) const { return id < 0 || (uint32_t)id >= npages; }
  __device__ __forceinline__ void settle() const {
    asm volatile("" ::"s"(nsplits), "s"(batch), "s"(nslots), "s"(total_dev), "s"(sscale), "s"(vscale));
  }
};

// Device lengths under SPLIT_BALANCED (a batch beyond the plan's argument copy): the page
// total P and the first request of unit w's page range [gb, ge) with its page prefix, in
// O(B / threads + log threads) steps.  Thread t sums the pages of requests
// [t c, (t + 1) c), c = ceil(B / threads); a scan of these sums over the workgroup (wave
// scans, then the wave totals through `xch`) places every chunk on the page axis, and the
// one thread whose chunk holds page gb walks it to the request.  Every thread of the
// workgroup calls it (two barriers); the results are uniform and returned in SGPRs.
// `xch`: at least NW + 2 int64 of LDS, free until the caller's next barrier.
template <int NW>
__device__ __forceinline__ bool device_unit_start(const int32_t* __restrict__ seq_lens, int batch, int maxp,
                                                  int64_t w, int64_t nwg, int64_t total,
                                                  int64_t* __restrict__ xch, int& r_first,
                                                  int64_t& pre_first, int64_t& gb, int64_t& ge) {
  constexpr int kThreads = NW * 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int chunk = (batch + kThreads - 1) / kThreads;
  const int r0 = min(tid * chunk, batch), r1 = min(r0 + chunk, batch);
  int64_t own = 0;
  for (int r = r0; r < r1; ++r) own += pages_of(seq_lens[r], maxp);
  int64_t inc = own;  // inclusive scan over the wave
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int64_t v = __shfl_up(inc, off);
    if (lane >= off) inc += v;
  }
  if (lane == 63) xch[wave] = inc;
  __syncthreads();
  int64_t P = 0, before = 0;
#pragma unroll
  for (int v = 0; v < NW; ++v) {
    const int64_t t = xch[v];
    before += v < wave ? t : 0;
    P += t;
  }
  // lengths that disagree with the plan's total: no piece (the merge writes NaN)
  if (P == 0 || P != total) return false;
  gb = balanced_start(w, P, nwg);
  ge = balanced_start(w + 1, P, nwg);
  int64_t pre = before + inc - own;  // pages of the requests before this thread's chunk
  if (own > 0 && pre <= gb && gb < pre + own) {
    for (int r = r0; r < r1; ++r) {
      const int pr = pages_of(seq_lens[r], maxp);
      if (pre + pr > gb) {
        xch[NW] = r;
        xch[NW + 1] = pre;
        break;
      }
      pre += pr;
    }
  }
  __syncthreads();
  r_first = __builtin_amdgcn_readfirstlane((int)xch[NW]);
  const int64_t pf = xch[NW + 1];
  pre_first = (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(pf >> 32)) << 32) |
                        (uint32_t)__builtin_amdgcn_readfirstlane((int)pf));
  return true;
}

// The pieces of work unit w (mla_internal.h): run(r, first page, end page, slot, L) for
// each, from the plan's lengths in the arguments when present, else from seq_lens (then
// every thread of the workgroup must call it; `xch` as for device_unit_start).
template <int NW, class F>
__device__ __forceinline__ void for_each_piece(const PartialParams& p, const HotArgs& a,
                                               const int32_t* __restrict__ seq_lens, int64_t w,
                                               int64_t* __restrict__ xch, F&& run_piece) {
  const bool use_plan = a.plan_n > 0;
  if (a.mode == SPLIT_FIXED) {
    const int S = a.nsplits;
    const int r = (int)(w / S), sp = (int)(w - (int64_t)r * S);
    const int L = use_plan ? (a.plan_n == 1 ? a.len0 : p.plan.len[r]) : max(seq_lens[r], 0);
    const int pages = pages_of(L, a.maxp);
    run_piece(r, fixed_page_begin(sp, pages, S), fixed_page_begin(sp + 1, pages, S), w, L);
  } else if (a.plan_n == 1) {  // one request: its pages are the whole page axis
    const int64_t gb = balanced_start(w, a.total32, a.nwg), ge = balanced_start(w + 1, a.total32, a.nwg);
    run_piece(0, (int)gb, (int)ge, w, a.len0);
  } else if (use_plan) {
    const int64_t P = a.total32;
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
    int r;
    int64_t pre, gb, ge;
    if (!device_unit_start<NW>(seq_lens, a.batch, a.maxp, w, a.nwg, a.total_dev, xch, r, pre, gb, ge)) return;
    for (; r < a.batch && pre < ge; ++r) {
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
// four consecutive columns starting at `col`.  NT: fp32 parts stored non-temporal, for
// plans whose parts are a large share of the kernel's traffic (kNtPartBytes): the partial
// kernel ends sooner (long32k 0.4 us of 11.6; the 96-head DCP shard 2.4 us of 53, whose
// 17 MB of parts otherwise sit dirty in L2 when the kernel ends), while plans with few
// parts lost more in the merge than their partial kernel saved
template <bool NT>
__device__ __forceinline__ void store_partial(float* part_o, int64_t orow, int col, int nslots, int64_t slot,
                                              f32x4 v) {
  const int64_t idx = ((orow * kMergeChunks + (col >> 5)) * nslots + slot) * kMergeCols + (col & 31);
  if constexpr (NT)
    __builtin_nontemporal_store(v, (f32x4*)(part_o + idx));
  else
    *(f32x4*)(part_o + idx) = v;
}

// ------------------------------------------------------------------- partial stage
//
// A workgroup of eight waves owns RBW row blocks of 16 query rows (RBW = 1 or 2) and the
// pieces of one work unit; all eight waves work on the same page.  In QK^T, with one row
// block, wave w computes the partial scores of the 16-position sub-tile u = w & 3 over
// half kh = w >> 2 of the latent (nine of the 18 k-steps of 32 columns), and the two
// halves are added through LDS; with two row blocks ("row split"), wave w computes the
// whole scores of sub-tile u for row block w >> 2, so every wave then takes its share of
// the softmax and no partial scores are exchanged.  In PV wave w produces output columns
// [64 w, 64 w + 64) of every row block over the page's 64 positions, every V^T operand
// read serving all row blocks.  One softmax state per row block for the whole workgroup,
// pages double-buffered (FP8: four in flight), and a page is processed as soon as it has
// landed, so once the stream ends only the last page's work remains.
//
// Row block rb = t * head_groups + hg holds heads 16 hg .. 16 hg + 15 of query token t.
// A problem with more than RBW row blocks runs row_groups = ceil(row blocks / RBW) workgroups
// per unit, each on the same pieces with its own row blocks.  They read the same pages:
// the block index puts all row groups of a unit on one XCD (workgroups are dealt to the
// eight XCDs by block index modulo 8) at about the same time, so the repeated reads of a
// page are served by that XCD's L2 rather than HBM.
template <bool FP8, int RBW>
struct KSplitCfg {
  using TG = TileGeom<FP8>;
  using QC = QueryCopy<8, RBW>;
  static constexpr int NW = 8;
  static constexpr int kTiles = FP8 ? 4 : 2;
  static constexpr int kPer = PageCopy<FP8, NW>::kPer;
  static constexpr int KS = kDLatent / 32 / 2;  // k-steps per half: 9
  static constexpr int CT = 4;                  // 16-column output tiles per wave
  static constexpr int kQTiles = (QC::kBlocks * 1024 + TG::kPageBytes - 1) / TG::kPageBytes;
  static_assert(RBW == 1 || RBW == 2, "row blocks per workgroup");
  static_assert(kPer * kTiles + QC::kPer <= 63, "outstanding operations exceed vmcnt");
  static_assert(kQTiles < kTiles, "tile plan");
};

template <bool FP8, int RBW>
struct KSplitSmem {
  using C = KSplitCfg<FP8, RBW>;
  __attribute__((aligned(1024))) unsigned char tiles[C::kTiles * C::TG::kPageBytes];
  f32x4 sx[RBW == 2 ? 1 : RBW][4][64];  // k-half 1 partial scores (not used with two row blocks)
  // P^T of the page (bf16); the FP8 row split keeps two pages'
  static constexpr int kPbufBytes = 2 * 64 * 16 * (FP8 && RBW == 2 ? 2 : 1);
  __attribute__((aligned(16))) unsigned char pbuf[RBW][kPbufBytes];
  float red[RBW][4 * 16];                                             // row maxima of the sub-tiles
  float red2[RBW][4 * 16];                                            // row denominators (epilogue)
  int32_t dlen[4];  // the piece's device length (plan path), landed by wave 0's LDS-DMA
};

// The (unit, row group) of this workgroup; false for a block past the last unit (the grid
// is rounded up to whole groups of eight units when there are several row groups).
__device__ __forceinline__ bool unit_of_block(int nwg, int rgroups, int64_t& w, int& g) {
  if (rgroups == 1) {
    w = blockIdx.x;
    g = 0;
    return true;
  }
  const int xcd = blockIdx.x & 7, q = blockIdx.x >> 3;
  const int wb = q / rgroups;
  g = q - wb * rgroups;
  w = (int64_t)wb * 8 + xcd;
  return w < nwg;
}

template <bool FP8, int RBW, bool RS, bool F8QK, bool HID, bool NT, bool ST>
__device__ __forceinline__ void partial_ks(
    const PartialParams& p, const HotArgs& args, const uint16_t* __restrict__ q_ptr,
    const uint8_t* __restrict__ pool, const int32_t* __restrict__ block_table,
    const int32_t* __restrict__ seq_lens, float* __restrict__ part_o, float* __restrict__ part_lse,
    KSplitSmem<FP8, RBW>& sm) {
  using C = KSplitCfg<FP8, RBW>;
  using TG = TileGeom<FP8>;
  constexpr int kTiles = C::kTiles, kPer = C::kPer, CT = C::CT, KS = C::KS;
  // RS (two row blocks): wave w takes sub-tile w & 3 of row block w >> 2 over the whole
  // latent instead of both row blocks over half of it: no partial-score exchange, and
  // every wave shares the softmax work
  static_assert(!RS || RBW == 2, "row split needs two row blocks");
  constexpr int KQ = RS ? 2 * KS : KS;  // k-steps of queries a wave holds
  // F8QK (FP8 pool, row split, on request): QK^T on the FP8 matrix cores, the pool's codes
  // entering as they are and the queries as split-precision E4M3FN pairs; four 32-column
  // k-steps per 128-deep product, the last two k-steps sharing one product (hi and lo side
  // by side).  Only the scores' rounding changes (hi + lo reproduces each bf16 query
  // element, see split_fp8x8); PV^T stays on bf16.
  static_assert(!F8QK || (FP8 && RS && KQ == 18), "FP8 QK^T needs the FP8 row split");
  constexpr int NQ = RS ? 1 : RBW;      // row blocks whose queries a wave holds
  constexpr int kEarlyTiles = kTiles - C::kQTiles;  // tiles not used to stage the queries
  int64_t w;
  int g;
  if (!unit_of_block(args.nwg, args.rgroups, w, g)) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int lrow = lane & 15, lgrp = lane >> 4;
  const int u = wave & 3, kh = wave >> 2;  // sub-tile, k-half
  // this workgroup's row blocks: token, output row of this lane's head, causal lag
  // (an odd row-block count is padded with one row block that repeats the last real one
  // and stores nothing)
  int orow[RBW], lag[RBW], tok[RBW];
  bool head_ok[RBW];
  const int rb_last = args.qlen * args.hgroups - 1;
#pragma unroll
  for (int j = 0; j < RBW; ++j) {
    const int rb = min(g * RBW + j, rb_last);
    const int t = rb / args.hgroups, hg = rb - t * args.hgroups;
    const int head = hg * kRowsPerBlock + lrow;
    head_ok[j] = head < args.heads && g * RBW + j <= rb_last;
    orow[j] = t * args.heads + head;
    tok[j] = t;
    lag[j] = args.causal ? args.qlen - 1 - t : 0;  // token t sees positions < L - lag
  }
  int lag_max = 0;
#pragma unroll
  for (int j = 0; j < RBW; ++j) lag_max = max(lag_max, lag[j]);
  // one row group: this workgroup alone reads its pages, so they may be copied with the
  // non-temporal hint (one row block: as the plan says; two: the ST kernels, which the
  // launcher picks for one-row-group plans that ask for it)
  const PageCopy<FP8, C::NW, RBW == 1 || ST> copy(wave, lane, RBW == 1 ? (bool)args.stream : ST);
  const OperandAddr<FP8> addr(lrow, lgrp, 4 * wave);  // V^T: output column tiles 4w .. 4w+3
  unsigned char* const tiles = sm.tiles;
  using SM = KSplitSmem<FP8, RBW>;
  const uint32_t tiles_lds = lds_addr(sm.tiles);   // LDS base of the workgroup's object
  const uint32_t red_lds = tiles_lds + (uint32_t)(__builtin_offsetof(SM, red) - __builtin_offsetof(SM, tiles));
  const uint32_t red2_lds = tiles_lds + (uint32_t)(__builtin_offsetof(SM, red2) - __builtin_offsetof(SM, tiles));
  const uint32_t pbuf_lds = tiles_lds + (uint32_t)(__builtin_offsetof(SM, pbuf) - __builtin_offsetof(SM, tiles));
  const uint32_t sx_lds = tiles_lds + (uint32_t)(__builtin_offsetof(SM, sx) - __builtin_offsetof(SM, tiles));
  const uint32_t dlen_lds = tiles_lds + (uint32_t)(__builtin_offsetof(SM, dlen) - __builtin_offsetof(SM, tiles));

  auto run_piece = [&](int r, int pb, int pe, int64_t slot, int L) {
    if constexpr (HID) {  // per-(request, token) hidden tails instead of the causal pattern
      lag_max = 0;
#pragma unroll
      for (int j = 0; j < RBW; ++j) {
        lag[j] = min(max(p.hidden[(int64_t)r * args.qlen + tok[j]], 0), L);
        lag_max = max(lag_max, lag[j]);
      }
    }
    const int32_t* trow = block_table + (int64_t)r * args.maxp;
    const int n = pe - pb;
    bool bad = false;
    // page i of the piece, whose block-table entry is id, into tile i % kTiles; an id
    // outside the pool is never dereferenced (page 0 is copied instead, the piece becomes NaN)
    auto page_id = [&](int i) -> int32_t { return i < n ? trow[pb + i] : 0; };
    auto issue_id = [&](int i, int32_t id) {
      if (i >= n) return;
      const int lp = pb + i;
      if (args.bad_id(id)) {
        bad = true;
        id = 0;
      }
      copy(tiles_lds + (i % kTiles) * TG::kPageBytes, pool + (int64_t)id * TG::kPageBytes,
           min(kPage, L - lp * kPage));
    };
    auto issue = [&](int i) { issue_id(i, page_id(i)); };
    // The same copy recorded, then issued in parts (pc_*): a CU queues only about twenty
    // page-copy operations before the issuing waves stall, so the multi-row and FP8
    // kernels spread each copy over the phases of a page.
    uint32_t pc_base = 0;
    const unsigned char* pc_src = pool;
    int pc_valid = kPage;
    bool pc_go = false;
    auto record_copy = [&](int i, int32_t id) {
      pc_go = i < n;
      if (!pc_go) return;
      const int lp = pb + i;
      if (args.bad_id(id)) {
        bad = true;
        id = 0;
      }
      pc_base = tiles_lds + (i % kTiles) * TG::kPageBytes;
      pc_src = pool + (int64_t)id * TG::kPageBytes;
      pc_valid = min(kPage, L - lp * kPage);
    };

    // ---- queries through LDS (one HBM read per workgroup), then the first pages.  The
    // one-row-block bf16 kernel (mostly two pages a piece) fetches the block-table entries
    // of its first pages ahead of the query copies, over LDS-DMA into this wave's slot of
    // the k-half score buffer (untouched until the first page's scores, several barriers
    // later): the wait for them is then explicit and covers nothing else, so the first
    // page copy goes out one memory round trip after entry, while the parameter block's
    // loads are still in flight (valid entries only: the piece's last page for ti >= n,
    // block_table[0] for an empty piece).  The FP8 and two-row-block kernels, whose first
    // pages wait for the queries anyway, measured faster with one scalar load per page
    // (the same fetch: dcp_fp8 +0.7 us, spec_verify +1.0 us a layer-step).
    constexpr bool kEarlyId = !FP8 && RBW == 1;
    static_assert(!kEarlyId || kTiles == 2, "two early entries");
    static_assert(sizeof(sm.sx) >= C::NW * 64, "block-table slots");
    const uint32_t bt_lds = __builtin_amdgcn_readfirstlane(sx_lds + wave * 64);
    int32_t first_id[kTiles] = {};
    if constexpr (kEarlyId) {
      if (lane < kTiles) {
        const int off = n > 0 ? (pb + min(lane, n - 1)) * 4 : 0;
        const int32_t* src = n > 0 ? trow : block_table;
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, %2"
                     :: "s"(bt_lds), "v"(off), "s"(src) : "memory", "m0");
      }
    }
    unsigned char* stage = tiles + kEarlyTiles * TG::kPageBytes;
    typename C::QC(wave, lane)(tiles_lds + kEarlyTiles * TG::kPageBytes, q_ptr + (int64_t)r * args.qlen * args.heads * kDLatent, args.heads,
                               args.hgroups, g * RBW, rb_last);
    if constexpr (kEarlyId) {
      wait_vmcnt<C::QC::kPer>();  // the entries are older than the query copies
      lds_read_ids<kTiles>(bt_lds, first_id);
#pragma unroll
      for (int ti = 0; ti < kTiles; ++ti) first_id[ti] = __builtin_amdgcn_readfirstlane(first_id[ti]);
    }
    // plan path: a request whose device length differs from the plan's gives a NaN piece
    // (the merge carries a NaN LSE to the row).  Wave 0 fetches the length over LDS-DMA
    // between the query copies and the first page copies, so the wait for the queries
    // covers it and no compiler-counted load stays in flight through the page loop; it is
    // compared in the epilogue.
    if (args.plan_n > 0 && wave == 0 && lane == 0) {
      const uint32_t dl = __builtin_amdgcn_readfirstlane(dlen_lds);
      asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, %2"
                   :: "s"(dl), "v"(r * 4), "s"(seq_lens) : "memory", "m0");
    }
    int early = 0;
#pragma unroll
    for (int ti = 0; ti < kEarlyTiles; ++ti) {
      if constexpr (kEarlyId) issue_id(ti, first_id[ti]);
      else issue(ti);
      early += ti < n ? 1 : 0;
    }
    MLA_TL(1);  // the first page copies are out
    args.settle();
    wait_pages<kPer, kEarlyTiles>(early);  // the query copies (and the length) are older: all landed
    barrier_lds();
    i32x4 qf[NQ][KQ];  // this wave's queries: half of each row block's, or all of one
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
#pragma unroll
      for (int s = 0; s < KQ; ++s) {
        const int kk = RS ? s : kh * KS + s;  // depends on the wave: offsets computed, not indexed
        const int jr = RS ? kh : j;
        const int kb = OperandAddr<false>::kbase_of(lrow, lgrp, kk & 1, 0);
        qf[j][s] = *(const i32x4*)(stage + jr * kRowsPerBlock * TileGeom<false>::kRowBytes + kb +
                                   OperandAddr<false>::kstep(kk));
      }
    }
    barrier_lds();  // the staging tiles are free again
    MLA_TL(2);
#pragma unroll
    for (int ti = kEarlyTiles; ti < kTiles; ++ti) {
      if constexpr (kEarlyId) issue_id(ti, first_id[ti]);
      else issue(ti);
    }

    // F8QK: each query row times a power of two 2^a that brings its largest magnitude into
    // [128, 256), split into hi + lo; the scores then come out times 2^a, which the row's
    // score scale takes back
    i32x8 q8h[4], q8l[4], q8t;
    float rsc = args.sscale;  // score scale of this lane's query row
    if constexpr (F8QK) {
      float amax = 0.f;
#pragma unroll
      for (int t = 0; t < KQ; ++t) {
        const bf16x8 v = __builtin_bit_cast(bf16x8, qf[0][t]);
#pragma unroll
        for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf((float)v[e]));
      }
      amax = max_over_rows(amax);  // the four lanes of this row
      const int ex = (int)((__float_as_uint(amax) >> 23) & 0xFF) - 126;  // amax in [2^(ex-1), 2^ex)
      const int a = amax > 0.f ? min(max(8 - ex, -100), 100) : 0;
      const float sc = __uint_as_float((uint32_t)(127 + a) << 23);
      rsc = args.sscale * __uint_as_float((uint32_t)(127 - a) << 23);
      i32x2 h[KQ], l[KQ];
#pragma unroll
      for (int t = 0; t < KQ; ++t) split_fp8x8(qf[0][t], sc, h[t], l[t]);
      // block b holds k-steps 4b, 4b+2, 4b+1, 4b+3 in that order, the order in which the
      // paired LDS reads deliver the key codes
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        q8h[b] = i32x8{h[4 * b][0], h[4 * b][1], h[4 * b + 2][0], h[4 * b + 2][1],
                       h[4 * b + 1][0], h[4 * b + 1][1], h[4 * b + 3][0], h[4 * b + 3][1]};
        q8l[b] = i32x8{l[4 * b][0], l[4 * b][1], l[4 * b + 2][0], l[4 * b + 2][1],
                       l[4 * b + 1][0], l[4 * b + 1][1], l[4 * b + 3][0], l[4 * b + 3][1]};
      }
      q8t = i32x8{h[16][0], h[16][1], h[17][0], h[17][1], l[16][0], l[16][1], l[17][0], l[17][1]};
    }

    float m[RBW], lsum[RBW];  // running row max (log2 units, the same in every wave) and
    f32x4 acc[RBW][CT];       // this lane's share of the denominator (k-half 0 waves; RS:
                              // lsum[0], of the wave's own row block)
#pragma unroll
    for (int j = 0; j < RBW; ++j) {
      m[j] = kNegInf;
      lsum[j] = 0.f;
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) acc[j][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    // FP8 with the row split: two pages an iteration.  One row-max exchange and one P^T
    // exchange serve both pages, and the scores of the two pages are four independent
    // MFMA chains.  The copies of pages i + 2 and i + 3 go out once pages i and i + 1 have
    // landed everywhere (into the tiles of pages i - 2 and i - 1), in parts over the
    // phases of the iteration.
    constexpr bool kPair = FP8 && RS;
    static_assert(!kPair || (kTiles == 4 && kPer == 5), "pair plan: four tiles, five operations a page");
    if constexpr (kPair) {
      // scores of sub-tile u for row block kh on page i (raw: the scale, rsc, comes later)
      auto qk = [&](int i) -> f32x4 {
        const unsigned char* kt = tiles + (i % kTiles) * TG::kPageBytes + u * 16 * TG::kRowBytes;
        f32x4 a[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
        if constexpr (F8QK) {
          // block b's operand: the codes of k-steps 4b, 4b+2, 4b+1, 4b+3 (see the queries)
          i32x2 kr[KQ];
#pragma unroll
          for (int s = 0; s < KQ; ++s)
            kr[s] = *(const i32x2*)(kt + OperandAddr<FP8>::kbase_of(lrow, lgrp, s & 1, u) + OperandAddr<FP8>::kstep(s));
#pragma unroll
          for (int b = 0; b < 4; ++b) {
            const i32x8 k8 = i32x8{kr[4 * b][0], kr[4 * b][1], kr[4 * b + 2][0], kr[4 * b + 2][1],
                                   kr[4 * b + 1][0], kr[4 * b + 1][1], kr[4 * b + 3][0], kr[4 * b + 3][1]};
            a[0] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(k8, q8h[b], a[0], 0, 0, 0, 0, 0, 0);
            a[1] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(k8, q8l[b], a[1], 0, 0, 0, 0, 0, 0);
          }
          const i32x8 k8 = i32x8{kr[16][0], kr[16][1], kr[17][0], kr[17][1], kr[16][0], kr[16][1], kr[17][0], kr[17][1]};
          a[0] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(k8, q8t, a[0], 0, 0, 0, 0, 0, 0);
        } else {
          bf16x8 kf[KQ];
#pragma unroll
          for (int s = 0; s < KQ; ++s)
            kf[s] = fp8x8_to_bf16x8(*(const i32x2*)(kt + OperandAddr<FP8>::kbase_of(lrow, lgrp, s & 1, u) +
                                                    OperandAddr<FP8>::kstep(s)));
#pragma unroll
          for (int s = 0; s < KQ; ++s)
            a[s & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[s], __builtin_bit_cast(bf16x8, qf[0][s]),
                                                               a[s & 1], 0, 0, 0);
        }
        return a[0] + a[1];
      };
      // positions at or past the row block's visible count (only a request's last pages)
      auto mask = [&](int i, f32x4& sv) {
        const int lp = pb + i;
        if ((lp + 1) * kPage > L - lag_max) {
          const int vis = L - (kh ? lag[RBW - 1] : lag[0]) - (lp * kPage + u * 16 + lgrp * 4);
#pragma unroll
          for (int e = 0; e < 4; ++e) sv[e] = e < vis ? sv[e] : kNegInf;
        }
      };
      // O^T += V^T P^T for this wave's 64 columns of both row blocks, page i (its P^T in
      // half pg of the buffer)
      auto pv = [&](int i, int pg) {
        const unsigned char* tile = tiles + (i % kTiles) * TG::kPageBytes;
        bf16x8 va[2][CT];
#pragma unroll
        for (int c = 0; c < 2; ++c) {
#pragma unroll
          for (int ct = 0; ct < CT; ++ct) {
            const unsigned char* va0 = tile + c * 32 * TG::kRowBytes + addr.vbase[ct] + OperandAddr<FP8>::vstep(ct);
            va[c][ct] = fp8x8_to_bf16x8(__builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)va0));
          }
        }
#pragma unroll
        for (int j = 0; j < RBW; ++j) {
          i32x4 p0, p1;
          lds_read_pair_b128(pbuf_lds + j * SM::kPbufBytes + pg * 2048 + lane * 16, p0, p1);
          const bf16x8 pf[2] = {__builtin_bit_cast(bf16x8, p0), __builtin_bit_cast(bf16x8, p1)};
#pragma unroll
          for (int c = 0; c < 2; ++c) {
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
              acc[j][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[c][ct], pf[c], acc[j][ct], 0, 0, 0);
          }
        }
      };
      // pages i + 2 and i + 3: a wave's 2 kPer operations in three parts, page i + 2's
      // [0, kA1) and page i + 3's [0, kB1) at the top, then [kA1, kPer) and [kB1, kB2),
      // then page i + 3's [kB2, kPer): 5 + 4 + 1 (4 + 4 + 2, 6 + 4 and 3 + 4 + 3 measured
      // up to 1% slower)
      constexpr int kA1 = 5, kB1 = 0, kB2 = 4;
      uint32_t cb[2] = {0, 0};
      const unsigned char* cs[2] = {pool, pool};
      int cv[2] = {kPage, kPage};
      bool cg[2] = {false, false};
      auto record_pair = [&](int i, int32_t id0, int32_t id1) {
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const int ip = i + k;
          int32_t id = k ? id1 : id0;
          cg[k] = ip < n;
          if (!cg[k]) continue;
          if (args.bad_id(id)) {
            bad = true;
            id = 0;
          }
          cb[k] = tiles_lds + (ip % kTiles) * TG::kPageBytes;
          cs[k] = pool + (int64_t)id * TG::kPageBytes;
          cv[k] = min(kPage, L - (pb + ip) * kPage);
        }
      };

      int32_t nid0 = page_id(kTiles), nid1 = page_id(kTiles + 1);  // ids of pages i + 2, i + 3
      for (int i = 0; i < n; i += 2) {
        const bool hasB = i + 1 < n;
        // the first pair may leave pages 2 and 3 in flight; later every page issued so
        // far is page i + 1 or older
        if (i == 0) wait_pages<kPer, 2>(min(n, kTiles) - 2);
        else wait_vmcnt<0>();
        barrier_lds();  // pages i, i + 1 landed; every wave is done with pages i - 2, i - 1
        if (i < 4) MLA_TL(3 + i / 2);
        cg[0] = cg[1] = false;
        if (i > 0) record_pair(i + 2, __builtin_amdgcn_readfirstlane(nid0), __builtin_amdgcn_readfirstlane(nid1));
        if (cg[0]) copy.template part<0, kA1>(cb[0], cs[0], cv[0]);
        if (cg[1]) copy.template part<0, kB1>(cb[1], cs[1], cv[1]);

        f32x4 sa = qk(i);
        f32x4 sb = qk(hasB ? i + 1 : i);
        mask(i, sa);
        if (hasB) mask(i + 1, sb);
        else sb = f32x4{kNegInf, kNegInf, kNegInf, kNegInf};
        // (scalar loads here land under the MFMAs; they share a counter with the LDS reads)
        nid0 = page_id(i + 4);
        nid1 = page_id(i + 5);
        float mx = fmaxf(fmaxf(fmaxf(sa[0], sa[1]), fmaxf(sa[2], sa[3])),
                         fmaxf(fmaxf(sb[0], sb[1]), fmaxf(sb[2], sb[3])));
        mx = max_over_rows(mx);
        if (lgrp == 0) sm.red[kh][u * 16 + lrow] = mx * rsc;
        barrier_lds();  // both pages' row maxima
        if (cg[0]) copy.template part<kA1, kPer>(cb[0], cs[0], cv[0]);
        if (cg[1]) copy.template part<kB1, kB2>(cb[1], cs[1], cv[1]);

        // online softmax update over both pages (exact running max; O rescaled only when
        // some row's max grows), P^T of this wave's sub-tile of each
        float alpha[RBW], msubs[RBW];
        bool grown = false;
        // (one round trip for both row blocks, as in the one-page loop, measured 0.5 us a
        // layer-step slower here)
#pragma unroll
        for (int j = 0; j < RBW; ++j) {
          const float m2 = lds_max_of<4>(red_lds + 4 * (j * 64 + lrow), kNegInf);
          const bool grow = m2 > m[j];
          const float m_new = grow ? m2 : m[j];
          const float msub = m_new == kNegInf ? 0.f : m_new;
          msubs[j] = msub;
          alpha[j] = grow ? exp2_fast(m[j] - msub) : 1.f;
          grown |= grow;
          m[j] = m_new;
        }
        const float msub = kh ? msubs[RBW - 1] : msubs[0];
        float ps = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sa[e] = exp2_fast(fmaf(sa[e], rsc, -msub));
          sb[e] = exp2_fast(fmaf(sb[e], rsc, -msub));  // -inf (no page B) -> 0
          ps += sa[e] + sb[e];
        }
        lsum[0] = fmaf(lsum[0], kh ? alpha[RBW - 1] : alpha[0], ps);
        unsigned char* pw = sm.pbuf[kh] + ((u >> 1) * 64 + lane) * 16 + (u & 1) * 8;
        *(bf16x4*)pw = bf16x4{(__bf16)sa[0], (__bf16)sa[1], (__bf16)sa[2], (__bf16)sa[3]};
        *(bf16x4*)(pw + 2048) = bf16x4{(__bf16)sb[0], (__bf16)sb[1], (__bf16)sb[2], (__bf16)sb[3]};
        if (__builtin_amdgcn_ballot_w64(grown)) {
#pragma unroll
          for (int j = 0; j < RBW; ++j) {
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) acc[j][ct] *= alpha[j];
          }
        }
        barrier_lds();  // both pages' P^T
        if (cg[1]) copy.template part<kB2, kPer>(cb[1], cs[1], cv[1]);

        pv(i, 0);
        if (hasB) pv(i + 1, 1);
      }
    } else {
      // Multi-row and FP8 kernels: the copy of page i + kTiles - 1 goes out as soon as page i
      // has landed everywhere.  The barrier that says so also says every wave is done with
      // page i - 1, whose tile it reuses, so no barrier of its own is needed, and its
      // block-table entry is read one page earlier, off the critical path.  The one-row-block
      // bf16 kernel (mostly a few pages per piece) measured faster with the copy of page
      // i + kTiles issued after a barrier at the end of page i.
      constexpr bool kTopIssue = FP8 || RBW == 2;
      // Parts of a top-issued copy: operations [0, kS1) at the top, [kS1, kSm) after K
      // read kMidRead of the QK^T phase (the copy engine drains them under the MFMAs),
      // [kSm, kS2) after the row-max barrier, the rest after the P^T barrier.  With four
      // FP8 tiles a copy has three pages to land (2 + 0 + 2 + 1 of five); with two bf16
      // tiles it must land within the page: 3 + 3 + 3 of nine (6 + 3 at the top and after
      // the row-max barrier 1.2% slower, 2 + 4 + 3 and 3 + 4 + 2 about as fast; 4 + 4 + 1,
      // 5 + 3 + 1, 3 + 3 + 3 after the P^T barrier, and the splits that spill, slower).
      constexpr int kS1 = kTiles >= 4 ? 2 : 3, kS2 = kTiles >= 4 ? 4 : kPer;
      constexpr int kSm = kTiles >= 4 ? kS1 : 6, kMidRead = 5;
      int32_t next_id = kTopIssue ? page_id(kTiles) : 0;
      for (int i = 0; i < n; ++i) {
        // the pages issued after page i may stay in flight (top issue: kTiles - 1 of them
        // before the loop's first copy, kTiles - 2 afterwards)
        if constexpr (kTopIssue)
          wait_pages<kPer, kTiles - 1>(min(n, i == 0 ? kTiles : i + kTiles - 1) - (i + 1));
        else
          wait_pages<kPer, kTiles - 1>(min(n, i + kTiles) - (i + 1));
        barrier_lds();  // every wave's copies of page i have landed
        if (i < 2) MLA_TL(3 + i);
        if constexpr (kTopIssue) {
          pc_go = false;
          if (i > 0) record_copy(i + kTiles - 1, __builtin_amdgcn_readfirstlane(next_id));  // uniform
          if (pc_go) copy.template part<0, kS1>(pc_base, pc_src, pc_valid);
        }
        const unsigned char* tile = tiles + (i % kTiles) * TG::kPageBytes;
        const int lp = pb + i;

        // ---- partial S^T of sub-tile u over this wave's k-half, then the V^T operands of
        // this wave's output columns (both 32-position chunks; they do not depend on the
        // softmax, so these transposing reads run under the MFMAs and the exchanges)
        const unsigned char* kt = tile + u * 16 * TG::kRowBytes;
        bf16x8 kf[KQ];
#pragma unroll
        for (int s = 0; s < KQ; ++s) {
          const int kk = RS ? s : kh * KS + s;
          const unsigned char* ka =
              kt + OperandAddr<FP8>::kbase_of(lrow, lgrp, kk & 1, u) + OperandAddr<FP8>::kstep(kk);
          if constexpr (FP8) kf[s] = fp8x8_to_bf16x8(*(const i32x2*)ka);
          else kf[s] = *(const bf16x8*)ka;
          if constexpr (kTopIssue && kSm > kS1) {
            if (s == kMidRead && pc_go) copy.template part<kS1, kSm>(pc_base, pc_src, pc_valid);
          }
        }
        f32x4 sp[RBW];
#pragma unroll
        for (int j = 0; j < RBW; ++j) sp[j] = f32x4{0.f, 0.f, 0.f, 0.f};
        if constexpr (RS) {
          // two accumulators (even and odd k-steps) halve the dependent MFMA chain
#pragma unroll
          for (int s = 0; s < KQ; ++s)
            sp[s & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[s], __builtin_bit_cast(bf16x8, qf[0][s]),
                                                                sp[s & 1], 0, 0, 0);
          sp[0] += sp[1];
        } else {
#pragma unroll
          for (int s = 0; s < KS; ++s) {
#pragma unroll
            for (int j = 0; j < RBW; ++j)
              sp[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[s], __builtin_bit_cast(bf16x8, qf[j][s]),
                                                              sp[j], 0, 0, 0);
          }
        }
        bf16x8 va[2][CT];
        auto read_v = [&]() {
#pragma unroll
          for (int c = 0; c < 2; ++c) {
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
              const unsigned char* va0 =
                  tile + c * 32 * TG::kRowBytes + addr.vbase[ct] + OperandAddr<FP8>::vstep(ct);
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
        };
        // bf16 with two row blocks: no registers to spare for early V^T operands
        constexpr bool kEarlyV = FP8 || RBW == 1;
        if constexpr (kEarlyV) read_v();
        if constexpr (!FP8 && RS) {
          // four K reads ahead of the MFMAs, then one MFMA per remaining read
          __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
          for (int s = 0; s < KQ - 4; ++s) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          }
          __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
        } else if constexpr (!FP8 && RBW == 1) {
          // instruction order: six K reads ahead of the MFMAs, then one MFMA per remaining
          // read; the sixteen V^T reads go between the last six MFMAs
          __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
#pragma unroll
          for (int s = 0; s < 3; ++s) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          }
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
          }
#pragma unroll
          for (int s = 0; s < 2; ++s) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
          }
        } else if constexpr (!FP8) {
          // two row blocks: four K reads ahead, then one k-step's two MFMAs per remaining read
          __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
          for (int s = 0; s < 5; ++s) {
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          }
          __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
        }

        // ---- the k-halves meet: half 1 hands its partial scores to half 0, which scales,
        // masks and takes its sub-tile's row max (RS: every wave has whole scores)
        if constexpr (!RS) {
          if (kh == 1) {
#pragma unroll
            for (int j = 0; j < RBW; ++j) sm.sx[j][u][lane] = sp[j];
          }
          barrier_lds();
        }
        // raw scores (the scale is applied to the max and inside the exponent); positions
        // at or past a row block's visible count are masked, which only a request's last
        // pages need
        f32x4 sv[RBW];
        if constexpr (RS) {
          sv[0] = sp[0];
          if ((lp + 1) * kPage > L - lag_max) {
            const int vis = L - (kh ? lag[RBW - 1] : lag[0]) - (lp * kPage + u * 16 + lgrp * 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) sv[0][e] = e < vis ? sv[0][e] : kNegInf;
          }
          float mx = fmaxf(fmaxf(sv[0][0], sv[0][1]), fmaxf(sv[0][2], sv[0][3]));
          mx = max_over_rows(mx);
          if (lgrp == 0) sm.red[kh][u * 16 + lrow] = mx * rsc;
        } else if (kh == 0) {
          const bool whole = (lp + 1) * kPage <= L - lag_max;
#pragma unroll
          for (int j = 0; j < RBW; ++j) {
            const f32x4 other = sm.sx[j][u][lane];
            sv[j] = sp[j] + other;
            if (!whole) {
              const int vis = L - lag[j] - (lp * kPage + u * 16 + lgrp * 4);
#pragma unroll
              for (int e = 0; e < 4; ++e) sv[j][e] = e < vis ? sv[j][e] : kNegInf;
            }
            float mx = fmaxf(fmaxf(sv[j][0], sv[j][1]), fmaxf(sv[j][2], sv[j][3]));
            mx = max_over_rows(mx);
            if (lgrp == 0) sm.red[j][u * 16 + lrow] = mx * args.sscale;
          }
        }
        barrier_lds();
        if constexpr (kTopIssue) {
          if (pc_go) copy.template part<kSm, kS2>(pc_base, pc_src, pc_valid);
        }

        // ---- online softmax update; half 0 builds P^T of its sub-tile for every wave.  The
        // running max is exact (the largest weight of a row is exactly 1 in bf16); O is
        // rescaled only on pages that raise some row's max, which become rare as the piece
        // goes on.
        float alpha[RBW], msubs[RBW];
        bool grown = false;
        float mxs[RBW];  // both row blocks' maxima in one round trip (spec_verify partial -2 us)
        lds_row_maxima<RBW>(red_lds + 4 * lrow, mxs);
#pragma unroll
        for (int j = 0; j < RBW; ++j) {
          const float mx = mxs[j];
          const bool grow = mx > m[j];  // m = -inf: any finite max
          const float m_new = grow ? mx : m[j];
          const float msub = m_new == kNegInf ? 0.f : m_new;
          msubs[j] = msub;
          alpha[j] = grow ? exp2_fast(m[j] - msub) : 1.f;  // m = -inf -> 0
          grown |= grow;
          m[j] = m_new;
          if (!RS && kh == 0) {
            float ps = 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              sv[j][e] = exp2_fast(fmaf(sv[j][e], args.sscale, -msub));
              ps += sv[j][e];
            }
            lsum[j] = fmaf(lsum[j], alpha[j], ps);
            *(bf16x4*)(sm.pbuf[j] + ((u >> 1) * 64 + lane) * 16 + (u & 1) * 8) =
                bf16x4{(__bf16)sv[j][0], (__bf16)sv[j][1], (__bf16)sv[j][2], (__bf16)sv[j][3]};
          }
        }
        if constexpr (RS) {  // this wave's sub-tile of its row block
          const float msub = kh ? msubs[RBW - 1] : msubs[0];
          float ps = 0.f;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            sv[0][e] = exp2_fast(fmaf(sv[0][e], rsc, -msub));
            ps += sv[0][e];
          }
          lsum[0] = fmaf(lsum[0], kh ? alpha[RBW - 1] : alpha[0], ps);
          *(bf16x4*)(sm.pbuf[kh] + ((u >> 1) * 64 + lane) * 16 + (u & 1) * 8) =
              bf16x4{(__bf16)sv[0][0], (__bf16)sv[0][1], (__bf16)sv[0][2], (__bf16)sv[0][3]};
        }
        // every lane of every wave sees the same maxima, so the branch is uniform
        if (__builtin_amdgcn_ballot_w64(grown)) {
#pragma unroll
          for (int j = 0; j < RBW; ++j) {
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) acc[j][ct] *= alpha[j];
          }
        }
        barrier_lds();
        if constexpr (kTopIssue) {
          if (pc_go) copy.template part<kS2, kPer>(pc_base, pc_src, pc_valid);
        }

        // ---- O^T += V^T P^T for this wave's 64 columns of every row block
        if constexpr (!kEarlyV) read_v();
#pragma unroll
        for (int j = 0; j < RBW; ++j) {
          i32x4 p0, p1;
          lds_read_pair_b128(pbuf_lds + j * SM::kPbufBytes + lane * 16, p0, p1);
          const bf16x8 pf[2] = {__builtin_bit_cast(bf16x8, p0), __builtin_bit_cast(bf16x8, p1)};
#pragma unroll
          for (int c = 0; c < 2; ++c) {
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
              acc[j][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[c][ct], pf[c], acc[j][ct], 0, 0, 0);
          }
        }
        if constexpr (kTopIssue) {
          // (a scalar load here lands under the MFMAs; earlier, it would hold up the first
          // wait for the page's LDS reads, which shares its counter)
          if (i > 0) next_id = page_id(i + kTiles);
        } else if (i + kTiles < n) {
          barrier_lds();  // every wave is done with this tile
          issue(i + kTiles);
        }
      }
    }

    // ---- epilogue: the row denominators from the four k-half 0 waves, normalise, store
    if constexpr (RS) {
      const float ls = sum_over_rows(lsum[0]);
      if (lgrp == 0) sm.red2[kh][u * 16 + lrow] = ls;
    } else {
#pragma unroll
      for (int j = 0; j < RBW; ++j) {
        const float ls = sum_over_rows(lsum[j]);
        if (kh == 0 && lgrp == 0) sm.red2[j][u * 16 + lrow] = ls;
      }
    }
    barrier_lds();
    MLA_TL(5);
    int dev_len = L;
#pragma unroll
    for (int j = 0; j < RBW; ++j) {
      float ls;
      if (j == 0) {  // the device length comes with the first row block's denominators
        int32_t dl;
        ls = lds_sum4_and_b32(red2_lds + 4 * lrow, dlen_lds, dl);
        if (args.plan_n > 0) dev_len = dl;
      } else {
        ls = lds_sum_of<4>(red2_lds + 4 * (j * 64 + lrow));
      }
      const bool empty = m[j] == kNegInf;
      float oscale = empty ? 0.f : args.vscale / ls;
      float lse = empty ? kNegInf : (m[j] + log2_fast(ls)) * kLn2;
      if (bad || dev_len != L) {
        oscale = __builtin_nanf("");
        lse = __builtin_nanf("");
      }
      if constexpr (NT) {
        // Whole 128-byte lines per store instruction.  A lane holds 4 columns of each half of
        // a 32-column line of its row (tiles ct = 2k and 2k + 1); lanes lrow and lrow ^ 8
        // trade one half, so that the first store writes the whole lines of rows 0-7 of the
        // block and the second those of rows 8-15 (eight lanes a line) instead of every
        // store writing half lines of all 16 rows.
        const bool lo = lrow < 8;
        const int head = orow[j] - tok[j] * args.heads;
        const bool mate_ok = g * RBW + j <= rb_last && (head ^ 8) < args.heads;
        const int64_t mate_row = orow[j] + (lo ? 8 : -8);
#pragma unroll
        for (int ct = 0; ct < CT; ct += 2) {
          const f32x4 a = acc[j][ct] * oscale, b = acc[j][ct + 1] * oscale;
          const f32x4 give = lo ? b : a;
          f32x4 got;  // lane lrow ^ 8's: a DPP rotate by 8 within each 16-lane row
#pragma unroll
          for (int e = 0; e < 4; ++e)
            got[e] = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(give[e]), 0x128, 0xF, 0xF, false));
          const int c0 = 64 * wave + 16 * ct + 4 * lgrp;  // a's columns; b's are c0 + 16
          if (lo ? head_ok[j] : mate_ok)
            store_partial<true>(part_o, lo ? orow[j] : mate_row, lo ? c0 : c0 + 16, args.nslots, slot, lo ? a : got);
          if (lo ? mate_ok : head_ok[j])
            store_partial<true>(part_o, lo ? mate_row : orow[j], lo ? c0 : c0 + 16, args.nslots, slot, lo ? got : b);
        }
        if (head_ok[j] && wave == 0 && lgrp == 0) part_lse[(int64_t)orow[j] * args.nslots + slot] = lse;
      } else if (head_ok[j]) {
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
          store_partial<NT>(part_o, orow[j], 64 * wave + 16 * ct + 4 * lgrp, args.nslots, slot,
                        acc[j][ct] * oscale);
        if (wave == 0 && lgrp == 0) part_lse[(int64_t)orow[j] * args.nslots + slot] = lse;
      }
    }
#ifdef MLA_TIMELINE
    MLA_TL(6);
    wait_vmcnt<0>();
    MLA_TL(7);
#endif
    barrier_lds();  // tiles and exchange buffers are reused by the next piece
  };

  // the cross-wave exchange of the device-length scan borrows the denominator buffer, which
  // the first piece writes only after several barriers
  static_assert(sizeof(sm.red2) >= (C::NW + 2) * sizeof(int64_t), "scan exchange");
  for_each_piece<C::NW>(p, args, seq_lens, w, reinterpret_cast<int64_t*>(&sm.red2[0][0]), run_piece);
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
  // a NaN LSE (a piece that met a bad page id) must reach the output (a select, not a
  // branch: fmaxf alone would return the other operand)
  const float m = fmaxf(a, b);
  return (a == a && b == b) ? m : __builtin_nanf("");
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

// Device lengths under SPLIT_BALANCED (a batch beyond the plan's argument copy): the page
// total P, the page prefix pre0 of request g0 and the page counts pr0, pr1 of requests g0
// and g0 + 1, by a reduction of seq_lens over the workgroup's NWAVES waves (thread t takes
// requests t, t + 64 NWAVES, ...).  Every thread of the workgroup calls it (one barrier
// when there are several waves).
struct DevicePages {
  int64_t P, pre0, pr0, pr1;
};
template <int NWAVES>
__device__ __forceinline__ DevicePages device_pages(const int32_t* __restrict__ seq_lens, int batch,
                                                    int maxp, int64_t g0,
                                                    int64_t (&xs)[NWAVES][4]) {
  int64_t v[4] = {0, 0, 0, 0};
  for (int r = threadIdx.x; r < batch; r += 64 * NWAVES) {
    const int pg = pages_of(seq_lens[r], maxp);
    v[0] += pg;
    v[1] += r < g0 ? pg : 0;
    v[2] += r == g0 ? pg : 0;
    v[3] += r == g0 + 1 ? pg : 0;
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v[k] += __shfl_xor(v[k], off);
    if (NWAVES > 1 && lane == 0) xs[wave][k] = v[k];
  }
  if constexpr (NWAVES == 1) return DevicePages{v[0], v[1], v[2], v[3]};
  __syncthreads();
  DevicePages d{0, 0, 0, 0};
#pragma unroll
  for (int wv = 0; wv < NWAVES; ++wv) {
    d.P += xs[wv][0];
    d.pre0 += xs[wv][1];
    d.pr0 += xs[wv][2];
    d.pr1 += xs[wv][3];
  }
  return d;
}

// Slot range [s0, s1) of request grp's partial answers.  Under SPLIT_BALANCED every work
// unit owns at least one page (W <= P), so every slot in the range holds a piece.  A
// one-request plan needs only the preloaded arguments here, so its first loads go out at
// entry; the plan path reads the plan's prefix page counts from the parameter block.  (A
// device length that differs from the plan's is caught by the partial stage, whose
// pieces of that request are NaN: every request of a plan has at least one piece.)
// Device lengths under SPLIT_BALANCED come in `dp` (device_pages with g0 = grp or
// grp - 1).
__device__ __forceinline__ void decode_slots(const MergeParams& p, int64_t grp, int plan_n, int mode,
                                             int nsplits, int nwg, const DevicePages& dp, int64_t g0,
                                             int64_t& s0, int64_t& s1, bool& inconsistent) {
  const int64_t total = p.total_pages;  // plan and device paths only
  if (plan_n == 1) {  // one request
    s1 = mode == SPLIT_FIXED ? nsplits : nwg;
  } else if (plan_n > 0) {  // slot range from the plan's lengths
    if (mode == SPLIT_FIXED) {
      s0 = grp * nsplits;
      s1 = s0 + nsplits;
    } else {
      const int64_t pre = p.plan.pre[grp], pr = p.plan.pre[grp + 1] - pre;
      s0 = balanced_wg_of(pre, total, nwg) + grp;
      s1 = balanced_wg_of(pre + pr - 1, total, nwg) + grp + 1;
    }
  } else if (mode == SPLIT_FIXED) {
    s0 = grp * nsplits;
    s1 = s0 + nsplits;
  } else {
    const bool second = grp != g0;
    const int64_t pre = second ? dp.pre0 + dp.pr0 : dp.pre0, pr = second ? dp.pr1 : dp.pr0;
    inconsistent = dp.P != total;
    if (pr > 0 && !inconsistent) {
      s0 = balanced_wg_of(pre, dp.P, nwg) + grp;
      s1 = balanced_wg_of(pre + pr - 1, dp.P, nwg) + grp + 1;
    }
  }
}

// The leading arguments (up to the parameter block) are preloaded into SGPRs: the first
// loads of a merge need nothing else.
#define MLA_MERGE_LEAD_ARGS                                                                        \
  const void* __restrict__ lead_part_o, const float* __restrict__ lead_part_lse, int32_t a_rows32,  \
      int32_t a_nwg, int32_t a_nsplits, int32_t a_mode, int32_t a_plan_n, int32_t a_nparts,          \
      int32_t a_nslots, int32_t a_len0
#define MLA_MERGE_LEAD_VALUES(p)                                                                    \
  (p).part_o, (p).part_lse, (int32_t)(p).rows, (p).num_wg, (p).num_splits, (p).split_mode, (p).plan.n, \
      (p).num_parts, (p).num_slots, (p).plan.len[0]

template <bool PART_BF16, bool OUT_BF16, bool DECODE>
__global__ __launch_bounds__(kMergeThreads) void mla_merge_kernel(MLA_MERGE_LEAD_ARGS, MergeParams p) {
  using MG = MergeGeom<PART_BF16>;
  MLA_TL_MERGE(0);
  constexpr int kCPT = MG::kCPT, kTPS = MG::kTPS, kSPP = MG::kSPP, kPasses = MG::kPasses;
  __shared__ float sm_m[kMergeWaves];
  __shared__ float sm_acc[kMergeWaves][kTPS][kCPT];
  __shared__ float sm_den[kMergeWaves];
  __shared__ int64_t sm_xs[kMergeWaves][4];
  const int64_t a_rows = a_rows32;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int sl = tid / kTPS, cp = tid - (tid / kTPS) * kTPS;
  const int64_t unit = blockIdx.x;
  const int64_t orow = unit / kMergeChunks;
  const int chunk = (int)(unit - orow * kMergeChunks);
  const int64_t grp = (int64_t)((uint32_t)orow / (uint32_t)a_rows);  // rows * groups < 2^31
  const int64_t row = orow - grp * a_rows;

  // slot range [s0, s1) of this group
  int64_t s0 = 0, s1 = 0;
  bool inconsistent = false;
  DevicePages dp{0, 0, 0, 0};
  if constexpr (!DECODE) {
    s1 = a_nparts;
  } else {
    if (a_plan_n == 0 && a_mode == SPLIT_BALANCED)  // uniform over the workgroup
      dp = device_pages<kMergeWaves>(p.seq_lens, p.batch, p.max_pages, grp, sm_xs);
    decode_slots(p, grp, a_plan_n, a_mode, a_nsplits, a_nwg, dp, grp, s0, s1, inconsistent);
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

  // first round: every pass's LSE, then every pass's O, all in flight together (loads
  // complete in order, so the LSE maximum and its exchange need not wait for the O loads).
  // Slots past the range load slot s0 (always a valid address) and are masked afterwards,
  // so the loads carry no branches.
  float o[kPasses][kCPT];
  float l[kPasses];
#pragma unroll
  for (int k = 0; k < kPasses; ++k) {
    const int64_t s = s0 + sl + kSPP * k;
    l[k] = lead_part_lse[lse_index(s < s1 ? s : s0)];
  }
#pragma unroll
  for (int k = 0; k < kPasses; ++k) {
    const int64_t s = s0 + sl + kSPP * k;
    load_piece<PART_BF16>(lead_part_o, o_index(s < s1 ? s : s0), o[k]);
  }
#pragma unroll
  for (int k = 0; k < kPasses; ++k) {
    const bool ok = s0 + sl + kSPP * k < s1;
    l[k] = ok ? l[k] : kNegInf;
#pragma unroll
    for (int c = 0; c < kCPT; ++c) o[k][c] = ok ? o[k][c] : 0.f;
  }
  // M over all slots (later rounds: LSEs only)
  float mx = kNegInf;
#pragma unroll
  for (int k = 0; k < kPasses; ++k) mx = nan_max(mx, l[k]);
  for (int64_t s = s0 + 256 + tid; s < s1; s += kMergeThreads) mx = nan_max(mx, lead_part_lse[lse_index(s)]);
  mx = wave_combine<1>(mx, [](float a, float b) { return nan_max(a, b); });
  if (lane == 0) sm_m[wave] = mx;
  __syncthreads();
  MLA_TL_MERGE(1);
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
        const float a = exp2_fast((lead_part_lse[lse_index(s)] - M) * kLog2e);
        float v[kCPT];
        load_piece<PART_BF16>(lead_part_o, o_index(s), v);
#pragma unroll
        for (int c = 0; c < kCPT; ++c) acc[c] += a * v[c];
        den += a;
      }
    }
  }
#ifdef MLA_TIMELINE
  asm volatile("" ::"v"(acc[0]), "v"(acc[kCPT - 1]), "v"(den));
  MLA_TL_MERGE(2);
#endif
  // sum over the slot lanes: lanes cp + kTPS k of a wave, then the waves.  Every thread of
  // a slot lane holds the same weights, so the denominator is summed over slot lanes only.
  auto plus = [](float a, float b) { return a + b; };
#pragma unroll
  for (int c = 0; c < kCPT; ++c) acc[c] = wave_combine<kTPS>(acc[c], plus);
  den = wave_combine<kTPS>(den, plus);
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
  MLA_TL_MERGE(3);
}

// Row-wise merge, for plans whose rows have at most kRowSlots partial answers each (many
// rows, few pieces per request: multi-token verification, large batches, DCP shards).
// One wave per (output row, 256-column half), each lane owning 4 of the row's columns;
// all of the row's partial answers and LSEs are loaded in one round trip, the LSE maximum
// and the weights are reduced across the wave's lanes, and each lane forms its columns'
// weighted sum.  Block b serves row b / 2, half b % 2.  One-wave workgroups spread the
// loads over as many compute units as there are row halves (a compute unit takes in about
// 55 GB/s): with 16 rows of 16 parts (tiny) four-wave workgroups left the merge waiting
// 1.1 us on its loads.
constexpr int kRowSlots = 32;
constexpr int kRowMergeThreads = 64;

template <bool PART_BF16, bool OUT_BF16, bool DECODE>
__global__ __launch_bounds__(kRowMergeThreads) void mla_merge_rows_kernel(MLA_MERGE_LEAD_ARGS, MergeParams p,
                                                                         int64_t total_rows) {
  MLA_TL_MERGE(0);
  const int64_t a_rows = a_rows32;
  const int lane = threadIdx.x;
  const int64_t orow = (int64_t)(blockIdx.x >> 1);  // < total_rows: the grid is 2 total_rows
  const int col = (blockIdx.x & 1) * 256 + lane * 4;
  const int64_t grp = (int64_t)((uint32_t)orow / (uint32_t)a_rows);  // rows * groups < 2^31
  const int64_t row = orow - grp * a_rows;
  DevicePages dp{0, 0, 0, 0};
  if (DECODE && a_plan_n == 0 && a_mode == SPLIT_BALANCED) {  // uniform over the workgroup
    int64_t unused[1][4];
    dp = device_pages<1>(p.seq_lens, p.batch, p.max_pages, grp, unused);
  }
  const int64_t g0 = grp;

  int64_t s0 = 0, s1 = 0;
  bool inconsistent = false;
  if constexpr (!DECODE) s1 = a_nparts;
  else decode_slots(p, grp, a_plan_n, a_mode, a_nsplits, a_nwg, dp, g0, s0, s1, inconsistent);
  const int ns = (int)(s1 - s0);
  auto o_index = [&](int64_t s) -> int64_t {
    if constexpr (DECODE) return ((row * kMergeChunks + (col >> 5)) * a_nslots + s) * kMergeCols + (col & 31);
    else return (s * a_rows + row) * kDV + col;
  };
  // all loads of the row at once: lane k < ns holds LSE of slot s0 + k (lanes past ns load
  // the range's first slot, a valid address, and are masked)
  const int64_t ls = s0 + (lane < ns ? lane : 0);
  const float lraw = lead_part_lse[DECODE ? row * a_nslots + ls : ls * a_rows + row];
  f32x4 o[kRowSlots];
#pragma unroll
  for (int k = 0; k < kRowSlots; ++k) {
    if (k < ns) {  // uniform
      if constexpr (PART_BF16) {
        const bf16x4 b = *(const bf16x4*)((const __bf16*)lead_part_o + o_index(s0 + k));
        o[k] = f32x4{(float)b[0], (float)b[1], (float)b[2], (float)b[3]};
      } else {
        o[k] = *(const f32x4*)((const float*)lead_part_o + o_index(s0 + k));
      }
    }
  }
  inconsistent = inconsistent || ns > kRowSlots;
  const float l = lane < ns ? lraw : kNegInf;
  const float M = wave_combine<1>(l, [](float x, float y) { return nan_max(x, y); });
  MLA_TL_MERGE(1);
  const float a = M == kNegInf ? 0.f : exp2_fast((l - M) * kLog2e);  // lanes past ns: 0
  const float den = wave_combine<1>(a, [](float x, float y) { return x + y; });
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int k = 0; k < kRowSlots; ++k) {
    if (k < ns) acc += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(a), k)) * o[k];
  }
  const bool empty = M == kNegInf && !inconsistent;
  f32x4 v = empty ? f32x4{0.f, 0.f, 0.f, 0.f} : acc * (1.0f / den);
  if (inconsistent) v = f32x4{__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf("")};
  if (p.out) {
    const int64_t off = orow * kDV + col;
    if constexpr (OUT_BF16)
      *(bf16x4*)((__bf16*)p.out + off) = bf16x4{(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
    else
      *(f32x4*)((float*)p.out + off) = v;
  }
  if (p.out_lse && (blockIdx.x & 1) == 0 && lane == 0)
    p.out_lse[orow] = inconsistent ? __builtin_nanf("") : (empty ? kNegInf : M + log2_fast(den) * kLn2);
  MLA_TL_MERGE(3);
}

// ------------------------------------------------------------------- cache append
//
// One workgroup per new row (request r, token t): 72 lanes take 8 of the 576 values each
// (16 bytes of bf16).  bf16 pools get the bits; FP8 pools get the E4M3FN code of the fp32
// quotient x / scale, converted two at a time by the gfx950 conversion instruction
// (round to nearest even) after a clamp to +-448, which makes it saturate.
constexpr int kAppendThreads = 128;

template <bool FP8>
__global__ __launch_bounds__(kAppendThreads) void mla_kv_append_kernel(
    uint8_t* __restrict__ pool, int64_t num_pages, const int32_t* __restrict__ block_table,
    int32_t max_pages, const int32_t* __restrict__ seq_lens, const uint16_t* __restrict__ latents,
    int32_t q_len, float kv_scale) {
  // every argument in one batch of scalar loads (the compiler would fetch them lazily,
  // one round trip each), then the latents: their load overlaps the length -> page-id chain
  asm volatile("" ::"s"(pool), "s"(num_pages), "s"(block_table), "s"(max_pages), "s"(seq_lens),
               "s"(latents), "s"(q_len), "s"(kv_scale));
  const int i = threadIdx.x;
  if (i >= kDLatent / 8) return;
  const int r = blockIdx.x / q_len, t = blockIdx.x - r * q_len;
  const bf16x8 x = *(const bf16x8*)(latents + (int64_t)blockIdx.x * kDLatent + 8 * i);
  asm volatile("" ::: "memory");  // keeps the latent load ahead of the chain below
  const int j = seq_lens[r] - q_len + t;  // the new position
  // the table entry is read at a clamped (in-bounds) index whatever j is, so that no
  // branch separates the loads; the checks only decide the store
  const int pg = min(max(j, 0) / kPage, max_pages - 1);
  const int32_t id = block_table[(int64_t)r * max_pages + pg];
  if (j < 0 || j / kPage >= max_pages || id < 0 || id >= num_pages) return;
  const int64_t row = (int64_t)id * kPage + j % kPage;
  if constexpr (!FP8) {
    *(bf16x8*)(pool + (row * kDLatent + 8 * i) * 2) = x;
  } else {
    float v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float q = (float)x[k] / kv_scale;  // correctly rounded fp32 division
      v[k] = q != q ? q : fminf(fmaxf(q, -448.f), 448.f);
    }
    i32x2 codes;
    codes[0] = __builtin_amdgcn_cvt_pk_fp8_f32(v[0], v[1], 0, false);
    codes[0] = __builtin_amdgcn_cvt_pk_fp8_f32(v[2], v[3], codes[0], true);
    codes[1] = __builtin_amdgcn_cvt_pk_fp8_f32(v[4], v[5], 0, false);
    codes[1] = __builtin_amdgcn_cvt_pk_fp8_f32(v[6], v[7], codes[1], true);
    *(i32x2*)(pool + row * kDLatent + 8 * i) = codes;
  }
}

// ------------------------------------------------------------------- read reference
//
// What the partial stage's page stream would cost with no attention arithmetic at all:
// every 16-byte word of a buffer read once, either into registers (plain vector loads,
// four in flight per thread) or into LDS with the same 128-bit direct copies the partial
// stage uses (two pages' worth, 144 KiB, per workgroup).  Nothing is written unless the
// (practically impossible) checksum below matches, so the kernels are pure reads.
constexpr int kReadThreads = 512;
constexpr int kReadChunk = 2 * kPage * kDLatent * 2;  // 147,456 B: the bf16 partial stage's two tiles

__global__ __launch_bounds__(kReadThreads) void mla_read_plain_kernel(const i32x4* __restrict__ buf, int64_t n16,
                                                                       uint32_t* __restrict__ sink) {
  const int64_t stride = (int64_t)gridDim.x * kReadThreads;
  int64_t i = (int64_t)blockIdx.x * kReadThreads + threadIdx.x;
  i32x4 acc = {0, 0, 0, 0};
  for (; i + 3 * stride < n16; i += 4 * stride) acc ^= buf[i] ^ buf[i + stride] ^ buf[i + 2 * stride] ^ buf[i + 3 * stride];
  for (; i < n16; i += stride) acc ^= buf[i];
  if (acc[0] == 0x13572468 && acc[1] == 0x2468ace0 && acc[2] == 0x0f1e2d3c) sink[0] = (uint32_t)acc[3];
}

__global__ __launch_bounds__(kReadThreads) void mla_read_lds_kernel(const unsigned char* __restrict__ buf,
                                                                     int64_t bytes, uint32_t* __restrict__ sink) {
  __shared__ __attribute__((aligned(1024))) unsigned char tiles[kReadChunk];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t base = (int64_t)blockIdx.x * kReadChunk;
  const int blocks = (int)min((int64_t)kReadChunk, bytes - base) / 1024;  // bytes is a multiple of 1 KiB
  const unsigned char* src = buf + base;
  const uint32_t lds = lds_addr(tiles);
  for (int k = wave; k < blocks; k += kReadThreads / 64) {
    const uint32_t dst = __builtin_amdgcn_readfirstlane(lds + k * 1024);
    const int off = k * 1024 + lane * 16;
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
                 :: "s"(dst), "v"(off), "s"(src) : "memory", "m0");
  }
  wait_vmcnt<0>();
  __syncthreads();
  const uint32_t x = *(volatile uint32_t*)(tiles + threadIdx.x * 4);
  if (x == 0x13572468u && blockIdx.x == 0x7fffffff) sink[0] = x;
}

__global__ void mla_empty_kernel() {}

hipError_t launch_read_reference(const void* buf, int64_t bytes, int mode, uint32_t* sink, hipStream_t stream) {
  if (mode == 0) {
    const int64_t n16 = bytes / 16;
    hipLaunchKernelGGL(mla_read_plain_kernel, dim3(4096), dim3(kReadThreads), 0, stream, (const i32x4*)buf, n16,
                       sink);
  } else if (mode == 1) {
    const int64_t grid = (bytes + kReadChunk - 1) / kReadChunk;
    if (grid > 0)
      hipLaunchKernelGGL(mla_read_lds_kernel, dim3((unsigned)grid), dim3(kReadThreads), 0, stream,
                         (const unsigned char*)buf, bytes, sink);
  } else {
    hipLaunchKernelGGL(mla_empty_kernel, dim3(1), dim3(64), 0, stream);
  }
  return hipGetLastError();
}

// ------------------------------------------------------------------- kernels

constexpr int kPartialThreads = 512;
static_assert(KSplitCfg<false, 1>::NW * 64 == kPartialThreads, "workgroup size");

// Eight waves, two per SIMD; the page tiles cap residency at one workgroup per compute
// unit, so each wave may hold up to 256 registers.
// The leading arguments (up to the parameter block) are the ones preloaded into SGPRs.
template <bool FP8, int RBW, bool F8QK, bool HID, bool NT, bool ST>
__global__ __launch_bounds__(kPartialThreads)
__attribute__((amdgpu_waves_per_eu(2, 2))) void mla_partial_kernel(
    const int32_t* __restrict__ block_table, const uint8_t* __restrict__ pool, const uint16_t* __restrict__ q_ptr,
    int32_t nwg, uint32_t unit_pack, int32_t total32, int32_t len0, int32_t maxp, uint32_t shape_pack,
    uint32_t npages, PartialParams p, const int32_t* __restrict__ seq_lens, float* __restrict__ part_o,
    float* __restrict__ part_lse) {
  __shared__ KSplitSmem<FP8, RBW> sm;
  MLA_TL(0);
  const HotArgs args(p, nwg, unit_pack, total32, len0, maxp, shape_pack, npages);
  partial_ks<FP8, RBW, RBW == 2, F8QK, HID, NT, ST>(p, args, q_ptr, pool, block_table, seq_lens, part_o, part_lse,
                                                   sm);
}

// ------------------------------------------------------------------ launchers

namespace {

template <bool FP8, int RBW, bool F8QK, bool HID, bool NT, bool ST>
void launch_partial_k(const PartialParams& p, hipStream_t stream) {
  const int32_t total32 = p.plan.n > 0 ? (int32_t)p.total_pages : 0;  // the plan path has P < 2^31
  const uint32_t unit_pack = (uint32_t)p.row_groups | (uint32_t)(p.mode & 1) << 16 | (uint32_t)p.plan.n << 17;
  const uint32_t shape_pack = (uint32_t)p.num_heads | (uint32_t)p.q_len << 16 | (uint32_t)(p.causal & 1) << 24 |
                              (uint32_t)(p.stream_pages & 1) << 25;
  const uint32_t npages = p.num_pages > (int64_t)UINT32_MAX ? UINT32_MAX : (uint32_t)p.num_pages;
  hipLaunchKernelGGL((mla_partial_kernel<FP8, RBW, F8QK, HID, NT, ST>), dim3(partial_grid(p.num_wg, p.row_groups)),
                     dim3(kPartialThreads), 0, stream, p.block_table, p.pool, p.q, p.num_wg, unit_pack, total32,
                     p.plan.len[0], p.max_pages, shape_pack, npages, p, p.seq_lens, p.part_o, p.part_lse);
}

template <bool FP8, int RBW, bool F8QK = false>
hipError_t launch_partial_t(const PartialParams& p, hipStream_t stream) {
  // the packed leading arguments' fields (kMaxRowBlocks keeps q_len <= 64 and heads <= 1024)
  if (p.num_heads > 0xFFFF || p.q_len > 0xFF || p.row_groups > 0xFFFF || p.plan.n > 0x7FFF)
    return hipErrorInvalidValue;
  // hidden tails get kernels of their own (the per-piece table read costs the plain
  // kernels a few percent when compiled in); non-temporal part stores as the plan says
  const bool nt = p.nt_parts && !p.hidden;
  // two row blocks in one row group over a large history: page copies with the
  // non-temporal hint (spec_verify at two tokens 212 -> 189 us a layer-step; with several
  // row groups the hint cost 3%: their pages are shared through L2)
  if constexpr (RBW == 2) {
    if (p.row_groups == 1 && p.stream_pages) {
      if (p.hidden) launch_partial_k<FP8, RBW, F8QK, true, false, true>(p, stream);
      else if (nt) launch_partial_k<FP8, RBW, F8QK, false, true, true>(p, stream);
      else launch_partial_k<FP8, RBW, F8QK, false, false, true>(p, stream);
      return hipGetLastError();
    }
  }
  if (p.hidden) launch_partial_k<FP8, RBW, F8QK, true, false, false>(p, stream);
  else if (nt) launch_partial_k<FP8, RBW, F8QK, false, true, false>(p, stream);
  else launch_partial_k<FP8, RBW, F8QK, false, false, false>(p, stream);
  return hipGetLastError();
}

}  // namespace

// LDS bytes of one partial-stage workgroup, for the planner's residency estimate.
size_t partial_lds_size(bool fp8, int rbw) {
  if (rbw == 1) return fp8 ? sizeof(KSplitSmem<true, 1>) : sizeof(KSplitSmem<false, 1>);
  if (rbw == 2) return fp8 ? sizeof(KSplitSmem<true, 2>) : sizeof(KSplitSmem<false, 2>);
  return 0;
}

hipError_t launch_partial(const PartialParams& p, bool fp8, bool fp8_qk, hipStream_t stream) {
  const int rbs = p.q_len * p.head_groups;
  if (p.row_groups < 1 || p.rbw * p.row_groups < rbs || p.rbw * (p.row_groups - 1) >= rbs)
    return hipErrorInvalidValue;
  if (fp8_qk) {  // only the FP8 row split has the FP8 QK^T form
    if (!fp8 || p.rbw != 2) return hipErrorInvalidValue;
    return launch_partial_t<true, 2, true>(p, stream);
  }
  if (p.rbw == 1) return fp8 ? launch_partial_t<true, 1>(p, stream) : launch_partial_t<false, 1>(p, stream);
  if (p.rbw == 2) return fp8 ? launch_partial_t<true, 2>(p, stream) : launch_partial_t<false, 2>(p, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_kv_append(void* pool, int64_t num_pages, bool fp8, const int32_t* block_table,
                            int32_t max_pages, const int32_t* seq_lens, const void* latents,
                            int32_t rows, int32_t q_len, float kv_scale, hipStream_t stream) {
  if (fp8)
    hipLaunchKernelGGL((mla_kv_append_kernel<true>), dim3(rows), dim3(kAppendThreads), 0, stream,
                       (uint8_t*)pool, num_pages, block_table, max_pages, seq_lens,
                       (const uint16_t*)latents, q_len, kv_scale);
  else
    hipLaunchKernelGGL((mla_kv_append_kernel<false>), dim3(rows), dim3(kAppendThreads), 0, stream,
                       (uint8_t*)pool, num_pages, block_table, max_pages, seq_lens,
                       (const uint16_t*)latents, q_len, kv_scale);
  return hipGetLastError();
}

bool partial_nt_parts(int64_t part_bytes, int64_t kv_bytes) {
  return part_bytes >= kNtPartBytes && 8 * part_bytes >= kv_bytes;
}

// lds_reserve: unused dynamic LDS per workgroup (the residency experiment), 0 normally.
hipError_t launch_merge(const MergeParams& p, bool part_bf16, bool decode, int64_t total_rows,
                        int max_row_slots, uint32_t lds_reserve, hipStream_t stream) {
  const int sel = (part_bf16 ? 4 : 0) + (p.out_bf16 ? 2 : 0) + (decode ? 1 : 0);
  if (max_row_slots <= kRowSlots) {
    const dim3 grid((unsigned)(2 * total_rows));
    switch (sel) {
#define MLA_MERGE_CASE(S, A, B, D) \
      case S: hipLaunchKernelGGL((mla_merge_rows_kernel<A, B, D>), grid, dim3(kRowMergeThreads), lds_reserve, stream, \
                                 MLA_MERGE_LEAD_VALUES(p), p, total_rows); break;
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
  const dim3 grid((unsigned)(total_rows * kMergeChunks));
  switch (sel) {
#define MLA_MERGE_CASE(S, A, B, D) \
    case S: hipLaunchKernelGGL((mla_merge_kernel<A, B, D>), grid, dim3(kMergeThreads), lds_reserve, stream, \
                               MLA_MERGE_LEAD_VALUES(p), p); break;
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

#ifdef MLA_TIMELINE
// The stamps of the last decode, host copies: partial [4096][8], merge [16384][4] (uint64,
// zero where a workgroup did not stamp).  0 on success.
extern "C" int mla_timeline_read(unsigned long long* partial, unsigned long long* merge) {
  if (hipMemcpyFromSymbol(partial, HIP_SYMBOL(mla::g_tl_partial), sizeof(mla::g_tl_partial)) != hipSuccess)
    return 1;
  if (hipMemcpyFromSymbol(merge, HIP_SYMBOL(mla::g_tl_merge), sizeof(mla::g_tl_merge)) != hipSuccess) return 2;
  return 0;
}
extern "C" int mla_timeline_clear(void) {
  static const unsigned long long zeros[mla::kTlMergeBlocks * mla::kTlMergeSlots] = {};
  static_assert(sizeof(zeros) >= sizeof(mla::g_tl_partial), "clear source");
  if (hipMemcpyToSymbol(HIP_SYMBOL(mla::g_tl_partial), zeros, sizeof(mla::g_tl_partial)) != hipSuccess) return 1;
  if (hipMemcpyToSymbol(HIP_SYMBOL(mla::g_tl_merge), zeros, sizeof(mla::g_tl_merge)) != hipSuccess) return 2;
  return 0;
}
#endif
