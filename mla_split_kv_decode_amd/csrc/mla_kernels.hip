// gfx950 kernels of absorbed-MLA split-KV decode.
//
// Stage 1, mla_partial_kernel: one workgroup per piece list (see mla_internal.h).  For
// each piece (request, page range) it streams the latent pages through LDS and computes,
// for every query row of the request, the softmax-attention partial answer over the
// piece: O_p (normalised, fp32) and LSE_p.  Kimi K3 on MI355X, section 4 "MLA": the
// history is split into partitions handled by separate workgroups; section 1 "Cache",
// DCP8 paragraph: a partial answer carries its normalisation so pieces can be merged.
//
// Stage 2, mla_merge_kernel: the LSE-weighted merge of the partial answers of each row.
//
// Matrix layout (all on the 16x16 MFMA grid, wave64):
//  * rows   : 16 query rows = 16 heads of one query token ("row block"); heads past the
//             real count are zero rows (section 4: padding heads leaves real heads
//             unchanged) that are never loaded or written.
//  * QK^T   : S^T[pos][row] = sum_k K[pos][k] Q[row][k] with v_mfma_f32_16x16x32_bf16,
//             A = 16 positions x 32 latent columns read from LDS row-major, B = the row
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

#include <atomic>

#include "mla_internal.h"

namespace mla {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

constexpr float kLn2 = 0.69314718055994531f;
constexpr float kNegInf = -__builtin_inff();

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_fast(float x) { return __builtin_amdgcn_logf(x); }

// Eight FP8 E4M3FN codes (little-endian bytes of `raw`) -> eight bf16, exactly.
__device__ __forceinline__ bf16x8 fp8x8_to_bf16x8(i32x2 raw) {
  bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw[0], 1.0f, false);
  bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw[0], 1.0f, true);
  bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw[1], 1.0f, false);
  bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw[1], 1.0f, true);
  return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

__device__ __forceinline__ const lds_bf16x4* as_lds_bf16x4(const unsigned char* p) {
  return (const lds_bf16x4*)(p);
}
__device__ __forceinline__ const lds_i32x2* as_lds_i32x2(const unsigned char* p) {
  return (const lds_i32x2*)(p);
}

template <bool FP8>
struct TileGeom {
  static constexpr int kElem = FP8 ? 1 : 2;
  static constexpr int kRowBytes = kDLatent * kElem;          // one latent in HBM
  static constexpr int kStride = kRowBytes + 16;              // LDS row pitch (bank skew)
  static constexpr int kPageBytes = kPage * kRowBytes;        // one page in HBM
  static constexpr int kChunks = kPageBytes / 16;             // 16-byte pieces per page
  static constexpr int kChunksPerRow = kRowBytes / 16;
  static constexpr int kLdsTile = kPage * kStride;
};

// Dynamic LDS of one workgroup: two page tiles, the P^T exchange and the row
// reductions.
template <bool FP8>
__host__ __device__ constexpr int partial_lds_bytes(int row_blocks, int G) {
  return 2 * TileGeom<FP8>::kLdsTile + (G > 1 ? row_blocks * 2 * 64 * 16 : 0) +
         row_blocks * G * 16 * 4;
}

template <bool FP8, int G, int MINW, int MAXW>
__global__ __launch_bounds__(MAXW * 64) void mla_partial_kernel(PartialParams p) {
  using TG = TileGeom<FP8>;
  constexpr int kMaxC = (TG::kChunks + 64 * MINW - 1) / (64 * MINW);
  constexpr int NST = 4 / G;   // 16-position sub-tiles of a page per wave
  constexpr int CT = 32 / G;   // 16-column output tiles per wave
  constexpr int kColsPerWave = kDV / G;

  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int tid = threadIdx.x;
  const int nthreads = blockDim.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int lrow = lane & 15, lgrp = lane >> 4;
  const int rb = wave / G, g = wave - (wave / G) * G;
  const int RB = p.q_len * p.head_groups;
  const int t = rb / p.head_groups, hg = rb - t * p.head_groups;
  const int head = hg * kRowsPerBlock + lrow;
  const bool head_ok = head < p.num_heads;

  unsigned char* const tiles = smem;
  unsigned char* const pbuf = smem + 2 * TG::kLdsTile;
  float* const red = (float*)(pbuf + (G > 1 ? RB * 2 * 64 * 16 : 0));

  // One piece: request r, local pages [pb, pe), partial slot `slot`.
  auto run_piece = [&](int r, int pb, int pe, int64_t slot) {
    const int L = max(p.seq_lens[r], 0);
    const int limit = p.causal ? L - p.q_len + t + 1 : L;  // visible: position < limit
    const int32_t* trow = p.block_table + (int64_t)r * p.max_pages;

    bf16x8 qf[kDLatent / 32];
    {
      const uint16_t* qrow =
          p.q + (((int64_t)r * p.q_len + t) * p.num_heads + head) * kDLatent + lgrp * 8;
#pragma unroll
      for (int kk = 0; kk < kDLatent / 32; ++kk) {
        qf[kk] = head_ok ? *(const bf16x8*)(qrow + kk * 32) : bf16x8{};
      }
    }

    float m = kNegInf;   // running max of this lane's row (log2 units)
    float lsum = 0.f;    // this lane's share of the running denominator
    f32x4 acc[CT];
#pragma unroll
    for (int i = 0; i < CT; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    bool bad = false;

    i32x4 stage[kMaxC];
    auto load_page = [&](int lp) {
      int32_t id = trow[lp];
      int valid_rows = min(kPage, L - lp * kPage);
      if ((uint64_t)(int64_t)id >= (uint64_t)p.num_pages) {  // never dereferenced
        bad = true;
        valid_rows = 0;
        id = 0;
      }
      const unsigned char* src = p.pool + (int64_t)id * TG::kPageBytes;
#pragma unroll
      for (int k = 0; k < kMaxC; ++k) {
        const int c = tid + k * nthreads;
        i32x4 v = i32x4{0, 0, 0, 0};
        if (c < TG::kChunks && c / TG::kChunksPerRow < valid_rows) {
          v = *(const i32x4*)(src + (int64_t)c * 16);
        }
        stage[k] = v;
      }
    };
    auto store_page = [&](unsigned char* tile) {
#pragma unroll
      for (int k = 0; k < kMaxC; ++k) {
        const int c = tid + k * nthreads;
        if (c < TG::kChunks) {
          const int row = c / TG::kChunksPerRow, col = c - row * TG::kChunksPerRow;
          *(i32x4*)(tile + row * TG::kStride + col * 16) = stage[k];
        }
      }
    };

    const int npages = pe - pb;
    if (npages > 0) {
      load_page(pb);
      store_page(tiles);
    }
    __syncthreads();

    for (int i = 0; i < npages; ++i) {
      const unsigned char* tile = tiles + (i & 1) * TG::kLdsTile;
      if (i + 1 < npages) load_page(pb + i + 1);

      // ---- S^T = K Q^T for this wave's sub-tiles
      f32x4 s[NST];
#pragma unroll
      for (int u = 0; u < NST; ++u) {
        const int pt = g * NST + u;
        const unsigned char* krow = tile + (pt * 16 + lrow) * TG::kStride + lgrp * 8 * TG::kElem;
        f32x4 a = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < kDLatent / 32; ++kk) {
          bf16x8 kf;
          if constexpr (FP8) {
            kf = fp8x8_to_bf16x8(*(const i32x2*)(krow + kk * 32));
          } else {
            kf = *(const bf16x8*)(krow + kk * 64);
          }
          a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[kk], a, 0, 0, 0);
        }
        s[u] = a;
      }

      // ---- scale, mask, tile max
      const int pos0 = (pb + i) * kPage;
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
        __syncthreads();
#pragma unroll
        for (int gg = 0; gg < G; ++gg) mx = fmaxf(mx, red[(rb * G + gg) * 16 + lrow]);
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
        __syncthreads();
#pragma unroll
        for (int c = 0; c < 2; ++c) pf[c] = *(const bf16x8*)(pbuf + ((rb * 2 + c) * 64 + lane) * 16);
      }

      // ---- O^T += V^T P^T over the page's two 32-position chunks
#pragma unroll
      for (int c = 0; c < 2; ++c) {
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          const int col0 = g * kColsPerWave + ct * 16;
          bf16x8 va;
          if constexpr (FP8) {
            const int h = lrow & 1, ii = lrow >> 1;
            const int row = 32 * c + (ii < 4 ? 4 * lgrp + ii : 16 + 4 * lgrp + ii - 4);
            const i32x2 raw = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                (lds_i32x2*)as_lds_i32x2(tile + row * TG::kStride + col0 + 8 * h));
            va = fp8x8_to_bf16x8(raw);
          } else {
            const int row = 32 * c + 4 * lgrp + (lrow >> 2);
            const unsigned char* a0 = tile + row * TG::kStride + (col0 + 4 * (lrow & 3)) * 2;
            const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)as_lds_bf16x4(a0));
            const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                (lds_bf16x4*)as_lds_bf16x4(a0 + 16 * TG::kStride));
            va = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          }
          acc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pf[c], acc[ct], 0, 0, 0);
        }
      }

      if (i + 1 < npages) store_page(tiles + ((i + 1) & 1) * TG::kLdsTile);
      __syncthreads();
    }

    // ---- epilogue: full row denominator, normalise, store the partial answer
    float ls = lsum;
    ls += __shfl_xor(ls, 16);
    ls += __shfl_xor(ls, 32);
    if constexpr (G > 1) {
      if (lgrp == 0) red[(rb * G + g) * 16 + lrow] = ls;
      __syncthreads();
      ls = 0.f;
#pragma unroll
      for (int gg = 0; gg < G; ++gg) ls += red[(rb * G + gg) * 16 + lrow];
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
      float* dst = p.part_o + (slot * p.rows + orow) * kDV + g * kColsPerWave + lgrp * 4;
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) *(f32x4*)(dst + ct * 16) = acc[ct] * oscale;
      if (g == 0 && lgrp == 0) p.part_lse[slot * p.rows + orow] = lse;
    }
    __syncthreads();  // LDS (tiles, exchange buffers) is reused by the next piece
  };

  const int64_t w = blockIdx.x;
  if (p.mode == SPLIT_FIXED) {
    const int S = p.num_splits;
    const int r = (int)(w / S), s = (int)(w - (int64_t)r * S);
    const int pages = pages_of(p.seq_lens[r], p.max_pages);
    run_piece(r, fixed_page_begin(s, pages, S), fixed_page_begin(s + 1, pages, S), w);
  } else {
    int64_t P = 0;
    for (int r = 0; r < p.batch; ++r) P += pages_of(p.seq_lens[r], p.max_pages);
    if (P == 0) return;
    const int64_t gb = balanced_start(w, P, p.num_wg), ge = balanced_start(w + 1, P, p.num_wg);
    int64_t pre = 0;
    for (int r = 0; r < p.batch && pre < ge; ++r) {
      const int pr = pages_of(p.seq_lens[r], p.max_pages);
      const int64_t lo = gb > pre ? gb : pre;
      const int64_t hi = ge < pre + pr ? ge : pre + pr;
      if (lo < hi) run_piece(r, (int)(lo - pre), (int)(hi - pre), w + r);
      pre += pr;
    }
  }
}

// ------------------------------------------------------------------- merge

constexpr int kMergeCols = 32;                // output columns per workgroup
constexpr int kMergeThreads = 256;            // 8 column quads x 32 part lanes
constexpr int kMergeLanes = kMergeThreads / (kMergeCols / 4);

template <bool PART_BF16, bool OUT_BF16>
__global__ __launch_bounds__(kMergeThreads) void mla_merge_kernel(MergeParams p) {
  __shared__ float red_f[kMergeThreads];
  __shared__ f32x4 red_v[kMergeThreads];
  const int tid = threadIdx.x;
  const int pl = tid >> 3, cq = tid & 7;  // part lane, column quad
  const int64_t bx = blockIdx.x;
  const int64_t orow = bx / (kDV / kMergeCols);
  const int cchunk = (int)(bx - orow * (kDV / kMergeCols));
  const int64_t grp = orow / p.rows;
  const int64_t row = orow - grp * p.rows;

  // slot range [s0, s1); validity of a slot for this group
  int64_t s0 = 0, s1 = 0, P = 0, pre = 0, pr = 0;
  bool balanced = false;
  if (p.mode == MERGE_GENERIC) {
    s1 = p.num_parts;
  } else if (p.split_mode == SPLIT_FIXED) {
    s0 = grp * p.num_splits;
    s1 = s0 + p.num_splits;
  } else {
    balanced = true;
    for (int r = 0; r < p.batch; ++r) {
      const int pg = pages_of(p.seq_lens[r], p.max_pages);
      if (r < grp) pre += pg;
      if (r == grp) pr = pg;
      P += pg;
    }
    if (pr > 0) {
      s0 = balanced_wg_of(pre, P, p.num_wg) + grp;
      s1 = balanced_wg_of(pre + pr - 1, P, p.num_wg) + grp + 1;
    }
  }
  auto slot_ok = [&](int64_t s) -> bool {
    if (!balanced) return true;
    const int64_t w = s - grp;
    const int64_t st = balanced_start(w, P, p.num_wg), en = balanced_start(w + 1, P, p.num_wg);
    return st < en && st < pre + pr && en > pre;
  };
  auto lse_at = [&](int64_t s) -> float { return p.part_lse[s * p.part_rows + row]; };

  // pass 1: M = max LSE.  A NaN LSE (a piece that met a bad page id) must reach the
  // output, so this max propagates NaN instead of dropping it as fmaxf would.
  auto nan_max = [](float a, float b) { return a != a ? a : (b != b ? b : fmaxf(a, b)); };
  float mx = kNegInf;
  for (int64_t s = s0 + tid; s < s1; s += kMergeThreads)
    if (slot_ok(s)) mx = nan_max(mx, lse_at(s));
  red_f[tid] = mx;
  __syncthreads();
  for (int off = kMergeThreads / 2; off > 0; off >>= 1) {
    if (tid < off) red_f[tid] = nan_max(red_f[tid], red_f[tid + off]);
    __syncthreads();
  }
  const float M = red_f[0];
  __syncthreads();

  // pass 2: weighted sum
  constexpr float kLog2e = 1.44269504088896341f;
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  float asum = 0.f;
  if (M != kNegInf) {
    for (int64_t s = s0 + pl; s < s1; s += kMergeLanes) {
      if (!slot_ok(s)) continue;
      const float a = exp2_fast((lse_at(s) - M) * kLog2e);
      const int64_t off = (s * p.part_rows + row) * kDV + cchunk * kMergeCols + cq * 4;
      f32x4 o;
      if constexpr (PART_BF16) {
        const bf16x4 b = *(const bf16x4*)((const __bf16*)p.part_o + off);
        o = f32x4{(float)b[0], (float)b[1], (float)b[2], (float)b[3]};
      } else {
        o = *(const f32x4*)((const float*)p.part_o + off);
      }
      acc += a * o;
      asum += a;
    }
  }
  red_v[tid] = acc;
  red_f[tid] = asum;
  __syncthreads();
  for (int off = kMergeLanes / 2; off > 0; off >>= 1) {
    if (pl < off) {
      red_v[tid] += red_v[tid + off * 8];
      red_f[tid] += red_f[tid + off * 8];
    }
    __syncthreads();
  }
  if (pl == 0) {
    const bool empty = M == kNegInf;
    const float den = red_f[cq];
    const f32x4 o = empty ? f32x4{0.f, 0.f, 0.f, 0.f} : red_v[cq] * (1.0f / den);
    if (p.out) {
      const int64_t off = orow * kDV + cchunk * kMergeCols + cq * 4;
      if constexpr (OUT_BF16) {
        *(bf16x4*)((__bf16*)p.out + off) = bf16x4{(__bf16)o[0], (__bf16)o[1], (__bf16)o[2], (__bf16)o[3]};
      } else {
        *(f32x4*)((float*)p.out + off) = o;
      }
    }
    if (p.out_lse && cchunk == 0 && cq == 0) {
      p.out_lse[orow] = empty ? kNegInf : M + log2_fast(den) * kLn2;
    }
  }
}

// ------------------------------------------------------------------ launchers

namespace {

template <typename K>
hipError_t set_lds_limit(K kernel, int bytes) {
  return hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
}

constexpr int kMaxLds = 160 * 1024;  // LDS of one gfx950 compute unit

template <bool FP8, int G, int MINW, int MAXW>
hipError_t launch_partial_t(const PartialParams& p, int row_blocks, hipStream_t stream) {
  auto kernel = mla_partial_kernel<FP8, G, MINW, MAXW>;
  const int lds = partial_lds_bytes<FP8>(row_blocks, G);
  // Dynamic LDS beyond the default limit must be allowed per function and device.
  static std::atomic<uint64_t> configured{0};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = dev < 64 ? (1ull << dev) : 0;
  if (!bit || !(configured.load() & bit)) {
    e = set_lds_limit(kernel, kMaxLds);
    if (e != hipSuccess) return e;
    configured.fetch_or(bit);
  }
  const int threads = row_blocks * G * 64;
  hipLaunchKernelGGL(kernel, dim3(p.num_wg), dim3(threads), lds, stream, p);
  return hipGetLastError();
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
  return fp8 ? partial_lds_bytes<true>(row_blocks, G) : partial_lds_bytes<false>(row_blocks, G);
}

hipError_t launch_partial(const PartialParams& p, bool fp8, hipStream_t stream) {
  const int RB = p.q_len * p.head_groups;
  const int G = partial_waves_per_row_block(RB);
  const int nw = RB * G;
  if (fp8) {
    if (G == 4) return launch_partial_t<true, 4, 4, 4>(p, RB, stream);
    if (G == 2) return nw == 4 ? launch_partial_t<true, 2, 4, 4>(p, RB, stream)
                               : launch_partial_t<true, 2, 5, 8>(p, RB, stream);
    return nw == 4 ? launch_partial_t<true, 1, 4, 4>(p, RB, stream)
                   : launch_partial_t<true, 1, 5, 8>(p, RB, stream);
  }
  if (G == 4) return launch_partial_t<false, 4, 4, 4>(p, RB, stream);
  if (G == 2) return nw == 4 ? launch_partial_t<false, 2, 4, 4>(p, RB, stream)
                             : launch_partial_t<false, 2, 5, 8>(p, RB, stream);
  return nw == 4 ? launch_partial_t<false, 1, 4, 4>(p, RB, stream)
                 : launch_partial_t<false, 1, 5, 8>(p, RB, stream);
}

hipError_t launch_merge(const MergeParams& p, int64_t total_rows, hipStream_t stream) {
  const dim3 grid((unsigned)(total_rows * (kDV / kMergeCols)));
  if (p.part_bf16) {
    if (p.out_bf16) hipLaunchKernelGGL((mla_merge_kernel<true, true>), grid, dim3(kMergeThreads), 0, stream, p);
    else hipLaunchKernelGGL((mla_merge_kernel<true, false>), grid, dim3(kMergeThreads), 0, stream, p);
  } else {
    if (p.out_bf16) hipLaunchKernelGGL((mla_merge_kernel<false, true>), grid, dim3(kMergeThreads), 0, stream, p);
    else hipLaunchKernelGGL((mla_merge_kernel<false, false>), grid, dim3(kMergeThreads), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace mla
