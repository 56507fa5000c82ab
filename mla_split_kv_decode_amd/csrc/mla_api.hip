// Host side of the C ABI declared in include/mla_decode.h: argument checks, the
// split-KV partition planner, workspace layout and kernel launches.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "mla_decode.h"
#include "mla_internal.h"

namespace mla {
hipError_t launch_partial(const PartialParams& p, bool fp8, bool fp8_qk, hipStream_t stream);
bool partial_nt_parts(int64_t part_bytes, int64_t kv_bytes);
hipError_t launch_merge(const MergeParams& p, bool part_bf16, bool decode, int64_t total_rows,
                        int max_row_slots, uint32_t lds_reserve, hipStream_t stream);
constexpr long long kMaxLdsReserve = 128 * 1024;
size_t partial_lds_size(bool fp8, int rbw);
hipError_t launch_read_reference(const void* buf, int64_t bytes, int mode, uint32_t* sink, hipStream_t stream);
hipError_t launch_kv_append(void* pool, int64_t num_pages, bool fp8, const int32_t* block_table,
                            int32_t max_pages, const int32_t* seq_lens, const void* latents,
                            int32_t rows, int32_t q_len, float kv_scale, hipStream_t stream);
}  // namespace mla

using namespace mla;

struct mla_plan {
  mla_decode_shape shape;
  int32_t kv_dtype;
  int32_t page_size;
  int32_t num_cus;
  int32_t head_groups;
  int32_t row_blocks;
  int32_t rbw;           // row blocks per workgroup
  int32_t row_groups;    // workgroups per unit
  int32_t rows;          // q_len * num_heads, real rows
  int32_t mode;          // SplitMode
  int32_t num_wg;        // work units of the partial stage
  int32_t num_splits;    // S (SPLIT_FIXED)
  int32_t num_slots;     // partial answers the workspace holds
  int32_t fp8_qk;        // QK^T on the FP8 matrix cores (mla_plan_set_fp8_qk)
  int64_t total_pages;
  int32_t max_req_pages;  // largest ceil(seq_len / page) of a request
  int32_t max_req_slots;  // most partial answers of one request
  size_t o_offset, o_bytes, lse_offset, workspace_bytes;
  uint32_t lds_reserve;   // unused LDS per merge workgroup (residency experiment)
  std::vector<int32_t> seq_lens;  // host copy, for get_work only
};

namespace {

thread_local std::string g_last_error;

mla_status fail(mla_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

mla_status ok() {
  g_last_error.clear();
  return MLA_OK;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// The plan's lengths for the kernel arguments (only for batches that fit).
void fill_plan_args(const mla_plan& pl, PlanArgs* a) {
  memset(a, 0, sizeof(*a));
  const int32_t B = pl.shape.batch;
  if (B > kArgBatch || pl.total_pages > INT32_MAX) return;
  a->n = B;
  int32_t pre = 0;
  for (int32_t r = 0; r < B; ++r) {
    a->len[r] = pl.seq_lens[r];
    a->pre[r] = pre;
    pre += pages_of(pl.seq_lens[r], INT32_MAX);
  }
  a->pre[B] = pre;
}

// Workgroups per compute unit the partial stage can keep resident (LDS bound).
int wg_per_cu(bool fp8, int rbw) {
  const size_t lds = partial_lds_size(fp8, rbw);
  const size_t cu_lds = 160 * 1024;
  int n = (int)(cu_lds / ((lds + 1279) / 1280 * 1280));
  return n < 1 ? 1 : (n > 2 ? 2 : n);
}

mla_status decode_impl(const mla_plan* plan, const void* q, const mla_paged_kv* kv, void* workspace,
                       size_t workspace_bytes, void* out, int32_t out_dtype, float* out_lse,
                       const int32_t* hidden, void* stream);

// Scratch of the entry point that allocates nothing (mla_decode_splitkv_noalloc): the
// partial answers between the two stages live in a file-scope device array, one copy per
// GPU, held until the process ends.  Host code never takes the array's name as an
// address (on the host it only stands for the symbol): each device's address comes from
// hipGetSymbolAddress, looked up once per device on the first call made with that device
// current, and that address is what the kernels receive.
constexpr size_t kScratchBytes = MLA_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` on device d, null until looked up

}  // namespace

static __device__ __align__(256) unsigned char scratch[MLA_NOALLOC_SCRATCH_BYTES];

namespace {

mla_status scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MLA_ERR_DEVICE, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(MLA_ERR_UNSUPPORTED, "device %d (at most %d)", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(MLA_ERR_DEVICE, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    if (!aligned(p, 256)) return fail(MLA_ERR_DEVICE, "scratch on device %d is not 256-byte aligned", dev);
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MLA_OK;
}

}  // namespace

extern "C" {

const char* mla_version(void) { return "mla_split_kv_decode_amd 0.7.8 (gfx950)"; }

const char* mla_last_error(void) { return g_last_error.c_str(); }

const char* mla_status_str(mla_status s) {
  switch (s) {
    case MLA_OK: return "ok";
    case MLA_ERR_INVALID_ARGUMENT: return "invalid argument";
    case MLA_ERR_UNSUPPORTED: return "unsupported";
    case MLA_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case MLA_ERR_DEVICE: return "device error";
  }
  return "unknown status";
}

size_t mla_page_bytes(int32_t page_size, int32_t kv_dtype) {
  if (page_size <= 0) return 0;
  if (kv_dtype == MLA_BF16) return (size_t)page_size * kDLatent * 2;
  if (kv_dtype == MLA_FP8_E4M3FN) return (size_t)page_size * kDLatent;
  return 0;
}

mla_status mla_block_table_check(const int32_t* table, int32_t batch, int32_t max_pages,
                                 const int32_t* seq_lens, int32_t page_size, int64_t num_pages) {
  if (!table || !seq_lens) return fail(MLA_ERR_INVALID_ARGUMENT, "null pointer");
  if (batch < 1 || max_pages < 1 || page_size < 1 || num_pages < 1)
    return fail(MLA_ERR_INVALID_ARGUMENT, "batch, max_pages_per_seq, page_size, num_pages must be >= 1");
  for (int32_t r = 0; r < batch; ++r) {
    if (seq_lens[r] < 0) return fail(MLA_ERR_INVALID_ARGUMENT, "seq_lens[%d] = %d < 0", r, seq_lens[r]);
    const int64_t pages = ((int64_t)seq_lens[r] + page_size - 1) / page_size;
    if (pages > max_pages)
      return fail(MLA_ERR_INVALID_ARGUMENT, "request %d needs %lld pages > max_pages_per_seq %d", r,
                  (long long)pages, max_pages);
    for (int64_t k = 0; k < pages; ++k) {
      const int32_t id = table[(int64_t)r * max_pages + k];
      if (id < 0 || id >= num_pages)
        return fail(MLA_ERR_INVALID_ARGUMENT, "block_table[%d][%lld] = %d outside [0, %lld)", r,
                    (long long)k, id, (long long)num_pages);
    }
  }
  return ok();
}

mla_status mla_plan_create(const mla_decode_shape* shape, const int32_t* seq_lens_host,
                           int32_t page_size, int32_t kv_dtype, int32_t num_cus, mla_plan** plan_out,
                           size_t* workspace_bytes) {
  if (!shape || !seq_lens_host || !plan_out) return fail(MLA_ERR_INVALID_ARGUMENT, "null pointer");
  *plan_out = nullptr;
  const mla_decode_shape s = *shape;
  if (s.batch < 1 || s.q_len < 1 || s.num_heads < 1)
    return fail(MLA_ERR_INVALID_ARGUMENT, "batch, q_len, num_heads must be >= 1");
  if (!(s.softmax_scale > 0.f) || !std::isfinite(s.softmax_scale))
    return fail(MLA_ERR_INVALID_ARGUMENT, "softmax_scale must be finite and > 0");
  if (s.causal != 0 && s.causal != 1) return fail(MLA_ERR_INVALID_ARGUMENT, "causal must be 0 or 1");
  if (s.num_splits < 0) return fail(MLA_ERR_INVALID_ARGUMENT, "num_splits must be >= 0");
  if (page_size != kPage) return fail(MLA_ERR_UNSUPPORTED, "page_size %d (only %d)", page_size, kPage);
  if (kv_dtype != MLA_BF16 && kv_dtype != MLA_FP8_E4M3FN)
    return fail(MLA_ERR_UNSUPPORTED, "kv_dtype %d", kv_dtype);
  const int64_t head_groups = ((int64_t)s.num_heads + kRowsPerBlock - 1) / kRowsPerBlock;
  const int64_t row_blocks = head_groups * s.q_len;
  if (row_blocks > kMaxRowBlocks)
    return fail(MLA_ERR_UNSUPPORTED, "q_len * ceil(num_heads/16) = %lld > %d", (long long)row_blocks,
                kMaxRowBlocks);
  int64_t total_pages = 0;
  int32_t max_req_pages = 0;
  for (int32_t r = 0; r < s.batch; ++r) {
    // causal: the query tokens are the last q_len positions; otherwise (a context shard
    // of a longer history) any non-empty history
    const int32_t min_len = s.causal ? s.q_len : 1;
    if (seq_lens_host[r] < min_len)
      return fail(MLA_ERR_INVALID_ARGUMENT, "seq_lens[%d] = %d < %d", r, seq_lens_host[r], min_len);
    const int32_t pg = pages_of(seq_lens_host[r], INT32_MAX);
    total_pages += pg;
    if (pg > max_req_pages) max_req_pages = pg;
  }
  if (num_cus == 0) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&num_cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return fail(MLA_ERR_DEVICE, "cannot query the compute-unit count");
  }
  if (num_cus < 1) return fail(MLA_ERR_INVALID_ARGUMENT, "num_cus must be >= 1 (or 0 = query)");

  mla_plan* pl = new (std::nothrow) mla_plan();
  if (!pl) return fail(MLA_ERR_INVALID_ARGUMENT, "out of host memory");
  pl->shape = s;
  pl->kv_dtype = kv_dtype;
  pl->page_size = page_size;
  pl->num_cus = num_cus;
  pl->head_groups = (int32_t)head_groups;
  pl->row_blocks = (int32_t)row_blocks;
  // two row blocks per workgroup from two on (every V^T operand read from LDS then feeds
  // two MFMAs; an odd count gets one padding row block), else one
  pl->rbw = row_blocks >= 2 ? 2 : 1;
  pl->row_groups = (int32_t)((row_blocks + pl->rbw - 1) / pl->rbw);
  pl->rows = s.q_len * s.num_heads;
  pl->total_pages = total_pages;
  pl->max_req_pages = max_req_pages;
  pl->seq_lens.assign(seq_lens_host, seq_lens_host + s.batch);
  pl->lds_reserve = 0;
  if (const char* env = getenv("MLA_LDS_RESERVE")) {
    const long long v = strtoll(env, nullptr, 10);
    pl->lds_reserve = (uint32_t)(v < 0 ? 0 : v > kMaxLdsReserve ? kMaxLdsReserve : v);
  }
  const bool fp8 = kv_dtype == MLA_FP8_E4M3FN;
  int64_t wg, slots;
  if (s.num_splits > 0) {
    pl->mode = SPLIT_FIXED;
    pl->num_splits = s.num_splits;
    wg = (int64_t)s.batch * s.num_splits;
    slots = wg;
  } else {
    // Balanced: fill every compute unit (resident workgroups, row_groups per unit), never
    // more units than pages.
    pl->mode = SPLIT_BALANCED;
    pl->num_splits = 0;
    const int64_t slots_per_cu = (int64_t)num_cus * wg_per_cu(fp8, pl->rbw);
    const int64_t G = pl->row_groups;
    int64_t target;
    if (G == 1) {
      target = slots_per_cu;
    } else {
      // the kernel deals blocks to the eight XCDs by block index and keeps a unit's row
      // groups on one XCD: whole units per XCD, so that no XCD gets a second round
      const int64_t per_xcd = slots_per_cu / 8;
      target = per_xcd >= G ? 8 * (per_xcd / G) : slots_per_cu / G;
    }
    if (target < 1) target = 1;
    wg = total_pages < target ? total_pages : target;
    slots = wg + s.batch - 1;
  }
  if (wg > INT32_MAX / 2 || slots > INT32_MAX / 2 || partial_grid(wg, pl->row_groups) > INT32_MAX / 2) {
    delete pl;
    return fail(MLA_ERR_UNSUPPORTED, "too many workgroups");
  }
  pl->num_wg = (int32_t)wg;
  pl->num_slots = (int32_t)slots;
  if (pl->mode == SPLIT_FIXED) {
    pl->max_req_slots = pl->num_splits;
  } else {
    int64_t pre = 0, most = 0;
    for (int32_t r = 0; r < s.batch; ++r) {
      const int64_t pr = pages_of(seq_lens_host[r], INT32_MAX);
      const int64_t n = balanced_wg_of(pre + pr - 1, total_pages, wg) - balanced_wg_of(pre, total_pages, wg) + 1;
      if (n > most) most = n;
      pre += pr;
    }
    pl->max_req_slots = (int32_t)most;
  }
  // [fp32 partial O | fp32 partial LSE], each 256-byte aligned
  pl->o_offset = 0;
  pl->o_bytes = align256((size_t)slots * pl->rows * kDV * sizeof(float));
  pl->lse_offset = pl->o_offset + pl->o_bytes;
  pl->workspace_bytes = pl->lse_offset + align256((size_t)slots * pl->rows * sizeof(float));
  if (workspace_bytes) *workspace_bytes = pl->workspace_bytes;
  *plan_out = pl;
  return ok();
}

void mla_plan_destroy(mla_plan* plan) { delete plan; }

int32_t mla_plan_num_units(const mla_plan* plan) { return plan ? plan->num_wg : -1; }

int32_t mla_plan_num_parts(const mla_plan* plan) { return plan ? plan->num_slots : -1; }

int32_t mla_plan_row_groups(const mla_plan* plan) { return plan ? plan->row_groups : -1; }

mla_status mla_plan_set_fp8_qk(mla_plan* plan, int32_t enable) {
  if (!plan) return fail(MLA_ERR_INVALID_ARGUMENT, "null plan");
  if (enable != 0 && enable != 1) return fail(MLA_ERR_INVALID_ARGUMENT, "enable must be 0 or 1");
  if (enable && (plan->kv_dtype != MLA_FP8_E4M3FN || plan->rbw != 2))
    return fail(MLA_ERR_UNSUPPORTED,
                "FP8 QK^T needs an FP8 pool and q_len * ceil(num_heads/16) >= 2 (two row blocks per workgroup)");
  plan->fp8_qk = enable;
  return ok();
}

int32_t mla_plan_get_work(const mla_plan* plan, int32_t* out, int32_t capacity) {
  if (!plan || capacity < 0 || (capacity > 0 && !out)) return -1;
  int32_t n = 0;
  auto emit = [&](int32_t w, int32_t r, int32_t pb, int32_t pe, int32_t slot) {
    if (n < capacity) {
      int32_t* o = out + 5 * (int64_t)n;
      o[0] = w, o[1] = r, o[2] = pb, o[3] = pe, o[4] = slot;
    }
    ++n;
  };
  const int32_t B = plan->shape.batch;
  const int32_t maxp = INT32_MAX;
  if (plan->mode == SPLIT_FIXED) {
    const int32_t S = plan->num_splits;
    for (int32_t w = 0; w < plan->num_wg; ++w) {
      const int32_t r = w / S, sp = w % S;
      const int32_t pages = pages_of(plan->seq_lens[r], maxp);
      emit(w, r, fixed_page_begin(sp, pages, S), fixed_page_begin(sp + 1, pages, S), w);
    }
  } else {
    const int64_t P = plan->total_pages, W = plan->num_wg;
    for (int64_t w = 0; w < W; ++w) {
      const int64_t gb = balanced_start(w, P, W), ge = balanced_start(w + 1, P, W);
      int64_t pre = 0;
      for (int32_t r = 0; r < B && pre < ge; ++r) {
        const int32_t pr = pages_of(plan->seq_lens[r], maxp);
        const int64_t lo = gb > pre ? gb : pre, hi = ge < pre + pr ? ge : pre + pr;
        if (lo < hi) emit((int32_t)w, r, (int32_t)(lo - pre), (int32_t)(hi - pre), (int32_t)(w + r));
        pre += pr;
      }
    }
  }
  return n;
}

mla_status mla_decode_splitkv(const mla_plan* plan, const void* q, const mla_paged_kv* kv,
                              void* workspace, size_t workspace_bytes, void* out, int32_t out_dtype,
                              float* out_lse, const int32_t* hidden, void* stream) {
  return decode_impl(plan, q, kv, workspace, workspace_bytes, out, out_dtype, out_lse, hidden, stream);
}

mla_status mla_decode_splitkv_noalloc(const mla_plan* plan, const void* q, const mla_paged_kv* kv,
                                      void* out, int32_t out_dtype, float* out_lse, const int32_t* hidden,
                                      void* stream) {
  if (!plan) return fail(MLA_ERR_INVALID_ARGUMENT, "null pointer");
  if (!out && !out_lse)
    return fail(MLA_ERR_INVALID_ARGUMENT, "out and out_lse are both NULL: the scratch is not the caller's to read");
  if (plan->workspace_bytes > kScratchBytes)
    return fail(MLA_ERR_UNSUPPORTED, "the plan needs %zu bytes of partial answers; the no-allocation scratch holds %zu",
                plan->workspace_bytes, kScratchBytes);
  void* ws = nullptr;
  const mla_status st = scratch_of_current_device(&ws);
  if (st != MLA_OK) return st;
  return decode_impl(plan, q, kv, ws, kScratchBytes, out, out_dtype, out_lse, hidden, stream);
}

}  // extern "C"

namespace {

mla_status decode_impl(const mla_plan* plan, const void* q, const mla_paged_kv* kv, void* workspace,
                       size_t workspace_bytes, void* out, int32_t out_dtype, float* out_lse,
                       const int32_t* hidden, void* stream) {
  if (!plan || !q || !kv || !workspace) return fail(MLA_ERR_INVALID_ARGUMENT, "null pointer");
  if (!kv->pool || !kv->block_table || !kv->seq_lens)
    return fail(MLA_ERR_INVALID_ARGUMENT, "null pointer in the KV descriptor");
  if (kv->kv_dtype != plan->kv_dtype)
    return fail(MLA_ERR_INVALID_ARGUMENT, "kv_dtype %d differs from the plan's %d", kv->kv_dtype,
                plan->kv_dtype);
  if (kv->page_size != plan->page_size)
    return fail(MLA_ERR_INVALID_ARGUMENT, "page_size %d differs from the plan's", kv->page_size);
  if (kv->num_pages < 1 || kv->max_pages_per_seq < 1)
    return fail(MLA_ERR_INVALID_ARGUMENT, "num_pages and max_pages_per_seq must be >= 1");
  if (kv->max_pages_per_seq < plan->max_req_pages)
    return fail(MLA_ERR_INVALID_ARGUMENT,
                "max_pages_per_seq %d < %d pages a request of the plan needs", kv->max_pages_per_seq,
                plan->max_req_pages);
  const bool fp8 = kv->kv_dtype == MLA_FP8_E4M3FN;
  if (fp8) {
    if (!(kv->kv_scale > 0.f) || !std::isfinite(kv->kv_scale))
      return fail(MLA_ERR_INVALID_ARGUMENT, "kv_scale must be finite and > 0");
  } else if (kv->kv_scale != 1.0f) {
    return fail(MLA_ERR_INVALID_ARGUMENT, "kv_scale must be 1 for bf16 KV");
  }
  if (!aligned(q, 16) || !aligned(kv->pool, 16) || !aligned(kv->block_table, 4) ||
      !aligned(kv->seq_lens, 4))
    return fail(MLA_ERR_INVALID_ARGUMENT, "q and pool must be 16-byte aligned, tables 4-byte");
  if (!aligned(workspace, 256)) return fail(MLA_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
  if (workspace_bytes < plan->workspace_bytes)
    return fail(MLA_ERR_WORKSPACE_TOO_SMALL, "workspace %zu < %zu bytes", workspace_bytes,
                plan->workspace_bytes);
  if (out) {
    if (out_dtype != MLA_BF16 && out_dtype != MLA_FP32)
      return fail(MLA_ERR_UNSUPPORTED, "out_dtype %d", out_dtype);
    if (!aligned(out, 16)) return fail(MLA_ERR_INVALID_ARGUMENT, "out must be 16-byte aligned");
  }
  if (out_lse && !aligned(out_lse, 4)) return fail(MLA_ERR_INVALID_ARGUMENT, "out_lse misaligned");
  if (hidden && !aligned(hidden, 4)) return fail(MLA_ERR_INVALID_ARGUMENT, "hidden misaligned");

  const mla_decode_shape& s = plan->shape;
  hipStream_t st = (hipStream_t)stream;
  float* part_o = (float*)((char*)workspace + plan->o_offset);
  float* part_lse = (float*)((char*)workspace + plan->lse_offset);

  PartialParams pp{};
  pp.q = (const uint16_t*)q;
  pp.pool = (const uint8_t*)kv->pool;
  pp.block_table = kv->block_table;
  pp.seq_lens = kv->seq_lens;
  pp.part_o = part_o;
  pp.part_lse = part_lse;
  pp.num_pages = kv->num_pages;
  pp.max_pages = kv->max_pages_per_seq;
  pp.batch = s.batch;
  pp.q_len = s.q_len;
  pp.num_heads = s.num_heads;
  pp.head_groups = plan->head_groups;
  pp.rbw = plan->rbw;
  pp.row_groups = plan->row_groups;
  pp.rows = plan->rows;
  pp.causal = s.causal;
  pp.mode = plan->mode;
  pp.num_wg = plan->num_wg;
  pp.num_splits = plan->num_splits;
  pp.num_slots = plan->num_slots;
  pp.total_pages = plan->total_pages;
  const float log2e = 1.44269504088896341f;
  pp.score_scale = s.softmax_scale * log2e * (fp8 ? kv->kv_scale : 1.0f);
  pp.v_scale = fp8 ? kv->kv_scale : 1.0f;
  fill_plan_args(*plan, &pp.plan);
  pp.hidden = hidden;
  const int64_t kv_bytes = plan->total_pages * (int64_t)mla_page_bytes(kPage, plan->kv_dtype);
  pp.nt_parts = partial_nt_parts((int64_t)plan->o_bytes, kv_bytes);
  pp.stream_pages = kv_bytes > kStreamKvBytes;
  if (!out && !out_lse) {
    if (plan->num_wg > 0) {
      hipError_t e = launch_partial(pp, fp8, plan->fp8_qk != 0, st);
      if (e != hipSuccess) return fail(MLA_ERR_DEVICE, "partial launch: %s", hipGetErrorString(e));
    }
    return ok();
  }

  MergeParams mp{};
  mp.part_o = part_o;
  mp.part_lse = part_lse;
  mp.out = out;
  mp.out_lse = out_lse;
  mp.rows = plan->rows;
  mp.out_bf16 = out_dtype == MLA_BF16;
  mp.seq_lens = kv->seq_lens;
  mp.batch = s.batch;
  mp.max_pages = kv->max_pages_per_seq;
  mp.split_mode = plan->mode;
  mp.num_wg = plan->num_wg;
  mp.num_splits = plan->num_splits;
  mp.num_slots = plan->num_slots;
  mp.total_pages = plan->total_pages;
  mp.plan = pp.plan;
  hipError_t e = hipSuccess;
  if (plan->num_wg > 0) {
    e = launch_partial(pp, fp8, plan->fp8_qk != 0, st);
    if (e != hipSuccess) return fail(MLA_ERR_DEVICE, "partial launch: %s", hipGetErrorString(e));
  }
  e = launch_merge(mp, false, true, (int64_t)s.batch * plan->rows, plan->max_req_slots, plan->lds_reserve, st);
  if (e != hipSuccess) return fail(MLA_ERR_DEVICE, "merge launch: %s", hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

mla_status mla_kv_append(void* pool, int64_t num_pages, int32_t page_size, int32_t kv_dtype,
                         float kv_scale, const int32_t* block_table, int32_t max_pages_per_seq,
                         const int32_t* seq_lens, const void* latents, int32_t batch,
                         int32_t q_len, void* stream) {
  if (!pool || !block_table || !seq_lens || !latents) return fail(MLA_ERR_INVALID_ARGUMENT, "null pointer");
  if (batch < 1 || q_len < 1 || num_pages < 1 || max_pages_per_seq < 1)
    return fail(MLA_ERR_INVALID_ARGUMENT, "batch, q_len, num_pages, max_pages_per_seq must be >= 1");
  if ((int64_t)batch * q_len > INT32_MAX) return fail(MLA_ERR_UNSUPPORTED, "batch * q_len too large");
  if (page_size != kPage) return fail(MLA_ERR_UNSUPPORTED, "page_size %d (only %d)", page_size, kPage);
  const bool fp8 = kv_dtype == MLA_FP8_E4M3FN;
  if (!fp8 && kv_dtype != MLA_BF16) return fail(MLA_ERR_UNSUPPORTED, "kv_dtype %d", kv_dtype);
  if (fp8) {
    if (!(kv_scale > 0.f) || !std::isfinite(kv_scale))
      return fail(MLA_ERR_INVALID_ARGUMENT, "kv_scale must be finite and > 0");
  } else if (kv_scale != 1.0f) {
    return fail(MLA_ERR_INVALID_ARGUMENT, "kv_scale must be 1 for bf16 KV");
  }
  if (!aligned(pool, 16) || !aligned(latents, 16) || !aligned(block_table, 4) || !aligned(seq_lens, 4))
    return fail(MLA_ERR_INVALID_ARGUMENT, "pool and latents must be 16-byte aligned, tables 4-byte");
  hipError_t e = launch_kv_append(pool, num_pages, fp8, block_table, max_pages_per_seq, seq_lens,
                                  latents, batch * q_len, q_len, kv_scale, (hipStream_t)stream);
  if (e != hipSuccess) return fail(MLA_ERR_DEVICE, "append launch: %s", hipGetErrorString(e));
  return ok();
}

mla_status mla_read_reference(const void* buf, size_t bytes, int32_t mode, uint32_t* sink, void* stream) {
  if (mode < 0 || mode > 2) return fail(MLA_ERR_INVALID_ARGUMENT, "mode must be 0, 1 or 2");
  if (mode != 2) {
    if (!buf || !sink) return fail(MLA_ERR_INVALID_ARGUMENT, "null pointer");
    if (!aligned(buf, 16) || !aligned(sink, 4)) return fail(MLA_ERR_INVALID_ARGUMENT, "misaligned pointer");
    if (bytes % 1024 != 0 || bytes > ((size_t)1 << 40))
      return fail(MLA_ERR_INVALID_ARGUMENT, "bytes must be a multiple of 1024 (and below 1 TiB)");
  }
  hipError_t e = launch_read_reference(buf, (int64_t)bytes, mode, sink, (hipStream_t)stream);
  if (e != hipSuccess) return fail(MLA_ERR_DEVICE, "read reference launch: %s", hipGetErrorString(e));
  return ok();
}

mla_status mla_merge_lse(const void* part_o, int32_t part_dtype, const float* part_lse,
                         int32_t num_parts, int64_t rows, void* out, int32_t out_dtype,
                         float* out_lse, void* stream) {
  if (!part_o || !part_lse) return fail(MLA_ERR_INVALID_ARGUMENT, "null pointer");
  if (num_parts < 1 || rows < 1) return fail(MLA_ERR_INVALID_ARGUMENT, "num_parts and rows must be >= 1");
  if (part_dtype != MLA_BF16 && part_dtype != MLA_FP32)
    return fail(MLA_ERR_UNSUPPORTED, "part_dtype %d", part_dtype);
  if (out && out_dtype != MLA_BF16 && out_dtype != MLA_FP32)
    return fail(MLA_ERR_UNSUPPORTED, "out_dtype %d", out_dtype);
  if (!aligned(part_o, 16) || !aligned(part_lse, 4) || (out && !aligned(out, 16)) ||
      (out_lse && !aligned(out_lse, 4)))
    return fail(MLA_ERR_INVALID_ARGUMENT, "misaligned pointer");
  if (rows > (int64_t)INT32_MAX / 16) return fail(MLA_ERR_UNSUPPORTED, "too many rows");
  if (!out && !out_lse) return ok();
  MergeParams mp{};
  mp.part_o = part_o;
  mp.part_lse = part_lse;
  mp.out = out;
  mp.out_lse = out_lse;
  mp.rows = rows;
  mp.out_bf16 = out_dtype == MLA_BF16;
  mp.num_parts = num_parts;
  hipError_t e = launch_merge(mp, part_dtype == MLA_BF16, false, rows, num_parts, 0, (hipStream_t)stream);
  if (e != hipSuccess) return fail(MLA_ERR_DEVICE, "merge launch: %s", hipGetErrorString(e));
  return ok();
}

}  // extern "C"
