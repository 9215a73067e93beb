// Host side of the C ABI declared in include/sparse_mla.h: argument checks, the
// data-independent split planner, and kernel launches on the caller's stream.
#include <math.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "sparse_mla.h"
#include "smla_kernels.h"

namespace {

constexpr uint32_t kPlanMagic = 0x534d4c41u;  // "SMLA"
constexpr int kMaxDevices = 64;

struct PlanImpl {
  uint32_t magic;
  int32_t num_splits;
  int32_t chunk;
  int32_t ps_log2;
  smla_problem p;
  uint64_t off_part_o;
  uint64_t off_part_lse;
  uint64_t off_err;
  uint64_t off_balance;   // SMLA_F_BALANCE_ROWS: row counts [R], split counts [R], jobs [R * S], job count
  uint64_t ws_bytes;
  int32_t slots;          // workgroup slots of the device (balanced rows' target job length)
};
static_assert(sizeof(PlanImpl) <= sizeof(smla_plan), "plan does not fit its opaque storage");

std::atomic<int> g_cu_count[kMaxDevices];

// Scratch of the allocation-free run entry point: the fp32 split partials (and their LSEs)
// that sparse_mla_decode_run keeps in the caller's workspace.  One copy per GPU, for the
// life of the process.  Host code never uses the array's name as an address: the device
// address comes from hipGetSymbolAddress, once per device, with that device current.
constexpr size_t kScratchBytes = (size_t)SMLA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];
void* g_scratch_ptr[kMaxDevices];
bool g_scratch_ready[kMaxDevices];
std::mutex g_scratch_mu;

// This device's scratch address, or nullptr if the runtime could not resolve it.
void* scratch_on(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ready[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return nullptr;
    g_scratch_ptr[dev] = ptr;
    g_scratch_ready[dev] = true;
  }
  return g_scratch_ptr[dev];
}

int cu_count(int* out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return -1;
  if (dev < kMaxDevices) {
    const int c = g_cu_count[dev].load(std::memory_order_relaxed);
    if (c > 0) {
      *out = c;
      return 0;
    }
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    return -1;
  if (dev < kMaxDevices) g_cu_count[dev].store(n, std::memory_order_relaxed);
  *out = n;
  return 0;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

uint64_t round_up(uint64_t x, uint64_t a) { return (x + a - 1) / a * a; }

int log2_exact(int v) {
  int l = 0;
  while ((1 << l) < v) ++l;
  return (1 << l) == v ? l : -1;
}

const PlanImpl* as_impl(const smla_plan* plan) {
  if (plan == nullptr) return nullptr;
  const PlanImpl* pi = reinterpret_cast<const PlanImpl*>(plan->opaque);
  return pi->magic == kPlanMagic ? pi : nullptr;
}

smla_status check_problem(const smla_problem* p) {
  if (p->num_rows < 0 || p->topk < 4 || p->num_pages < 1) return SMLA_ERR_BAD_SHAPE;
  if (p->topk % 4 != 0) return SMLA_ERR_MISALIGNED;
  if (p->num_heads % 16 != 0 || p->num_heads < 16 || p->num_heads > SMLA_MAX_HEADS)
    return SMLA_ERR_UNSUPPORTED;
  if (p->kv_format != SMLA_KV_BF16 && p->kv_format != SMLA_KV_FP8_UE8M0 && p->kv_format != SMLA_KV_FP8_TENSOR)
    return SMLA_ERR_UNSUPPORTED;
  if (p->index_mode != SMLA_IDX_LOGICAL && p->index_mode != SMLA_IDX_GLOBAL) return SMLA_ERR_UNSUPPORTED;
  if (p->flags & ~(SMLA_F_PARTIALS_ONLY | SMLA_F_CHECK_INDICES | SMLA_F_BALANCE_ROWS))
    return SMLA_ERR_UNSUPPORTED;
  // the documented partials are chunks of positions, which balancing would change
  if ((p->flags & SMLA_F_BALANCE_ROWS) && (p->flags & SMLA_F_PARTIALS_ONLY)) return SMLA_ERR_UNSUPPORTED;
  // balanced jobs are coded as row | split << 24
  if ((p->flags & SMLA_F_BALANCE_ROWS) && p->num_rows >= (1 << 24)) return SMLA_ERR_BAD_SHAPE;
  const int l = log2_exact(p->page_size);
  if (p->page_size < 1 || p->page_size > 1024 || l < 0) return SMLA_ERR_BAD_SHAPE;
  // FP8 pages are 648 * page_size bytes; the 16-byte copies need an even page size
  if (p->kv_format == SMLA_KV_FP8_UE8M0 && p->page_size < 2) return SMLA_ERR_UNSUPPORTED;
  if ((int64_t)p->num_pages * p->page_size > INT32_MAX) return SMLA_ERR_BAD_SHAPE;
  if (p->index_mode == SMLA_IDX_LOGICAL) {
    if (p->num_requests < 1 || p->max_pages_per_req < 1) return SMLA_ERR_BAD_SHAPE;
    if ((int64_t)p->max_pages_per_req * p->page_size > INT32_MAX) return SMLA_ERR_BAD_SHAPE;
  }
  if (p->num_splits < 0 || p->num_splits > SMLA_MAX_SPLITS || p->num_splits > p->topk)
    return SMLA_ERR_BAD_SHAPE;
  if (!isfinite(p->softmax_scale)) return SMLA_ERR_BAD_SHAPE;
  if (p->kv_format == SMLA_KV_FP8_TENSOR && !(isfinite(p->kv_scale) && p->kv_scale > 0.f))
    return SMLA_ERR_BAD_SHAPE;
  return SMLA_OK;
}

// Splits: enough (row, split) workgroups to give every CU work when there are few rows,
// chunks of at least 128 positions, and at most the per-workgroup position capacity.
// With at least one row per CU, the split count that finishes the grid soonest: the grid
// runs in rounds of `slots` workgroups (two per CU when a workgroup has at most two waves,
// one otherwise), so a count is priced as rounds x (chunk + kSplitOverhead), the overhead
// being a workgroup's set-up, its partial write and its share of the merge, in positions
// (measured: 627 rows of 64 heads and a 2048-entry list on 256 CUs run 1.22 rounds at one
// split and 2.45 at two, and two splits are 7 % faster; 512 rows of 128 heads stay at one).
constexpr int kSplitOverhead = 512;
int choose_splits(const smla_problem* p, int num_cus) {
  const int cap = smla::max_chunk_positions();
  const int min_s = (p->topk + cap - 1) / cap;
  int s = min_s;
  const int64_t rows = p->num_rows > 0 ? p->num_rows : 1;
  if (rows < num_cus) {
    int want = (int)((num_cus + rows - 1) / rows);
    // chunks of at least 128 positions, but a list of two tiles or more still splits in two
    // (two one-tile chunks and the merge beat one two-tile pass when rows are few)
    int by_len = p->topk / 128;
    const int short_split = p->topk >= 64 ? 2 : 1;
    if (by_len < short_split) by_len = short_split;
    if (want > by_len) want = by_len;
    if (want > s) s = want;
  } else {
    const int64_t slots = (int64_t)num_cus * ((p->num_heads + 31) / 32 <= 2 ? 2 : 1);
    // balanced rows with a row per workgroup slot: the device gives each row its own split
    // count, up to one more than the least, so that only the longest rows split (chunks of
    // at least 128 positions)
    if (p->flags & SMLA_F_BALANCE_ROWS) {
      if (p->topk / (s + 1) >= 128 && s < SMLA_MAX_SPLITS) ++s;
      return s;
    }
    auto cost = [&](int c) {
      const int64_t rounds = (rows * c + slots - 1) / slots;
      return rounds * ((p->topk + c - 1) / c + kSplitOverhead);
    };
    for (int c = min_s + 1; c <= min_s + 2; ++c)
      if (p->topk / c >= 128 && (p->topk + c - 1) / c <= cap && cost(c) < cost(s)) s = c;
  }
  if (s > SMLA_MAX_SPLITS) s = SMLA_MAX_SPLITS;
  return s;
}

}  // namespace

extern "C" {

smla_status sparse_mla_decode_plan(const smla_problem* p, int32_t num_cus, smla_plan* plan,
                                   size_t* workspace_bytes) {
  if (p == nullptr || plan == nullptr || workspace_bytes == nullptr) return SMLA_ERR_NULL_ARG;
  const smla_status st = check_problem(p);
  if (st != SMLA_OK) return st;
  int cus = num_cus;
  if (cus <= 0 && cu_count(&cus) != 0) return SMLA_ERR_HIP;
  const int cap = smla::max_chunk_positions();
  int s = p->num_splits > 0 ? p->num_splits : choose_splits(p, cus);
  const int chunk = (p->topk + s - 1) / s;
  if (chunk > cap) return SMLA_ERR_UNSUPPORTED;

  PlanImpl pi;
  memset(&pi, 0, sizeof(pi));
  pi.magic = kPlanMagic;
  pi.num_splits = s;
  pi.chunk = chunk;
  pi.ps_log2 = log2_exact(p->page_size);
  pi.p = *p;
  uint64_t off = 0;
  const bool partials_in_ws = s > 1 && !(p->flags & SMLA_F_PARTIALS_ONLY);
  if (partials_in_ws) {
    // the decode's own split format: O blocks of whole 32-head groups (padded heads
    // included), then (reference max, probability sum) per head
    const uint64_t rs = (uint64_t)p->num_rows * s;
    const uint64_t groups = (uint64_t)(p->num_heads + 31) / 32;
    pi.off_part_o = off;
    off = round_up(off + rs * groups * 32 * SMLA_V_DIM * sizeof(float), 256);
    pi.off_part_lse = off;
    off = round_up(off + rs * p->num_heads * 2 * sizeof(float), 256);
  }
  if (p->flags & SMLA_F_CHECK_INDICES) {
    pi.off_err = off;
    off = round_up(off + sizeof(unsigned long long), 256);
  }
  if (p->flags & SMLA_F_BALANCE_ROWS) {
    pi.off_balance = off;
    off = round_up(off + ((2 + (uint64_t)s) * p->num_rows + 1) * sizeof(int32_t), 256);
  }
  pi.slots = cus * ((p->num_heads + 31) / 32 <= 2 ? 2 : 1);
  pi.ws_bytes = off;
  memset(plan, 0, sizeof(*plan));
  memcpy(plan->opaque, &pi, sizeof(pi));
  *workspace_bytes = (size_t)off;
  return SMLA_OK;
}

int32_t sparse_mla_plan_num_splits(const smla_plan* plan) {
  const PlanImpl* pi = as_impl(plan);
  return pi ? pi->num_splits : -1;
}

}  // extern "C"

namespace {

// Pointer checks of a run (host only; rows > 0).
smla_status check_run_args(const PlanImpl* pi, const void* q, const void* kv_cache,
                           const int32_t* indices, const int32_t* row_req, const int32_t* page_table,
                           const float* sinks, const void* out, const float* lse,
                           const float* partial_o, const float* partial_lse) {
  const smla_problem& p = pi->p;
  const bool partials_only = (p.flags & SMLA_F_PARTIALS_ONLY) != 0;
  const bool logical = p.index_mode == SMLA_IDX_LOGICAL;
  if (q == nullptr || kv_cache == nullptr || indices == nullptr) return SMLA_ERR_NULL_ARG;
  if (logical && (row_req == nullptr || page_table == nullptr)) return SMLA_ERR_NULL_ARG;
  if (partials_only ? (partial_o == nullptr || partial_lse == nullptr) : out == nullptr)
    return SMLA_ERR_NULL_ARG;
  if (!aligned(q, 16) || !aligned(kv_cache, 16) || !aligned(indices, 16) || !aligned(out, 16) ||
      !aligned(partial_o, 16) || !aligned(partial_lse, 4) || !aligned(lse, 4) ||
      !aligned(sinks, 4) || !aligned(row_req, 4) || !aligned(page_table, 4))
    return SMLA_ERR_MISALIGNED;
  return SMLA_OK;
}

// The body of sparse_mla_decode_run, shared with the allocation-free entry point.
smla_status run_impl(const PlanImpl* pi, const void* q, const void* kv_cache, const int32_t* indices,
                     const int32_t* row_req, const int32_t* page_table, const float* sinks, void* out,
                     float* lse, float* partial_o, float* partial_lse, void* workspace,
                     size_t workspace_bytes, void* stream) {
  const smla_problem& p = pi->p;
  const bool partials_only = (p.flags & SMLA_F_PARTIALS_ONLY) != 0;
  const bool logical = p.index_mode == SMLA_IDX_LOGICAL;
  if (p.num_rows == 0) return SMLA_OK;  // nothing to do; empty tensors may pass NULL
  const smla_status ca = check_run_args(pi, q, kv_cache, indices, row_req, page_table, sinks, out, lse,
                                        partial_o, partial_lse);
  if (ca != SMLA_OK) return ca;
  if (pi->ws_bytes > 0 && workspace == nullptr) return SMLA_ERR_NULL_ARG;
  if (workspace_bytes < pi->ws_bytes) return SMLA_ERR_WORKSPACE_TOO_SMALL;
  if (!aligned(workspace, 256)) return SMLA_ERR_MISALIGNED;

  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  uint8_t* ws = reinterpret_cast<uint8_t*>(workspace);
  smla::DecodeArgs a;
  memset(&a, 0, sizeof(a));
  a.q = reinterpret_cast<const uint16_t*>(q);
  a.kv = reinterpret_cast<const uint8_t*>(kv_cache);
  a.indices = indices;
  a.row_req = row_req;
  a.page_table = page_table;
  a.sinks = sinks;
  a.R = p.num_rows;
  a.H = p.num_heads;
  a.K = p.topk;
  a.S = pi->num_splits;
  a.chunk = pi->chunk;
  a.B = logical ? p.num_requests : 0;
  a.ps_log2 = pi->ps_log2;
  a.num_pages = p.num_pages;
  a.num_slots = p.num_pages * p.page_size;
  a.max_pages = logical ? p.max_pages_per_req : 0;
  a.index_mode = p.index_mode;
  const bool tensor_fp8 = p.kv_format == SMLA_KV_FP8_TENSOR;
  a.scale_log2 = p.softmax_scale * (tensor_fp8 ? p.kv_scale : 1.0f) * 1.4426950408889634f;
  a.out_scale = tensor_fp8 ? p.kv_scale : 1.0f;
  if (p.flags & SMLA_F_CHECK_INDICES) {
    a.err = reinterpret_cast<unsigned long long*>(ws + pi->off_err);
    if (smla::launch_fill_u64(a.err, ~0ull, st) != hipSuccess) return SMLA_ERR_HIP;
  }
  const bool merge = pi->num_splits > 1 && !partials_only;
  const bool balance = (p.flags & SMLA_F_BALANCE_ROWS) != 0;
  if (partials_only) {
    a.write_partials = 1;
    a.part_o = partial_o;
    a.part_lse = partial_lse;
  } else if (merge) {
    a.write_partials = 2;
    a.part_o = reinterpret_cast<float*>(ws + pi->off_part_o);
    a.part_lse = reinterpret_cast<float*>(ws + pi->off_part_lse);
    if (balance) {   // rows of one split write their output directly
      a.out = reinterpret_cast<uint16_t*>(out);
      a.lse = lse;
    }
  } else {
    a.write_partials = 0;
    a.out = reinterpret_cast<uint16_t*>(out);
    a.lse = lse;
  }
  if (balance) {
    int32_t* counts = reinterpret_cast<int32_t*>(ws + pi->off_balance);
    int32_t* row_splits = counts + p.num_rows;
    int32_t* jobs = row_splits + p.num_rows;
    int32_t* job_count = jobs + (size_t)p.num_rows * pi->num_splits;
    if (smla::launch_balance(a, pi->slots, counts, row_splits, jobs, job_count, st) != hipSuccess)
      return SMLA_ERR_HIP;
    a.row_count = counts;
    a.row_splits = row_splits;
    a.jobs = jobs;
    a.job_count = job_count;
  }
  if (smla::launch_decode(a, p.kv_format, st) != hipSuccess) return SMLA_ERR_HIP;
  if (merge) {
    if (smla::launch_merge_native(a.part_o, a.part_lse, a.R, a.S, a.H, sinks, a.out_scale,
                                  reinterpret_cast<uint16_t*>(out), lse, a.row_splits, st) != hipSuccess)
      return SMLA_ERR_HIP;
  }
  return SMLA_OK;
}

}  // namespace

extern "C" {

smla_status sparse_mla_decode_run(const smla_plan* plan, const void* q, const void* kv_cache,
                                  const int32_t* indices, const int32_t* row_req,
                                  const int32_t* page_table, const float* sinks, void* out,
                                  float* lse, float* partial_o, float* partial_lse,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  const PlanImpl* pi = as_impl(plan);
  if (pi == nullptr) return SMLA_ERR_BAD_PLAN;
  return run_impl(pi, q, kv_cache, indices, row_req, page_table, sinks, out, lse, partial_o,
                  partial_lse, workspace, workspace_bytes, stream);
}

smla_status sparse_mla_decode_run_noalloc(const smla_plan* plan, const void* q, const void* kv_cache,
                                          const int32_t* indices, const int32_t* row_req,
                                          const int32_t* page_table, const float* sinks, void* out,
                                          float* lse, void* stream) {
  const PlanImpl* pi = as_impl(plan);
  if (pi == nullptr) return SMLA_ERR_BAD_PLAN;
  if (pi->p.flags & (SMLA_F_PARTIALS_ONLY | SMLA_F_CHECK_INDICES)) return SMLA_ERR_UNSUPPORTED;
  if (pi->ws_bytes > kScratchBytes) return SMLA_ERR_WORKSPACE_TOO_SMALL;
  if (pi->p.num_rows == 0) return SMLA_OK;
  const smla_status ca = check_run_args(pi, q, kv_cache, indices, row_req, page_table, sinks, out, lse,
                                        nullptr, nullptr);
  if (ca != SMLA_OK) return ca;   // every argument check comes before the first HIP call
  void* ws = nullptr;
  if (pi->ws_bytes > 0) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return SMLA_ERR_HIP;
    ws = scratch_on(dev);
    if (ws == nullptr) return SMLA_ERR_HIP;
  }
  return run_impl(pi, q, kv_cache, indices, row_req, page_table, sinks, out, lse, nullptr, nullptr,
                  ws, pi->ws_bytes > 0 ? kScratchBytes : 0, stream);
}

smla_status sparse_mla_merge_partials(const float* partial_o, const float* partial_lse,
                                      int32_t num_rows, int32_t num_splits, int32_t num_heads,
                                      const float* sinks, void* out, float* lse, void* stream) {
  if (num_rows < 0 || num_splits < 1 || num_splits > SMLA_MAX_SPLITS || num_heads < 1 ||
      num_heads > 1024)
    return SMLA_ERR_BAD_SHAPE;
  if ((int64_t)num_rows * num_heads > INT32_MAX) return SMLA_ERR_BAD_SHAPE;
  if (num_rows == 0) return SMLA_OK;
  if (partial_o == nullptr || partial_lse == nullptr || out == nullptr) return SMLA_ERR_NULL_ARG;
  if (!aligned(partial_o, 16) || !aligned(out, 16) || !aligned(partial_lse, 4) || !aligned(lse, 4) ||
      !aligned(sinks, 4))
    return SMLA_ERR_MISALIGNED;
  if (smla::launch_merge(partial_o, partial_lse, num_rows, num_splits, num_heads, sinks,
                         reinterpret_cast<uint16_t*>(out), lse,
                         reinterpret_cast<hipStream_t>(stream)) != hipSuccess)
    return SMLA_ERR_HIP;
  return SMLA_OK;
}

smla_status sparse_mla_gather_debug(const void* kv_cache, int32_t kv_format, int32_t page_size,
                                    int32_t num_pages, const int32_t* slots, int32_t n, void* out,
                                    void* stream) {
  if (kv_format != SMLA_KV_BF16 && kv_format != SMLA_KV_FP8_UE8M0 && kv_format != SMLA_KV_FP8_TENSOR)
    return SMLA_ERR_UNSUPPORTED;
  const int l = log2_exact(page_size);
  if (n < 0 || num_pages < 1 || page_size < 1 || page_size > 1024 || l < 0 ||
      (int64_t)num_pages * page_size > INT32_MAX)
    return SMLA_ERR_BAD_SHAPE;
  if (n == 0) return SMLA_OK;
  if (kv_cache == nullptr || slots == nullptr || out == nullptr) return SMLA_ERR_NULL_ARG;
  if (!aligned(kv_cache, 16) || !aligned(out, 16) || !aligned(slots, 4)) return SMLA_ERR_MISALIGNED;
  if (smla::launch_gather_debug(reinterpret_cast<const uint8_t*>(kv_cache), kv_format, l,
                                num_pages * page_size, slots, n, reinterpret_cast<uint16_t*>(out),
                                reinterpret_cast<hipStream_t>(stream)) != hipSuccess)
    return SMLA_ERR_HIP;
  return SMLA_OK;
}

smla_status sparse_mla_cache_store(const void* latent, const void* rope, const int32_t* slots,
                                   int32_t num_tokens, int32_t kv_format, int32_t page_size,
                                   int32_t num_pages, void* kv_cache, void* stream) {
  if (kv_format != SMLA_KV_BF16 && kv_format != SMLA_KV_FP8_UE8M0) return SMLA_ERR_UNSUPPORTED;
  const int l = log2_exact(page_size);
  if (num_tokens < 0 || num_pages < 1 || page_size < 1 || page_size > 1024 || l < 0 ||
      (int64_t)num_pages * page_size > INT32_MAX)
    return SMLA_ERR_BAD_SHAPE;
  if (kv_format == SMLA_KV_FP8_UE8M0 && page_size < 2) return SMLA_ERR_UNSUPPORTED;
  if (num_tokens == 0) return SMLA_OK;
  if (latent == nullptr || rope == nullptr || slots == nullptr || kv_cache == nullptr)
    return SMLA_ERR_NULL_ARG;
  if (!aligned(latent, 16) || !aligned(rope, 16) || !aligned(kv_cache, 16) || !aligned(slots, 4))
    return SMLA_ERR_MISALIGNED;
  if (smla::launch_store(reinterpret_cast<const uint16_t*>(latent), reinterpret_cast<const uint16_t*>(rope),
                         slots, num_tokens, kv_format, l, num_pages * page_size,
                         reinterpret_cast<uint8_t*>(kv_cache), reinterpret_cast<hipStream_t>(stream)) != hipSuccess)
    return SMLA_ERR_HIP;
  return SMLA_OK;
}

smla_status sparse_mla_indexer_logits(const void* q_codes, const float* weights, const void* key_cache,
                                      const int32_t* row_len, const int32_t* page_table,
                                      int32_t num_requests, int32_t next_n, int32_t num_heads,
                                      int32_t page_size, int32_t num_pages, int32_t max_pages,
                                      int32_t width, float* logits, void* stream) {
  if (num_heads != 64 || page_size != 64 || next_n < 1 || next_n > 4) return SMLA_ERR_UNSUPPORTED;
  if (num_requests < 0 || num_pages < 1 || width < 64 || width % 64 != 0 || width > (1 << 28) ||
      max_pages < width / 64 ||
      (int64_t)num_requests * next_n > INT32_MAX / 64 || (int64_t)num_pages * page_size > INT32_MAX)
    return SMLA_ERR_BAD_SHAPE;
  if (num_requests == 0) return SMLA_OK;
  if (q_codes == nullptr || weights == nullptr || key_cache == nullptr || row_len == nullptr ||
      page_table == nullptr || logits == nullptr)
    return SMLA_ERR_NULL_ARG;
  if (!aligned(q_codes, 16) || !aligned(weights, 16) || !aligned(key_cache, 16) || !aligned(logits, 16) ||
      !aligned(row_len, 4) || !aligned(page_table, 4))
    return SMLA_ERR_MISALIGNED;
  smla::IndexerLogitsArgs a;
  a.q = reinterpret_cast<const uint8_t*>(q_codes);
  a.weights = weights;
  a.keys = reinterpret_cast<const uint8_t*>(key_cache);
  a.row_len = row_len;
  a.page_table = page_table;
  a.logits = logits;
  a.max_pages = max_pages;
  a.num_pages = num_pages;
  a.width = width;
  a.num_requests = num_requests;
  // the schedule's slots: three workgroups per CU (what fits beside each other), so every
  // CU streams an equal share of the key pages
  int cus = 0;
  if (cu_count(&cus) != 0) return SMLA_ERR_HIP;
  a.slots = 3 * cus;
  if (smla::launch_indexer_logits(a, next_n, num_requests, reinterpret_cast<hipStream_t>(stream)) != hipSuccess)
    return SMLA_ERR_HIP;
  return SMLA_OK;
}

smla_status sparse_mla_indexer_topk(const float* logits, const int32_t* row_len, int32_t rows,
                                    int32_t width, int32_t topk, int32_t* indices, void* stream) {
  if (rows < 0 || width < 4 || width % 4 != 0 || topk < 1 || topk > (1 << 20)) return SMLA_ERR_BAD_SHAPE;
  if (rows == 0) return SMLA_OK;
  if (logits == nullptr || row_len == nullptr || indices == nullptr) return SMLA_ERR_NULL_ARG;
  if (!aligned(logits, 16) || !aligned(row_len, 4) || !aligned(indices, 4)) return SMLA_ERR_MISALIGNED;
  smla::IndexerTopkArgs a;
  a.logits = logits;
  a.row_len = row_len;
  a.out = indices;
  a.width = width;
  a.topk = topk;
  int cus = 0;
  if (cu_count(&cus) != 0) return SMLA_ERR_HIP;
  a.cus = cus;
  if (smla::launch_indexer_topk(a, rows, reinterpret_cast<hipStream_t>(stream)) != hipSuccess)
    return SMLA_ERR_HIP;
  return SMLA_OK;
}

smla_status sparse_mla_translate_indices(const int32_t* indices, const int32_t* row_req,
                                        const int32_t* page_table, int32_t rows, int32_t topk,
                                        int32_t num_requests, int32_t max_pages, int32_t page_size,
                                        int32_t num_pages, int32_t* slots, void* stream) {
  const int l = log2_exact(page_size);
  if (rows < 0 || topk < 1 || num_requests < 1 || max_pages < 1 || num_pages < 1 || l < 0 ||
      page_size > 1024 || (int64_t)num_pages * page_size > INT32_MAX || (int64_t)rows * topk > INT32_MAX)
    return SMLA_ERR_BAD_SHAPE;
  if (rows == 0) return SMLA_OK;
  if (indices == nullptr || row_req == nullptr || page_table == nullptr || slots == nullptr)
    return SMLA_ERR_NULL_ARG;
  if (!aligned(indices, 4) || !aligned(row_req, 4) || !aligned(page_table, 4) || !aligned(slots, 4))
    return SMLA_ERR_MISALIGNED;
  if (smla::launch_translate(indices, row_req, page_table, rows, topk, num_requests, max_pages, l, num_pages,
                             slots, reinterpret_cast<hipStream_t>(stream)) != hipSuccess)
    return SMLA_ERR_HIP;
  return SMLA_OK;
}

smla_status sparse_mla_read_index_error(const smla_plan* plan, const void* workspace,
                                        int32_t* row_pos, void* stream) {
  const PlanImpl* pi = as_impl(plan);
  if (pi == nullptr) return SMLA_ERR_BAD_PLAN;
  if (row_pos == nullptr || workspace == nullptr) return SMLA_ERR_NULL_ARG;
  if (!(pi->p.flags & SMLA_F_CHECK_INDICES)) return SMLA_ERR_UNSUPPORTED;
  unsigned long long v = 0;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const uint8_t* src = reinterpret_cast<const uint8_t*>(workspace) + pi->off_err;
  if (hipMemcpyAsync(&v, src, sizeof(v), hipMemcpyDeviceToHost, st) != hipSuccess) return SMLA_ERR_HIP;
  if (hipStreamSynchronize(st) != hipSuccess) return SMLA_ERR_HIP;
  if (v == ~0ull) {
    row_pos[0] = -1;
    row_pos[1] = -1;
  } else {
    row_pos[0] = (int32_t)(v >> 32);
    row_pos[1] = (int32_t)(v & 0xffffffffu);
  }
  return SMLA_OK;
}

// The code arrives as a plain int: an out-of-range value must not be loaded as the enum.
const char* sparse_mla_status_string(int32_t status) {
  switch (status) {
    case SMLA_OK: return "ok";
    case SMLA_ERR_NULL_ARG: return "a required pointer is NULL";
    case SMLA_ERR_BAD_SHAPE: return "invalid or inconsistent size";
    case SMLA_ERR_UNSUPPORTED: return "unsupported head count, format, index mode, flag or split";
    case SMLA_ERR_MISALIGNED: return "pointer or row stride breaks the alignment rule";
    case SMLA_ERR_WORKSPACE_TOO_SMALL: return "workspace smaller than the plan requires";
    case SMLA_ERR_HIP: return "HIP runtime error";
    case SMLA_ERR_BAD_PLAN: return "plan was not produced by sparse_mla_decode_plan";
    default: return "unknown status";
  }
}

int32_t sparse_mla_version(void) { return 100; }

}  // extern "C"
