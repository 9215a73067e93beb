// Test infrastructure: stand-ins for the kernel launchers and the few HIP runtime calls
// that the host API (smla_api.hip) makes, so that its argument checks, planning and launch
// marshalling can be built for the CPU alone with AddressSanitizer and UBSan and driven
// through the C ABI with no GPU and no HIP runtime.  A launcher records what it was asked
// to launch and touches no memory; the runtime stand-ins report one device with the CU
// count set by smla_hostcheck_set_cus, and a fake scratch address that is never
// dereferenced.  Built by tests/host_check/hostcheck_build.py; nothing in the library uses
// this file.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>

#include "smla_kernels.h"

#ifndef SMLA_HOSTCHECK_CMAX
#error "SMLA_HOSTCHECK_CMAX (the decode kernel's positions per workgroup) must be defined"
#endif

namespace {

enum Kind { kDecode, kMerge, kGather, kFill, kStore, kLogits, kTopk, kTranslate, kMergeNative, kBalance,
            kKinds };

int g_counts[kKinds];
smla::DecodeArgs g_last_decode;
int g_last_decode_format = -1;
int g_last_merge[3];             // R, S, H
const void* g_last_merge_ptrs[2];  // part_o, part_lse
int g_cus = 256;
float g_last_merge_scale = 0.f;
const int32_t* g_last_merge_splits = nullptr;
int g_last_balance[4];               // R, K, S, slots
const void* g_last_balance_ptrs[5];  // indices, counts, row_splits, jobs, job_count
unsigned char g_fatbin_stand_in[16];

// Where the stand-in hipGetSymbolAddress says the scratch array lives: an address that
// no test dereferences (every launch is a stand-in).
constexpr uintptr_t kFakeScratch = 0x7f0000000000ull;

}  // namespace

namespace smla {

int max_chunk_positions() { return SMLA_HOSTCHECK_CMAX; }

hipError_t launch_decode(const DecodeArgs& a, int kv_format, hipStream_t) {
  ++g_counts[kDecode];
  g_last_decode = a;
  g_last_decode_format = kv_format;
  return hipSuccess;
}
hipError_t launch_merge(const float* part_o, const float* part_lse, int R, int S, int H, const float*,
                        uint16_t*, float*, hipStream_t) {
  ++g_counts[kMerge];
  g_last_merge[0] = R;
  g_last_merge[1] = S;
  g_last_merge[2] = H;
  g_last_merge_ptrs[0] = part_o;
  g_last_merge_ptrs[1] = part_lse;
  return hipSuccess;
}
hipError_t launch_merge_native(const float* part_o, const float* part_ml, int R, int S, int H,
                               const float*, float out_scale, uint16_t*, float*, const int32_t* row_splits,
                               hipStream_t) {
  ++g_counts[kMergeNative];
  g_last_merge_splits = row_splits;
  g_last_merge_scale = out_scale;
  g_last_merge[0] = R;
  g_last_merge[1] = S;
  g_last_merge[2] = H;
  g_last_merge_ptrs[0] = part_o;
  g_last_merge_ptrs[1] = part_ml;
  return hipSuccess;
}
hipError_t launch_balance(const DecodeArgs& a, int slots, int32_t* counts, int32_t* row_splits,
                          int32_t* jobs, int32_t* job_count, hipStream_t) {
  ++g_counts[kBalance];
  g_last_balance[0] = a.R;
  g_last_balance[1] = a.K;
  g_last_balance[2] = a.S;
  g_last_balance[3] = slots;
  g_last_balance_ptrs[0] = a.indices;
  g_last_balance_ptrs[1] = counts;
  g_last_balance_ptrs[2] = row_splits;
  g_last_balance_ptrs[3] = jobs;
  g_last_balance_ptrs[4] = job_count;
  return hipSuccess;
}
hipError_t launch_gather_debug(const uint8_t*, int, int, int, const int*, int, uint16_t*, hipStream_t) {
  ++g_counts[kGather];
  return hipSuccess;
}
hipError_t launch_fill_u64(unsigned long long*, unsigned long long, hipStream_t) {
  ++g_counts[kFill];
  return hipSuccess;
}
hipError_t launch_store(const uint16_t*, const uint16_t*, const int32_t*, int, int, int, int, uint8_t*,
                        hipStream_t) {
  ++g_counts[kStore];
  return hipSuccess;
}
hipError_t launch_indexer_logits(const IndexerLogitsArgs&, int, int, hipStream_t) {
  ++g_counts[kLogits];
  return hipSuccess;
}
hipError_t launch_indexer_topk(const IndexerTopkArgs&, int, hipStream_t) {
  ++g_counts[kTopk];
  return hipSuccess;
}
hipError_t launch_translate(const int32_t*, const int32_t*, const int32_t*, int, int, int, int, int, int,
                            int32_t*, hipStream_t) {
  ++g_counts[kTranslate];
  return hipSuccess;
}

}  // namespace smla

extern "C" {

// ---- the HIP runtime calls of the host API ------------------------------------------------
hipError_t hipGetDevice(int* deviceId) {
  *deviceId = 0;
  return hipSuccess;
}
hipError_t hipDeviceGetAttribute(int* pi, hipDeviceAttribute_t attr, int) {
  if (attr != hipDeviceAttributeMultiprocessorCount) return hipErrorInvalidValue;
  *pi = g_cus;
  return hipSuccess;
}
hipError_t hipGetSymbolAddress(void** devPtr, const void*) {
  *devPtr = reinterpret_cast<void*>(kFakeScratch);
  return hipSuccess;
}
// Only the index-error word is ever copied back: report "no bad index" (all ones).
hipError_t hipMemcpyAsync(void* dst, const void*, size_t sizeBytes, hipMemcpyKind, hipStream_t) {
  std::memset(dst, 0xff, sizeBytes);
  return hipSuccess;
}
hipError_t hipStreamSynchronize(hipStream_t) { return hipSuccess; }

// ---- code-object registration that host compilation emits for the scratch array ------------
void** __hipRegisterFatBinary(const void*) { return reinterpret_cast<void**>(g_fatbin_stand_in); }
void __hipRegisterVar(void**, void*, char*, char*, int, size_t, int, int) {}
void __hipUnregisterFatBinary(void**) {}
unsigned char smla_hostcheck_fatbin[16];

// ---- what the tests read back --------------------------------------------------------------
void smla_hostcheck_reset() {
  std::memset(g_counts, 0, sizeof(g_counts));
  std::memset(&g_last_decode, 0, sizeof(g_last_decode));
  g_last_decode_format = -1;
  std::memset(g_last_merge, 0, sizeof(g_last_merge));
  g_last_merge_ptrs[0] = g_last_merge_ptrs[1] = nullptr;
  std::memset(g_last_balance, 0, sizeof(g_last_balance));
  std::memset(g_last_balance_ptrs, 0, sizeof(g_last_balance_ptrs));
  g_last_merge_splits = nullptr;
}
void smla_hostcheck_set_cus(int n) { g_cus = n; }
float smla_hostcheck_last_merge_scale() { return g_last_merge_scale; }
// Launch counts by kind: 0 decode, 1 merge (documented partials), 2 gather_debug, 3 fill,
// 4 store, 5 indexer logits, 6 indexer top-k, 7 translate, 8 merge of the decode's own format,
// 9 row count and order (balanced splits).
int smla_hostcheck_launches(int kind) { return kind >= 0 && kind < kKinds ? g_counts[kind] : -1; }
uintptr_t smla_hostcheck_fake_scratch() { return kFakeScratch; }
// The last decode launch: ints = R, H, K, S, chunk, B, ps_log2, num_pages, num_slots,
// max_pages, index_mode, write_partials, kv_format; floats = scale_log2, out_scale;
// ptrs = q, kv, indices, row_req, page_table, sinks, out, lse, part_o, part_lse, err.
void smla_hostcheck_last_decode(int32_t* ints, float* floats, uintptr_t* ptrs) {
  const smla::DecodeArgs& a = g_last_decode;
  const int32_t iv[13] = {a.R, a.H, a.K, a.S, a.chunk, a.B, a.ps_log2, a.num_pages, a.num_slots,
                          a.max_pages, a.index_mode, a.write_partials, g_last_decode_format};
  std::memcpy(ints, iv, sizeof(iv));
  floats[0] = a.scale_log2;
  floats[1] = a.out_scale;
  const void* pv[11] = {a.q, a.kv, a.indices, a.row_req, a.page_table, a.sinks,
                        a.out, a.lse, a.part_o, a.part_lse, a.err};
  for (int i = 0; i < 11; ++i) ptrs[i] = reinterpret_cast<uintptr_t>(pv[i]);
}
// The last balance launch: ints = R, K, S, slots; ptrs = indices, counts, row_splits, jobs,
// job_count, then the last decode launch's row_count, row_splits, jobs and job_count, then the
// last native merge's row_splits.
void smla_hostcheck_last_balance(int32_t* ints, uintptr_t* ptrs) {
  std::memcpy(ints, g_last_balance, sizeof(g_last_balance));
  for (int i = 0; i < 5; ++i) ptrs[i] = reinterpret_cast<uintptr_t>(g_last_balance_ptrs[i]);
  ptrs[5] = reinterpret_cast<uintptr_t>(g_last_decode.row_count);
  ptrs[6] = reinterpret_cast<uintptr_t>(g_last_decode.row_splits);
  ptrs[7] = reinterpret_cast<uintptr_t>(g_last_decode.jobs);
  ptrs[8] = reinterpret_cast<uintptr_t>(g_last_decode.job_count);
  ptrs[9] = reinterpret_cast<uintptr_t>(g_last_merge_splits);
}
// The last merge launch (either kind): ints = R, S, H; ptrs = part_o, part_lse or part_ml.
void smla_hostcheck_last_merge(int32_t* ints, uintptr_t* ptrs) {
  std::memcpy(ints, g_last_merge, sizeof(g_last_merge));
  ptrs[0] = reinterpret_cast<uintptr_t>(g_last_merge_ptrs[0]);
  ptrs[1] = reinterpret_cast<uintptr_t>(g_last_merge_ptrs[1]);
}

}  // extern "C"
