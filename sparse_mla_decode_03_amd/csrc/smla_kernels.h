// Launch interface between the host API and the gfx950 kernels (library-internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace smla {

struct DecodeArgs {
  const uint16_t* q;            // bf16 [R][H][576]
  const uint8_t* kv;            // paged cache bytes
  const int32_t* indices;       // [R][K]
  const int32_t* row_req;       // [R]            (LOGICAL)
  const int32_t* page_table;    // [B][max_pages] (LOGICAL)
  const float* sinks;           // [H] or null
  uint16_t* out;                // bf16 [R][H][512]      (final mode)
  float* lse;                   // [R][H] or null        (final mode)
  float* part_o;                // [R][S][H][512]        (partial mode)
  float* part_lse;              // [R][S][H]             (partial mode)
  unsigned long long* err;      // first bad (row << 32 | pos), or null
  // balanced rows (jobs set, else null): entries the decode keeps per row, each row's split
  // count (1..S), the (row | split << 24) jobs longest first, and their number
  const int32_t* row_count;     // [R]
  const int32_t* row_splits;    // [R]
  const int32_t* jobs;          // [R * S]
  const int32_t* job_count;     // [1]
  int32_t R, H, K, S, chunk, B;
  int32_t ps_log2, num_pages, num_slots, max_pages, index_mode;
  int32_t write_partials;       // 0 final output, 1 documented partials, 2 the merge's own format
  float scale_log2;             // softmax_scale * log2(e) (times the tensor scale, FMT 2)
  float out_scale;              // value scale applied to the output (the tensor scale, FMT 2; else 1)
};

struct IndexerLogitsArgs {
  const uint8_t* q;             // e4m3fn [R][64][128]
  const float* weights;         // [R][64]
  const uint8_t* keys;          // key pages: codes [64][128] | fp32 scales [64]
  const int32_t* row_len;       // [R]
  const int32_t* page_table;    // [B][max_pages]
  float* logits;                // [R][width]
  int32_t max_pages, num_pages, width;
  int32_t num_requests;          // B (rows = B * next_n)
  int32_t slots;                 // workgroups of the balanced schedule (a few per CU)
};

struct IndexerTopkArgs {
  const float* logits;          // [R][width]
  const int32_t* row_len;       // [R]
  int32_t* out;                 // [R][topk]
  int32_t width, topk;
  int32_t cus;                  // compute units of the device (row order across CUs)
};

int max_chunk_positions();
hipError_t launch_decode(const DecodeArgs& a, int kv_format, hipStream_t st);
// Balanced rows: count each row's entries that the decode with these arguments keeps into
// counts[R], give each row its split count (row_splits[R], 1..a.S, from its share of the work
// of `slots` workgroup slots) and list the (row, split) jobs longest first (jobs[R * a.S],
// job_count[1]).
hipError_t launch_balance(const DecodeArgs& a, int slots, int32_t* counts, int32_t* row_splits,
                          int32_t* jobs, int32_t* job_count, hipStream_t st);
hipError_t launch_merge(const float* part_o, const float* part_lse, int R, int S, int H,
                        const float* sinks, uint16_t* out, float* lse, hipStream_t st);
// Merge of the decode's own split format (DecodeArgs.write_partials == 2): part_o holds,
// per (row, split) and 32-head group, 16 blocks x 4 runs of 64 lanes x 4 unnormalized
// floats; part_ml holds (reference max in the log2 domain, probability sum) per head;
// out_scale multiplies the merged output (the per-tensor FP8 value scale, else 1).
// With row_splits (balanced rows) a row merges its first row_splits[r] chunks, and a row of
// one chunk is skipped (the decode wrote its output).
hipError_t launch_merge_native(const float* part_o, const float* part_ml, int R, int S, int H,
                               const float* sinks, float out_scale, uint16_t* out, float* lse,
                               const int32_t* row_splits, hipStream_t st);
hipError_t launch_gather_debug(const uint8_t* kv, int kv_format, int ps_log2, int num_slots,
                               const int* slots, int n, uint16_t* out, hipStream_t st);
hipError_t launch_fill_u64(unsigned long long* p, unsigned long long v, hipStream_t st);
hipError_t launch_store(const uint16_t* latent, const uint16_t* rope, const int32_t* slots, int n,
                        int kv_format, int ps_log2, int num_slots, uint8_t* kv, hipStream_t st);

hipError_t launch_indexer_logits(const IndexerLogitsArgs& a, int next_n, int num_requests, hipStream_t st);
hipError_t launch_indexer_topk(const IndexerTopkArgs& a, int rows, hipStream_t st);
hipError_t launch_translate(const int32_t* idx, const int32_t* row_req, const int32_t* page_table,
                            int rows, int topk, int num_requests, int max_pages, int ps_log2,
                            int num_pages, int32_t* out, hipStream_t st);

}  // namespace smla
