// Indexer for gfx950: FP8 paged MQA logits over each query row's context, and the top-k
// selection that turns them into the index lists the decode path reads.
//
// The indexer's FP8 paged MQA logits are named on prhub sglang#24692 (implementation
// breakdown item 5, key files); prhub vllm#52164 (implementation breakdown items 1-5,
// key code excerpts) has the kernel take a request's next_n query rows natively, so that
// every key page is read once for all of them, with per-row context lengths.  The logit
// of row r at position t is sum_h w[r][h] * max(0, scale_t * <q[r][h], codes_t>) with
// 128-dimensional e4m3fn queries and keys; top-k keeps the K largest logits, a tie at the
// boundary going to the smaller position.
//
// Logits: a fixed grid of three workgroups per compute unit, each taking an equal run of
// the key pages of all requests (request order), segment by segment; a segment's pages
// stream through a four-page LDS ring by global_load_lds.  Wave w serves row w % next_n of
// the request on its share of each page's two 32-token blocks, so a page is read from HBM
// once for all rows.  Scores come from the FP8 MFMA 32x32x64 (rows = 32 heads, columns =
// 32 tokens); each lane then holds one token and 16 heads of a block, so the weighted ReLU
// sum over heads is 32 FMAs, and one swap between lane halves finishes both token blocks of a
// page (block 0 in lanes 0..31, block 1 in lanes 32..63), stored together.  The key scale multiplies
// the head sum (the ReLU is positively homogeneous; scales are >= 0).  Logits are stored
// from the loop through a buffer descriptor of the row's length, so stores past it are
// dropped and every page issues the same stores, which the loop's vmcnt waits count.
//
// Top-k: one workgroup per row, two per CU, rows ordered by length so that a CU holds a
// long row and a short one.  Logits map to order-preserving 32-bit keys.  A histogram of
// the top 12 bits finds the bin of the K-th largest key; while it is built, every key at or
// above a capture bin estimated from the row's first 8192 positions is kept in LDS with its
// position, so a row is normally read once.  Two histogram levels (10 + 10 bits) over the
// kept keys give the K-th largest key T and how many of its ties are taken (the smallest
// positions), the selected positions are set in an LDS bitmap, and the output is the bitmap
// read in order.  When the estimate fails the row is read again; rows past the bitmap's
// 131072 positions, or with a crowded boundary bin, write the output in a last pass.
#include <type_traits>

#include "smla_device.h"
#include "smla_kernels.h"

namespace smla {

namespace {

typedef int __attribute__((ext_vector_type(8))) i32x8;

constexpr int kIdxDim = 128;
constexpr int kIdxHeads = 64;
constexpr int kKeyPage = 64;                       // tokens per key page
constexpr int kKeyPageCodes = kIdxDim * kKeyPage;  // 8192 bytes of codes, then 64 fp32 scales
constexpr int kKeyPageBytes = kKeyPageCodes + 4 * kKeyPage;
constexpr int kSegPages = 256;                   // page ids staged per segment
constexpr int kRing = 4;
constexpr int kSlotBytes = kKeyPageBytes;          // one LDS ring slot

// Copies (global -> LDS, 16 or 4 bytes per lane) from a wave-uniform base address in SGPRs
// plus a 32-bit per-lane byte offset, so the page loop keeps no 64-bit per-lane address
// arithmetic; lds_addr is the wave's LDS destination (m0).
__device__ __forceinline__ void dma16_sv(const void* sbase, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :: "v"(voff), "s"(sbase), "s"(lds_addr) : "memory");
}
__device__ __forceinline__ void dma4_sv(const void* sbase, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1"
               :: "v"(voff), "s"(sbase), "s"(lds_addr) : "memory");
}

__device__ __forceinline__ float halves_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// LDS key page: token t's codes at t*128, its logical 16-byte chunk c stored at chunk
// c ^ ((t >> 1) & 7), so the 16 lanes of a B-operand read (16 tokens, one chunk) hit 16
// different chunk slots; the scales follow at byte 8192.
__device__ __forceinline__ int key_swz(int t) { return (t >> 1) & 7; }

// Wait until this wave's copy of the current page has landed.  After it, in issue order,
// the wave has issued the copies of `lc` later pages (PER instructions each) and the logit
// stores of `ls` earlier pages (ST instructions each); all of those may stay in flight.
template <int PER, int ST>
__device__ __forceinline__ void wait_page_sched(int lc, int ls) {
  static_assert(kRing == 4, "the table covers up to three later pages");
#define SMLA_W(L, S) case 4 * L + S: wait_vm_le<L * PER + S * ST>(); break;
  switch (4 * lc + ls) {
    SMLA_W(0, 0) SMLA_W(0, 1) SMLA_W(0, 2) SMLA_W(0, 3)
    SMLA_W(1, 0) SMLA_W(1, 1) SMLA_W(1, 2) SMLA_W(1, 3)
    SMLA_W(2, 0) SMLA_W(2, 1) SMLA_W(2, 2) SMLA_W(2, 3)
    SMLA_W(3, 0) SMLA_W(3, 1) SMLA_W(3, 2) SMLA_W(3, 3)
    default: wait_vm(); break;
  }
#undef SMLA_W
}

// Key pages of request b: its longest row, capped at the width, in 64-token pages.
template <int NN>
__device__ __forceinline__ int request_pages(const IndexerLogitsArgs& a, int b) {
  int m = 0;
#pragma unroll
  for (int i = 0; i < NN; ++i) m = max(m, min(a.row_len[(size_t)b * NN + i], a.width));
  return (m + kKeyPage - 1) / kKeyPage;
}

// Block-wide inclusive scan of one 64-bit value per thread (256 threads); `tmp` holds 4.
__device__ __forceinline__ long long block_incl_scan64(long long v, long long* tmp, long long& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  long long x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const long long y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  if (lane == 63) tmp[wave] = x;
  __syncthreads();
  long long before = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    before += w < wave ? tmp[w] : 0;
    total += tmp[w];
  }
  __syncthreads();
  return x + before;
}

// Logits: a fixed grid of a.slots workgroups (a few per CU).  The key pages of all requests,
// in request order, are cut into a.slots equal runs of consecutive pages; workgroup k takes
// run k, request by request, in segments of at most kSegPages pages.  A segment loads the
// request's queries, weights and page ids, fills the four-page ring, and then streams its
// pages with the copies kRing - 1 pages ahead; a request's next_n rows are served by the
// waves as before, so a key page is read once for all of them.
template <int NN>
__global__ __launch_bounds__(256, 3) void indexer_logits_kernel(IndexerLogitsArgs a) {
  // G groups of next_n waves split each page's two 32-token blocks
  constexpr int G = NN <= 2 ? 2 : 1;
  // logit stores per page of an active wave: one (a wave serving both 32-token blocks
  // stores them together, block 0 from lanes 0..31 and block 1 from lanes 32..63)
  constexpr int ST = 1;
  __shared__ __attribute__((aligned(16))) uint8_t sRing[kRing * kSlotBytes];
  __shared__ int sPage[kSegPages];
  __shared__ int sOk[kSegPages];
  __shared__ long long sScan[4];
  __shared__ long long sStart[2];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int B = a.num_requests;

  // ---- this workgroup's run of pages [g0, g1) and the request and page it starts at
  long long T = 0;
  for (int base = 0; base < B; base += 256) {
    const int bb = base + tid;
    long long tot;
    block_incl_scan64(bb < B ? request_pages<NN>(a, bb) : 0, sScan, tot);
    T += tot;
  }
  const long long g0 = (long long)blockIdx.x * T / a.slots;
  const long long g1 = (long long)(blockIdx.x + 1) * T / a.slots;
  if (g0 >= g1) return;                              // the whole workgroup
  {
    long long run = 0;
    for (int base = 0; base < B; base += 256) {
      const int bb = base + tid;
      const int np = bb < B ? request_pages<NN>(a, bb) : 0;
      long long tot;
      const long long incl = run + block_incl_scan64(np, sScan, tot);
      if (np > 0 && incl - np <= g0 && g0 < incl) {
        sStart[0] = bb;
        sStart[1] = g0 - (incl - np);
      }
      run += tot;
    }
    __syncthreads();
  }
  // uniform: kept in SGPRs (so the output buffer descriptor below is scalar)
  int b = __builtin_amdgcn_readfirstlane((int)sStart[0]);
  int p = __builtin_amdgcn_readfirstlane((int)sStart[1]);
  long long g = g0;

  const bool active = wave < NN * G;
  const int ri = wave % NN, grp = wave / NN;
  // byte offset of this lane's token in a page's logits, per token block; lanes 32..63
  // start at 2^31, past any row's length in bytes
  int st_base[2];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) st_base[nb] = lane < 32 ? 4 * (32 * nb + lane) : (int)0x80000000u;
  // byte offsets in a ring slot of this lane's B-operand chunks of token block 0 (k-step ks,
  // half hh); token block 1 is 32 tokens (4096 bytes) further with the same swizzle, since
  // the swizzle depends on token bits 1..3 only
  int koff[2][2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int tn0 = lane & 31;
      const int lc = 4 * ks + 2 * (lane >> 5) + hh;
      koff[ks][hh] = tn0 * kIdxDim + 16 * (lc ^ key_swz(tn0));
    }
  static_assert(((32 >> 1) & 7) == 0, "token block 1 shares block 0's swizzle");

  // Page copies: wave w's instruction j fills 1 KB of codes (tokens 8(4j + w) .. +7, lane
  // = physical chunk); wave 0 also copies the 64 scales.
  // this lane's source offsets in a key page (fixed), and the ring's LDS address
  uint32_t src_off[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int t = 8 * (4 * j + wave) + (lane >> 3);
    src_off[j] = t * kIdxDim + 16 * ((lane & 7) ^ key_swz(t));
  }
  const uint32_t ring_lds = lds_offset(sRing);
  auto issue_page = [&](int it, int u) {             // u = it % kRing
    const uint8_t* src = a.keys + (size_t)__builtin_amdgcn_readfirstlane(sPage[it]) * kKeyPageBytes;
    const uint32_t slot = ring_lds + u * kSlotBytes;
#pragma unroll
    for (int j = 0; j < 2; ++j) dma16_sv(src, src_off[j], slot + 1024 * (4 * j + wave));
    if (wave == 0) dma4_sv(src, kKeyPageCodes + 4 * lane, slot + kKeyPageCodes);
  };

  while (g < g1) {
    const int npb = request_pages<NN>(a, b);
    if (p >= npb) {                                 // next request (uniform)
      ++b;
      p = 0;
      continue;
    }
    const int n = (int)min((long long)min(npb - p, kSegPages), g1 - g);
    const int row = b * NN + ri;
    const int row_len = __builtin_amdgcn_readfirstlane(min(a.row_len[row], a.width));

    // page ids of the segment
    if (tid < n) {
      const int pid = a.page_table[(size_t)b * a.max_pages + p + tid];
      const bool ok = pid >= 0 && pid < a.num_pages;
      sPage[tid] = ok ? pid : 0;                    // invalid pages are read from page 0
      sOk[tid] = ok;
    }
    // A operands (queries) and weights of this wave's row: head block mb holds heads
    // 32mb + lane%32; k-step ks covers dims 64ks .. 64ks+63, lane half lane/32 its bytes
    // 32*(lane/32) .. +31.  The accumulator register j of a block holds head
    // 8(j/4) + 4(lane/32) + j%4, whose weight is wj[mb][j].  Inactive waves load a real
    // row (row0 + wave % NN) whose values go unused.
    i32x8 qa[2][2];
    float wj[2][16];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      const uint8_t* qh = a.q + ((size_t)row * kIdxHeads + 32 * mb + (lane & 31)) * kIdxDim + 32 * (lane >> 5);
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const u32x4 lo = *reinterpret_cast<const u32x4*>(qh + 64 * ks);
        const u32x4 hi = *reinterpret_cast<const u32x4*>(qh + 64 * ks + 16);
        qa[mb][ks] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
      }
      const float* wr = a.weights + (size_t)row * kIdxHeads + 32 * mb + 4 * (lane >> 5);
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const f32x4 w4 = *reinterpret_cast<const f32x4*>(wr + 8 * g4);
#pragma unroll
        for (int e = 0; e < 4; ++e) wj[mb][4 * g4 + e] = w4[e];
      }
    }
    // this wave's row of logits as a range-checked buffer of row_len floats: a store at or
    // past the row's length is dropped by the hardware, so every page issues the same store
    // instructions (the waits below count them) and positions past the length stay untouched
    const __amdgpu_buffer_rsrc_t out_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        a.logits + (size_t)row * a.width, (short)0, active ? row_len * 4 : 0, 0x00020000);
    __syncthreads();                                // page ids visible

    for (int it = 0; it < min(n, kRing); ++it) issue_page(it, it);
    // The compiler does not see the page copies (inline asm): one full wait here, which it
    // does see, lets it count the query, weight and page-id loads as done, so it puts no
    // waits of its own inside the page loop.  It costs the spread of the first copies.
    wait_vm();

    // the page loop unrolled by the ring: each page's slot is a constant LDS offset
    // (folded into the reads' immediate offsets)
    for (int it0 = 0; it0 < n; it0 += kRing)
#pragma unroll
    for (int u = 0; u < kRing; ++u) {
      const int it = it0 + u;
      if (it >= n) break;                             // uniform
      {
        const int lc = min(kRing - 1, n - 1 - it), ls = min(it, kRing - 1);
        if (wave == 0) wait_page_sched<3, ST>(lc, ls);
        else if (active) wait_page_sched<2, ST>(lc, ls);
        else wait_page_sched<2, 0>(lc, ls);
      }
      __syncthreads();
      if (active) {
        const uint8_t* slot = sRing + u * kSlotBytes;
        const float* scl = reinterpret_cast<const float*>(slot + kKeyPageCodes);
        const bool page_ok = sOk[it] != 0;
        // per token block served: the head sum of each lane's 32 scores, its two head-block
        // halves kept apart (halves the dependent FMA chain)
        float xs[2 / G];
#pragma unroll
        for (int q = 0; q < 2 / G; ++q) {
          const int nb = G == 1 ? q : grp;
          f32x16 acc[2] = {f32x16{}, f32x16{}};
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
            const u32x4 lo = *reinterpret_cast<const u32x4*>(slot + 32 * kIdxDim * nb + koff[ks][0]);
            const u32x4 hi = *reinterpret_cast<const u32x4*>(slot + 32 * kIdxDim * nb + koff[ks][1]);
            const i32x8 kb = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
              acc[mb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(qa[mb][ks], kb, acc[mb], 0, 0, 0, 127, 0, 127);
          }
          // ReLU as a signed-integer max on the bits (a negative float is a negative
          // integer, so it becomes +0; a non-negative one is unchanged): one instruction,
          // where fmaxf costs two (its NaN-quieting canonicalization, then the max)
          float part[2] = {0.f, 0.f};
#pragma unroll
          for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int j = 0; j < 16; ++j) {
              const float r = __int_as_float(max(__float_as_int(acc[mb][j]), 0));
              part[mb] = __builtin_fmaf(wj[mb][j], r, part[mb]);
            }
          xs[q] = part[0] + part[1];
        }
        // The lane halves hold the other half of each token's heads.  Serving both blocks,
        // one swap of block 0's upper lanes with block 1's lower lanes and one add leave
        // block 0's logits in lanes 0..31 and block 1's in lanes 32..63: lane = token.
        float tot;
        int tok;
        if constexpr (G == 1) {
          const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(xs[0]), __float_as_uint(xs[1]), false, false);
          tot = __uint_as_float(r[0]) + __uint_as_float(r[1]);
          tok = lane;
        } else {
          tot = halves_sum(xs[0]);
          tok = 32 * grp + (lane & 31);
        }
        const float logit = page_ok ? tot * scl[tok] : -INFINITY;
        // with one block served, lanes 32..63 repeat lanes 0..31: their offset is past any
        // row (2^31 and up), so they store nothing
        const int off = (G == 1 ? 4 * lane : st_base[grp]) + 4 * kKeyPage * (p + it);
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(logit), out_rsrc, off, 0, 0);
      }
      __syncthreads();
      if (it + kRing < n) issue_page(it + kRing, u);
    }
    g += n;
    p += n;
    __syncthreads();                                // the ring and the page ids are free
  }
}

// ---- top-k ------------------------------------------------------------------------------

// Order-preserving key of a float: larger floats give larger unsigned keys (-inf lowest
// among non-NaN values).  A non-negative float keeps its bits with the sign bit set; a
// negative one becomes the two's complement negation of its bits, so -0 and +0 (equal
// floats) share the key 0x80000000 and the more negative a float, the smaller its key.
// Branch-free: m is 0 or all ones by the sign, and (u ^ (m | sign)) - m is u | sign or -u.
__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t u = __float_as_uint(f);
  const uint32_t m = (uint32_t)((int32_t)u >> 31);
  return (u ^ (m | 0x80000000u)) - m;
}

constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / 64;
constexpr int kBins1 = 4096;                   // first level: the top 12 bits of a key
constexpr int kShift1 = 20;
constexpr int kListCap = 6080;                 // keys and positions kept in LDS
constexpr int kBitCap = 131072;                // longest row whose selection is a bitmap in LDS
constexpr int kOrderBuckets = 32;              // length classes of the row order

// Block-wide exclusive prefix sum of one value per thread; returns the prefix and the
// total.  Uses `scratch` (kTopkWaves ints).
__device__ __forceinline__ int block_excl_scan(int v, int* scratch, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  if (lane == 63) scratch[wave] = x;
  __syncthreads();
  int before = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < kTopkWaves; ++w) {
    const int s = scratch[w];
    if (w < wave) before += s;
    total += s;
  }
  __syncthreads();
  return before + x - v;
}

constexpr int kPerThread = 8;                  // consecutive positions per thread and round
// Keys of positions ip .. ip + kPerThread - 1.  FULL: the whole round lies inside the row
// (no checks); otherwise positions >= n give key 0, below every real key but never counted
// (callers check the position).  The values are loaded first and the keys formed after
// both paths join, so all of a thread's loads are in flight together.
template <bool FULL>
__device__ __forceinline__ void load_keys_run(const float* lg, int ip, int n, uint32_t (&k)[kPerThread]) {
  float v[kPerThread];
  if (FULL || ip + kPerThread <= n) {
#pragma unroll
    for (int g = 0; g < kPerThread / 4; ++g) {
      const f32x4 x = *reinterpret_cast<const f32x4*>(lg + ip + 4 * g);
#pragma unroll
      for (int e = 0; e < 4; ++e) v[4 * g + e] = x[e];
    }
  } else {
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) v[e] = ip + e < n ? lg[ip + e] : 0.f;
  }
#pragma unroll
  for (int e = 0; e < kPerThread; ++e) k[e] = (FULL || ip + e < n) ? order_key(v[e]) : 0u;
}
constexpr int kRound = kPerThread * kTopkThreads;

// The bin holding the need-th largest of a histogram counted from the top: thread i owns
// bins nbins-1-per*i .. nbins-per*(i+1) (descending).  Writes (bin, count still needed
// from it) to sel.  All threads call it.
__device__ __forceinline__ void find_bin(const int* hist, int nbins, int need, int* scratch, int* sel) {
  const int tid = threadIdx.x;
  const int per = nbins / kTopkThreads;
  int local = 0;
  for (int j = 0; j < per; ++j) local += hist[nbins - 1 - (per * tid + j)];
  int total;
  const int before = block_excl_scan(local, scratch, total);
  if (before < need && before + local >= need) {
    int acc = before;
    for (int j = 0; j < per; ++j) {
      const int bin = nbins - 1 - (per * tid + j);
      const int c = hist[bin];
      if (acc + c >= need) {
        sel[0] = bin;
        sel[1] = need - acc;
        break;
      }
      acc += c;
    }
  }
  __syncthreads();
}

__global__ __launch_bounds__(kTopkThreads, 8) void indexer_topk_kernel(IndexerTopkArgs a) {
  __shared__ int sHist[kBins1];
  __shared__ uint32_t sKey[kListCap];
  __shared__ int sPos[kListCap];
  __shared__ uint32_t sBits[kBitCap / 32];
  __shared__ int sListN;
  __shared__ int sScan[kTopkWaves];
  __shared__ int sSel[2];
  __shared__ int sRow;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // ---- which row.  Two workgroups of this kernel share a CU, and a grid that fills the
  // chip in order puts blocks b and b + cus on one CU, so the CU's time is the sum of its
  // two rows'.  With cus < rows <= kTopkThreads every workgroup orders the rows the same
  // way (by length class, longest first, ties by index: a bijection) and block b < cus
  // takes rank b, block cus + j rank P - 1 - j (P = min(rows, 2 cus): a long row and a
  // short one per CU), later blocks the ranks after P in order.
  int r = blockIdx.x;
  const int R = (int)gridDim.x;
  if (R > a.cus && R <= kTopkThreads) {
    int* table = sHist;                         // counts per (class desc, wave), then prefixes
    const int wave = tid >> 6;
    int cls = -1;
    if (tid < R) {
      const long long L = max(0, min(a.row_len[tid], a.width));
      cls = (int)(L * kOrderBuckets / ((long long)a.width + 1));
    }
    int inr = 0, wc = 0;                        // rank among the wave's rows of its class
#pragma unroll 1
    for (int v = 0; v < kOrderBuckets; ++v) {
      const uint64_t m = __ballot(cls == v);
      if (cls == v)
        inr = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
      if (lane == v) wc = __popcll(m);
    }
    if (lane < kOrderBuckets) table[(kOrderBuckets - 1 - lane) * kTopkWaves + wave] = wc;
    __syncthreads();
    constexpr int kEntries = kOrderBuckets * kTopkWaves;
    static_assert(kEntries <= kTopkThreads && kEntries <= kBins1, "row order table");
    int total;
    const int pre = block_excl_scan(tid < kEntries ? table[tid] : 0, sScan, total);
    if (tid < kEntries) table[tid] = pre;
    __syncthreads();
    const int P = min(R, 2 * a.cus);
    const int b = (int)blockIdx.x;
    const int want = b < a.cus ? b : (b < P ? P - 1 - (b - a.cus) : b);
    if (tid < R && table[(kOrderBuckets - 1 - cls) * kTopkWaves + wave] + inr == want) sRow = tid;
    __syncthreads();
    r = sRow;
  }
  const int n = max(0, min(a.row_len[r], a.width));
  const int K = a.topk;
  const float* lg = a.logits + (size_t)r * a.width;
  int32_t* out = a.out + (size_t)r * K;

  if (n <= K) {
    for (int j = tid; j < K; j += kTopkThreads) out[j] = j < n ? j : -1;
    return;
  }
  // A row of at most kBitCap positions ends in an LDS bitmap of the selected positions,
  // read in order for the output.
  const bool bitmap = n <= kBitCap;             // block uniform
  const int nwords = (n + 31) >> 5;
  for (int i = tid; i < kBins1; i += kTopkThreads) sHist[i] = 0;
  if (bitmap)
    for (int i = tid; i < nwords; i += kTopkThreads) sBits[i] = 0u;
  if (tid == 0) {
    sSel[0] = 0;
    sSel[1] = K;
    sListN = 0;
  }
  __syncthreads();
  // rounds wholly inside the row run without position checks; the ragged last round after
  const int nfull = n - n % kRound;             // block uniform

  // The round's keys k with lo <= k <= hi, and their positions, appended to the LDS list in
  // any order: per element a ballot of the lanes holding one, a lane's slot the count in
  // the earlier elements' ballots plus its rank in its own, one reservation per wave.
  // Slots past kListCap are counted in sListN but not written.  Every lane calls it.
  auto append = [&](auto full, int base, const uint32_t (&k)[kPerThread], uint32_t lo, uint32_t hi) {
    constexpr bool F = decltype(full)::value;
    const int ip = base + kPerThread * tid;
    uint64_t sel[kPerThread];
    int before[kPerThread], total = 0;            // wave uniform
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) {
      sel[e] = __ballot((F || ip + e < n) && k[e] >= lo && k[e] <= hi);
      before[e] = total;
      total += __popcll(sel[e]);
    }
    if (total > 0) {
      int slot0 = 0;
      if (lane == 0) slot0 = atomicAdd(&sListN, total);
      slot0 = __builtin_amdgcn_readfirstlane(slot0);
#pragma unroll
      for (int e = 0; e < kPerThread; ++e)
        if (sel[e] != 0ull && ((sel[e] >> lane) & 1ull)) {
          const int at = slot0 + before[e] +
                         (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(sel[e] >> 32),
                                                        __builtin_amdgcn_mbcnt_lo((uint32_t)sel[e], 0u));
          if (at < kListCap) {
            sKey[at] = k[e];
            sPos[at] = ip + e;
          }
        }
    }
  };
  auto hist_round = [&](auto full, int base, uint32_t (&k)[kPerThread]) {
    constexpr bool F = decltype(full)::value;
    const int ip = base + kPerThread * tid;
    load_keys_run<F>(lg, ip, n, k);
#pragma unroll
    for (int e = 0; e < kPerThread; ++e)
      if (F || ip + e < n) atomicAdd(&sHist[k[e] >> kShift1], 1);
  };

  // ---- pass 1: histogram of the top 12 bits.  On a bitmap row the first round (up to
  // kRound positions) is a sample: the bin holding its ts-th largest key, ts the share of K
  // expected in the sample plus three standard deviations, is the capture bin bt, and every
  // key of bin bt or above is listed while the pass goes on.  When the K-th largest key of
  // the row lies in bin bt or above and the list held every such key, the row is read once.
  int bt = kBins1;                              // no capture
  if (bitmap) {
    uint32_t k0[kPerThread];
    if (nfull > 0) hist_round(std::true_type{}, 0, k0);
    else hist_round(std::false_type{}, 0, k0);
    __syncthreads();
    const int n0 = min(n, kRound);
    int ts = K;
    if (n0 < n) {
      const float mu = (float)K * (float)n0 / (float)n;
      ts = min(n0, (int)ceilf(mu + 3.0f * sqrtf(mu)) + 8);
    }
    find_bin(sHist, kBins1, ts, sScan, sSel);
    bt = sSel[0];
    const uint32_t lo = (uint32_t)bt << kShift1;
    if (nfull > 0) append(std::true_type{}, 0, k0, lo, 0xFFFFFFFFu);
    else append(std::false_type{}, 0, k0, lo, 0xFFFFFFFFu);
#pragma unroll 1
    for (int base = kRound; base < nfull; base += kRound) {
      uint32_t k[kPerThread];
      hist_round(std::true_type{}, base, k);
      append(std::true_type{}, base, k, lo, 0xFFFFFFFFu);
    }
    if (nfull > 0 && nfull < n) {
      uint32_t k[kPerThread];
      hist_round(std::false_type{}, nfull, k);
      append(std::false_type{}, nfull, k, lo, 0xFFFFFFFFu);
    }
  } else {
#pragma unroll 1
    for (int base = 0; base < nfull; base += kRound) {
      uint32_t k[kPerThread];
      hist_round(std::true_type{}, base, k);
    }
    if (nfull < n) {
      uint32_t k[kPerThread];
      hist_round(std::false_type{}, nfull, k);
    }
  }
  __syncthreads();
  find_bin(sHist, kBins1, K, sScan, sSel);
  const int b1 = sSel[0];                       // the bin of the K-th largest key
  int need = sSel[1];                           // how many of b1's keys are taken
  const int c1 = sHist[b1];
  const int listed = sListN;
  __syncthreads();

  uint32_t T;
  int ties_total = -1;                          // how many keys equal T (every route sets it)
  const bool single = bitmap && bt <= b1 && listed <= kListCap;   // block uniform
  if (single || c1 <= kListCap) {
    int nlist = listed;
    if (!single) {
      nlist = c1;
      if (tid == 0) sListN = 0;
      __syncthreads();
      const uint32_t lo = (uint32_t)b1 << kShift1, hi = lo | ((1u << kShift1) - 1u);
      if (bitmap) {
        // ---- pass 2: the positions of the bins above b1 marked in the bitmap, b1's keys
        // listed (any order) ----
        auto pass2_round = [&](auto full, int base) {
          constexpr bool F = decltype(full)::value;
          const int ip = base + kPerThread * tid;
          uint32_t k[kPerThread];
          load_keys_run<F>(lg, ip, n, k);
          uint32_t bits = 0u;
#pragma unroll
          for (int e = 0; e < kPerThread; ++e) bits |= ((F || ip + e < n) && k[e] > hi ? 1u : 0u) << e;
          // a thread's 8 positions sit in one word (ip is a multiple of 8); bits is 0 past n
          if (bits) atomicOr(&sBits[ip >> 5], bits << (ip & 31));
          append(full, base, k, lo, hi);
        };
#pragma unroll 1
        for (int base = 0; base < nfull; base += kRound) pass2_round(std::true_type{}, base);
        if (nfull < n) pass2_round(std::false_type{}, nfull);
      } else {
        // ---- pass 2: b1's keys and positions in position order (one block scan per
        // round over the counts) ----
        int cand_before = 0;
#pragma unroll 1
        for (int base = 0; base < n; base += kRound) {
          const int ip = base + kPerThread * tid;
          uint32_t k[kPerThread];
          load_keys_run<false>(lg, ip, n, k);
          int nc = 0;
#pragma unroll
          for (int e = 0; e < kPerThread; ++e)
            if (ip + e < n) nc += (k[e] >> kShift1) == (uint32_t)b1 ? 1 : 0;
          int tot;
          int pc = cand_before + block_excl_scan(nc, sScan, tot);
#pragma unroll
          for (int e = 0; e < kPerThread; ++e)
            if (ip + e < n && (k[e] >> kShift1) == (uint32_t)b1) {
              sKey[pc] = k[e];
              sPos[pc] = ip + e;
              ++pc;
            }
          cand_before += tot;
        }
      }
    }
    // ---- the K-th largest key T among the listed keys of bin b1: bits 19..10, then 9..0 ----
    uint32_t prefix = (uint32_t)b1 << kShift1, mask = 0xFFFu << kShift1;
#pragma unroll 1
    for (int pass = 0; pass < 2; ++pass) {
      const int shift = pass == 0 ? 10 : 0;
      __syncthreads();
      for (int i = tid; i < 1024; i += kTopkThreads) sHist[i] = 0;
      __syncthreads();
      for (int c = tid; c < nlist; c += kTopkThreads) {
        const uint32_t k = sKey[c];
        if ((k & mask) == prefix) atomicAdd(&sHist[(k >> shift) & 1023], 1);
      }
      __syncthreads();
      find_bin(sHist, 1024, need, sScan, sSel);
      prefix |= (uint32_t)sSel[0] << shift;
      mask |= 1023u << shift;
      need = sSel[1];
      if (pass == 1) ties_total = sHist[sSel[0]];
    }
    T = prefix;
    if (bitmap) {
      // ---- selection: listed keys above T, and the `need` ties at T with the smallest
      // positions (all of them when every tie is taken) ----
      const bool all_ties = ties_total == need;
      int last_tie = INT32_MAX;                  // ties at positions <= last_tie are taken
      if (!all_ties) {
        // the need-th smallest tie position, by two histogram levels over its bits
        // (position / 64, then position % 64), counted from the top on reversed bins
        int lvl_need = need, hi = 0;
#pragma unroll 1
        for (int lvl = 0; lvl < 2; ++lvl) {
          __syncthreads();
          for (int i = tid; i < 2048; i += kTopkThreads) sHist[i] = 0;
          __syncthreads();
          for (int c = tid; c < nlist; c += kTopkThreads) {
            const int pos = sPos[c];
            if (sKey[c] == T && (lvl == 0 || (pos >> 6) == hi))
              atomicAdd(&sHist[2047 - (lvl == 0 ? (pos >> 6) : (pos & 63))], 1);
          }
          __syncthreads();
          find_bin(sHist, 2048, lvl_need, sScan, sSel);
          if (lvl == 0) hi = 2047 - sSel[0];
          else last_tie = 64 * hi + (2047 - sSel[0]);
          lvl_need = sSel[1];
        }
      }
      for (int c = tid; c < nlist; c += kTopkThreads) {
        const uint32_t k = sKey[c];
        const int pos = sPos[c];
        if (k > T || (k == T && pos <= last_tie)) atomicOr(&sBits[pos >> 5], 1u << (pos & 31));
      }
      __syncthreads();
      // ---- output: the bitmap in position order (each thread a run of words) ----
      const int per = (nwords + kTopkThreads - 1) / kTopkThreads;
      const int w0 = min(nwords, per * tid), w1 = min(nwords, w0 + per);
      int cnt = 0;
      for (int w = w0; w < w1; ++w) cnt += __popc(sBits[w]);
      int tot;
      int at = block_excl_scan(cnt, sScan, tot);
      // with K within the list's capacity the positions are staged in the list (no longer
      // read) and leave in contiguous runs; otherwise each goes straight out
      const bool stage = K <= kListCap;             // block uniform
      int* stg = reinterpret_cast<int*>(sKey);
      for (int w = w0; w < w1; ++w) {
        uint32_t m = sBits[w];
        while (m) {
          const int bit = __ffs(m) - 1;
          if (at < K) {
            if (stage) stg[at] = 32 * w + bit;
            else out[at] = 32 * w + bit;
          }
          ++at;
          m &= m - 1u;
        }
      }
      if (stage) {
        __syncthreads();
        for (int j = tid; j < K; j += kTopkThreads) out[j] = stg[j];
      }
      return;
    }
  } else {
    // ---- passes 2 and 3 over the row (a crowded first bin): bits 19..10, then 9..0 ----
    uint32_t prefix = (uint32_t)b1 << kShift1, mask = 0xFFFu << kShift1;
#pragma unroll 1
    for (int pass = 0; pass < 2; ++pass) {
      const int shift = pass == 0 ? 10 : 0;
      for (int i = tid; i < 1024; i += kTopkThreads) sHist[i] = 0;
      __syncthreads();
      for (int ip = kPerThread * tid; ip < n; ip += kRound) {
        uint32_t k[kPerThread];
        load_keys_run<false>(lg, ip, n, k);
#pragma unroll
        for (int e = 0; e < kPerThread; ++e)
          if (ip + e < n && (k[e] & mask) == prefix) atomicAdd(&sHist[(k[e] >> shift) & 1023], 1);
      }
      __syncthreads();
      find_bin(sHist, 1024, need, sScan, sSel);
      prefix |= (uint32_t)sSel[0] << shift;
      mask |= 1023u << shift;
      need = sSel[1];
      if (pass == 1) ties_total = sHist[sSel[0]];   // every key of the last bin equals T
      __syncthreads();
    }
    T = prefix;
  }
  // ---- last pass: every key above T and the first `need` keys equal to T, written in
  // ascending position order: a thread owns kPerThread consecutive positions of each round, so a
  // block scan over the threads keeps that order.  When every tie is taken, one scan per
  // round suffices.
  const bool all_ties = ties_total == need;
  int ties_before = 0, out_before = 0;
#pragma unroll 1
  for (int base = 0; base < n; base += kRound) {
    const int ip = base + kPerThread * tid;
    uint32_t k[kPerThread];
    load_keys_run<false>(lg, ip, n, k);
    int sel[kPerThread], cnt = 0;
    if (all_ties) {
#pragma unroll
      for (int e = 0; e < kPerThread; ++e) {
        sel[e] = (ip + e < n && k[e] >= T) ? 1 : 0;
        cnt += sel[e];
      }
    } else {
      int tie = 0;
#pragma unroll
      for (int e = 0; e < kPerThread; ++e) tie += (ip + e < n && k[e] == T) ? 1 : 0;
      int tie_total;
      int tie_rank = ties_before + block_excl_scan(tie, sScan, tie_total);
#pragma unroll
      for (int e = 0; e < kPerThread; ++e) {
        bool s2 = false;
        if (ip + e < n) {
          if (k[e] > T) s2 = true;
          else if (k[e] == T) { s2 = tie_rank < need; ++tie_rank; }
        }
        sel[e] = s2;
        cnt += sel[e];
      }
      ties_before += tie_total;
    }
    int out_total;
    int pos = out_before + block_excl_scan(cnt, sScan, out_total);
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) {
      if (sel[e] && pos < K) out[pos] = ip + e;
      pos += sel[e];
    }
    out_before += out_total;
  }
}

// ---- global index build ----------------------------------------------------------------
// Request-local top-k positions to global cache slots through the block table, once per
// step, for the decode calls of every layer to read in GLOBAL mode (the once-per-step
// sparse index build cached in the step's metadata, prhub vllm#43827 implementation
// breakdown 3).  Entries the decode path would mask (-1, out of the table, a page id outside
// the pool, a request out of range) become -1.
__global__ __launch_bounds__(256) void translate_kernel(const int32_t* __restrict__ idx,
                                                        const int32_t* __restrict__ row_req,
                                                        const int32_t* __restrict__ page_table,
                                                        int rows, int topk, int num_requests,
                                                        int max_pages, int ps_log2, int num_pages,
                                                        int32_t* __restrict__ out) {
  const long long e = (long long)blockIdx.x * 256 + threadIdx.x;
  if (e >= (long long)rows * topk) return;
  const int r = (int)(e / topk);
  const int t = idx[e];
  const int req = row_req[r];
  int slot = -1;
  if (t >= 0 && req >= 0 && req < num_requests && (t >> ps_log2) < max_pages) {
    const int pg = page_table[(size_t)req * max_pages + (t >> ps_log2)];
    if (pg >= 0 && pg < num_pages) slot = (pg << ps_log2) | (t & ((1 << ps_log2) - 1));
  }
  out[e] = slot;
}

}  // namespace

hipError_t launch_translate(const int32_t* idx, const int32_t* row_req, const int32_t* page_table,
                            int rows, int topk, int num_requests, int max_pages, int ps_log2,
                            int num_pages, int32_t* out, hipStream_t st) {
  const long long n = (long long)rows * topk;
  hipLaunchKernelGGL(translate_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, idx, row_req,
                     page_table, rows, topk, num_requests, max_pages, ps_log2, num_pages, out);
  return hipGetLastError();
}

hipError_t launch_indexer_logits(const IndexerLogitsArgs& a, int next_n, int num_requests, hipStream_t st) {
  if (a.slots < 1 || a.num_requests != num_requests) return hipErrorInvalidValue;
  const dim3 grid(a.slots);
  switch (next_n) {
    case 1: hipLaunchKernelGGL(indexer_logits_kernel<1>, grid, dim3(256), 0, st, a); break;
    case 2: hipLaunchKernelGGL(indexer_logits_kernel<2>, grid, dim3(256), 0, st, a); break;
    case 3: hipLaunchKernelGGL(indexer_logits_kernel<3>, grid, dim3(256), 0, st, a); break;
    case 4: hipLaunchKernelGGL(indexer_logits_kernel<4>, grid, dim3(256), 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_indexer_topk(const IndexerTopkArgs& a, int rows, hipStream_t st) {
  hipLaunchKernelGGL(indexer_topk_kernel, dim3(rows), dim3(kTopkThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace smla
