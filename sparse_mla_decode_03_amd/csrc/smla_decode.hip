// Fused top-k sparse MLA decode kernel for gfx950.
//
// One workgroup handles one (query row, split) pair with all H query heads, as
// ceil(H/32) waves of 32 heads each (for ragged batches, the next pair of a longest-first
// job list that the two scheduling kernels at the end of this file build on the device).
// Steps, in the order of the Triton decode path described on prhub sglang#24692 ("SM120
// support for DeepSeek-V4", implementation breakdown 2-3):
//   1. index translation + compaction: the row's top-k positions of this split are
//      turned into cache slots through the page table (the block-table translation of
//      prhub vllm#43477, key code excerpts: forward_mqa); -1 and out-of-range entries
//      are dropped, the surviving slots are packed densely into LDS (order kept);
//   2. per tile of 32 slots: the entries' bytes are copied from HBM straight into LDS
//      (global_load_lds, no registers held) while the previous tile is computed; FP8
//      entries are then dequantized (e4m3fn code x 2^(scale-127)) by the lane that
//      copied them into a bf16 tile K[32][576]; BF16 entries land in K directly;
//   3. QK: S^T[32 tokens][32 heads] per wave on bf16 MFMA 32x32x16, K rows as the A
//      operand, q (register resident) as B;
//   4. softmax in the exp2 domain against a per-head reference max taken at the first
//      tile (see kRestartLog2);
//   5. PV: O[32 heads][512] += P[32][32] V[32][512] on bf16 MFMA with P straight from
//      the QK accumulator registers and V read from the same K tile with LDS transpose
//      reads (no separate V^T copy);
//   6. epilogue: final output with the sink folded in, or the sink-free split partial.
#include <type_traits>

#include "sparse_mla.h"
#include "smla_device.h"
#include "smla_kernels.h"

namespace smla {

namespace {

constexpr int kT = 32;                  // tokens per tile (MFMA M dimension)
constexpr int kRowB = 1280;             // LDS bytes per latent row slot (1024 B of data + pad)
constexpr int kRopeOff = kT * kRowB / 2;   // rope region: [32][64] bf16 after the latent rows
constexpr int kTile = kRopeOff + kT * 64;  // bf16 per tile (45,056 bytes)
constexpr int kCMax = 2048;             // positions per split handled by one workgroup
// Slot list length: the copies run up to three tiles past the last one and the scale copies
// one tile further, so indices reach (kCMax / kT + 4) * kT - 1; the tail repeats a valid slot.
constexpr int kSlotLen = kCMax + 4 * kT;
constexpr int kDepth = 4;               // LDS operand loads kept in flight (QK)
constexpr int kDepthV = 3;              // LDS operand load pairs kept in flight (PV)
// Exponentials are taken against a per-head reference max fixed at the first tile, so P
// may exceed 1.  fp32 and bf16 hold P <= 2^64 without overflow (and the sum over 2048
// entries of P times a value below 2^50 stays inside fp32), so the reference stays put
// while no score exceeds it by more than 64 log2 units.  Beyond that the reference is
// raised to the tile's max and the workgroup repeats the pass over the row: where the
// tile's max is known before its exponentials (the first tile, a partial tile, a repeated
// pass) it is that max; in the steady state (exponentials first) it is read off the
// exponent of the head's largest probability, or is the reference plus 128 when that
// probability is +inf (a score past exp2's fp32 range against the reference).
constexpr float kRestartLog2 = 64.0f;
constexpr unsigned kRestartBits = 0x5F800000u;   // bit pattern of 2^kRestartLog2
constexpr unsigned kInfBits = 0x7F800000u;       // bit pattern of +inf

// K tile layout.  LDS serves 64 banks of 4 bytes: 16 lanes per cycle for 16-byte reads
// and 32 lanes per cycle for 8-byte (and transpose) reads.  Latent row r is 1024 contiguous
// bytes (64 chunks of 16 bytes) at lat_row_byte(r) = 1280 r + 16 pad(r), with
// pad(r) = 4 (r%4) + (r/4)%4.  A row slot is a multiple of 256 bytes, so a row starts on bank
// 4 pad(r), and both operand patterns are conflict free:
//   QK A operand: 16 consecutive rows at one chunk -> pad takes all 16 values, 16 different
//   4-bank groups;
//   PV transpose reads: 4 consecutive rows 4m..4m+3 x 64 bytes -> pads m, 4+m, 8+m, 12+m,
//   four disjoint 16-bank windows.
// Since each row is contiguous, a lane's operand addresses differ only by constants (one
// base register for all latent QK steps, two for PV).  Rope rows are 128 bytes (two per bank
// row) with the chunk XORed with (row/2)%8.  A chunk is 16 bytes (8 bf16 dims).
__device__ __forceinline__ int lat_pad(int row) { return ((row & 3) << 2) | ((row >> 2) & 3); }
__device__ __forceinline__ int lat_row_byte(int row) { return row * kRowB + 16 * lat_pad(row); }

// Cross-half reductions: lanes l and l ^ 32 hold the same head (other tokens); one
// permlane32 swap gives every lane both values.
__device__ __forceinline__ float max_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ unsigned umax_halves(unsigned x) {
  const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return max(r[0], r[1]);
}
__device__ __forceinline__ float sum_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Token position (0..31) held in accumulator register r (0..15) of lane group G (lane/32)
// by a 32x32 MFMA whose rows are tokens.
__device__ __forceinline__ int acc_row(int r, int G) { return 8 * (r >> 2) + 4 * G + (r & 3); }


// Per-configuration LDS and work split.  A tile is gathered by 64-lane DMA instructions
// that each fill 1 KB of LDS, of two kinds:
//   latent: FP8 instruction i (0..15) copies the 512 latent codes of tokens 2i, 2i+1 into
//           a raw staging area; BF16 instruction i (0..31) copies token i's 1024-byte
//           latent row straight into the K tile;
//   rope:   instruction r (0..3) copies the 128-byte rope rows of tokens 8r..8r+7.
// Wave w issues latent instructions w, w+NW, ... and rope instructions w, w+NW, ..., so
// the kind of every part is known at compile time.  FP8 tiles also need their 32 x 8
// scale bytes: one wave (the scale wave, NW-1) copies them into a shared ring, one tile
// ahead of the codes, and the other waves read them after the end-of-tile barrier.
// With three or more waves (one workgroup per CU) the K tile is double-buffered; with
// fewer, a single tile keeps the workgroup small enough for two per CU.
// FMT: 0 = BF16 pages, 1 = FP8 with UE8M0 group scales, 2 = per-tensor FP8 (576 codes per
// entry, contiguous; the tensor scale is folded into the softmax scale and the output).
template <int NW, int FMT>
struct Cfg {
  static constexpr int NL = FMT != 0 ? 16 : 32;         // latent instructions per tile
  static constexpr int RR = FMT == 2 ? 2 : 4;           // rope instructions per tile
  static constexpr int LP = (NL + NW - 1) / NW;         // latent parts per wave
  static constexpr int RP = (RR + NW - 1) / NW;         // rope parts per wave
  // Tiles in flight and K tile buffers.  FP8 stages raw bytes (NS stages) and dequantizes
  // into NK bf16 K tiles; BF16 copies into a ring of NS + 1 K tiles, or synchronously
  // (NS = 0) when the workgroup must stay small enough for two per CU.
  static constexpr bool BIG = NW >= 3;                  // one workgroup per CU
  static constexpr int NS = FMT != 0 ? (BIG ? 3 : 1) : (BIG ? 2 : 0);
  static constexpr int NK = FMT != 0 ? (BIG ? 2 : 1) : (BIG ? NS + 1 : 1);
  static constexpr int RAW_BYTES = FMT != 0 ? NS * 20 * 1024 : 16;
  static constexpr int SCL_BYTES = FMT == 1 ? (NS + 1) * 256 : 16;
  // copies every wave issues per tile at least (the scale wave one more)
  static constexpr int NMIN = NL / NW + RR / NW;
};

// NATIVE: the epilogue writes split partials in the merge's own format (write_partials 2)
// and nothing else; otherwise it writes the output or the documented partials.  BAL (with
// NATIVE): the balanced job list and rank-window splits (jobs set); a row of one split
// writes its output directly.  Separate instantiations, so that neither epilogue nor the
// balanced set-up changes another variant's register allocation.
template <int NW, int FMT, bool NATIVE, bool BAL>
__global__ __launch_bounds__(NW * 64) void decode_kernel(DecodeArgs a) {
  using C = Cfg<NW, FMT>;
  // load_slots(tile) reads up to index (tile + 1) * kT + kT - 1 (the scale copy of the next
  // tile), for tile <= kCMax / kT - 1 + max(NS, 1)
  static_assert((kCMax / kT + (C::NS > 1 ? C::NS : 1) + 1) * kT <= kSlotLen, "slot list too short");
  constexpr int NT = NW * 64;
  __shared__ __attribute__((aligned(16))) uint16_t sK[C::NK * kTile];
  __shared__ __attribute__((aligned(16))) uint8_t sRaw[C::RAW_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t sScl[C::SCL_BYTES];
  __shared__ int sSlots[kSlotLen];
  __shared__ int sWcnt[8 * NW];
  __shared__ int sRestart;
  // Balanced rows: what the direct output of a one-split row needs, kept in LDS from the
  // set-up to the epilogue so that it holds no registers through the tile loop
  struct EpiArgs {
    uint16_t* out;
    float* lse;
    const float* sinks;
    float out_scale;
    int one_split;
  };
  __shared__ EpiArgs sEpi;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int lane_id = lane;
  // wave-uniform, in an SGPR; the clamp tells the compiler its range
  const int wave = NW == 4 ? (int)((unsigned)__builtin_amdgcn_readfirstlane(tid >> 6) & 3u)
                           : __builtin_amdgcn_readfirstlane(tid >> 6);
  // Work item.  Positional splits: row blockIdx.x, positions [split * chunk, +chunk).
  // Balanced (jobs set): the dispatch index picks the next (row, split) job of a list ordered
  // longest first, so the longest work starts first and short jobs fill the tail; a row of
  // S_r splits gives each an equal share of its entries by rank (the last one takes the
  // rest), and a row of one split writes its output directly.  Dispatch slots past the job
  // count leave at once.
  int row, split, p0, p1;
  int lo = 0, hi = INT_MAX;   // ranks of the valid entries this split keeps
  int s_row = a.S;            // the row's split count
  if constexpr (BAL) {
    const long long L = blockIdx.x + (long long)blockIdx.y * gridDim.x;
    if (L >= (long long)*a.job_count) return;      // uniform: the whole workgroup leaves
    const int job = a.jobs[L];
    // the clamps keep any count, split count or job in bounds
    row = min(max(job & 0xFFFFFF, 0), a.R - 1);
    s_row = min(max(a.row_splits[row], 1), a.S);
    split = min((int)((unsigned)job >> 24), s_row - 1);
    const int n = min(max(a.row_count[row], 0), a.K);
    // 32-bit products suffice: split < 256 and n <= K <= 256 * kCMax (2^19)
    lo = (int)((unsigned)split * (unsigned)n / (unsigned)s_row);
    if (split < s_row - 1) hi = (int)((unsigned)(split + 1) * (unsigned)n / (unsigned)s_row);
    p0 = 0;
    p1 = a.K;
    if (tid == 0) sEpi = EpiArgs{a.out, a.lse, a.sinks, a.out_scale, s_row == 1};
  } else {
    row = blockIdx.x;
    split = blockIdx.y;
    p0 = split * a.chunk;
    p1 = min(p0 + a.chunk, a.K);
  }
  const int ps_mask = (1 << a.ps_log2) - 1;
  if (tid == 0) sRestart = 0;

  // ---- 1a. the loads of the index translation come first: the split's first batch of
  // indices and the request's page-table row (into LDS, borrowed from the K buffers, when
  // it has at most kPtPer * NT entries), so their use below does not wait for q ----
  int req = 0;
  bool req_ok = true;
  if (a.index_mode == 0) {
    req = a.row_req[row];
    req_ok = req >= 0 && req < a.B;
  }
  constexpr int kCB = 8;
  constexpr int kPtPer = 8;
  int* sPt = reinterpret_cast<int*>(sK);
  // typed LDS view for the lookups, so they stay LDS reads (a pointer that may be LDS or
  // global would become a flat load, whose wait also covers the q loads)
  const __attribute__((address_space(3))) int* sPtL = (const __attribute__((address_space(3))) int*)(sPt);
  const bool pt_lds = a.index_mode == 0 && req_ok && a.max_pages <= kPtPer * NT;   // uniform
  int tv0[kCB];
#pragma unroll
  for (int i = 0; i < kCB; ++i) {
    const int p = p0 + i * NT + tid;
    tv0[i] = p < p1 ? a.indices[(size_t)row * a.K + p] : -1;
  }
  int ptv[kPtPer];
  if (pt_lds) {
#pragma unroll
    for (int j = 0; j < kPtPer; ++j) {
      const int e = j * NT + tid;
      ptv[j] = e < a.max_pages ? a.page_table[(size_t)req * a.max_pages + e] : -1;
    }
  }

  // ---- q fragments: lane holds head 32*wave + lane%32, dims 16*ks + 8*(lane/32) + 0..7
  // (padded heads read a real head's q; their results are never written).  Their latency
  // overlaps the index translation.
  const int hl = lane & 31;
  const int G = lane >> 5;
  const int h = wave * 32 + hl;
  const bool h_ok = h < a.H;
  u32x4 qf[36];
  {
    const uint16_t* qp = a.q + ((size_t)row * a.H + min(h, a.H - 1)) * kQK + 8 * G;
#pragma unroll
    for (int ks = 0; ks < 36; ++ks) qf[ks] = *reinterpret_cast<const u32x4*>(qp + 16 * ks);
  }
  if (pt_lds) {
#pragma unroll
    for (int j = 0; j < kPtPer; ++j)
      if (j * NT + tid < a.max_pages) sPt[j * NT + tid] = ptv[j];
  }
  __syncthreads();

  // ---- 1. translate and compact the split's indices --------------------------------
  // Positions are taken in batches of kCB per thread; all index loads of a batch, then all
  // its page-table loads (LDS reads when the row is staged), are in flight together.
  int n_valid = 0;
  for (int base = p0; base < p1; base += kCB * NT) {
    int tv[kCB];
#pragma unroll
    for (int i = 0; i < kCB; ++i) {
      const int p = base + i * NT + tid;
      tv[i] = base == p0 ? tv0[i] : (p < p1 ? a.indices[(size_t)row * a.K + p] : -1);
    }
    int slot[kCB];
    bool ok[kCB];
    if (a.index_mode == 0) {
#pragma unroll
      for (int i = 0; i < kCB; ++i) {
        ok[i] = req_ok && tv[i] >= 0 && (tv[i] >> a.ps_log2) < a.max_pages;
        slot[i] = 0;
      }
      // the page of each position for now; each branch consumes its own loads (the empty
      // asm), so no wait after the join has to cover both kinds of load
      if (pt_lds) {
#pragma unroll
        for (int i = 0; i < kCB; ++i)
          if (ok[i]) slot[i] = sPtL[tv[i] >> a.ps_log2];
#pragma unroll
        for (int i = 0; i < kCB; ++i) asm volatile("" : "+v"(slot[i]));
      } else {
#pragma unroll
        for (int i = 0; i < kCB; ++i)
          if (ok[i]) slot[i] = a.page_table[(size_t)req * a.max_pages + (tv[i] >> a.ps_log2)];
#pragma unroll
        for (int i = 0; i < kCB; ++i) asm volatile("" : "+v"(slot[i]));
      }
    } else {
#pragma unroll
      for (int i = 0; i < kCB; ++i) {
        ok[i] = tv[i] >= 0 && tv[i] < a.num_slots;
        slot[i] = tv[i];
      }
    }
    unsigned long long m[kCB];
#pragma unroll
    for (int i = 0; i < kCB; ++i) {
      const int t = tv[i];
      if (a.index_mode == 0 && ok[i]) {
        const int pg = slot[i];
        ok[i] = pg >= 0 && pg < a.num_pages;
        slot[i] = (pg << a.ps_log2) | (t & ps_mask);
      }
      if (t != -1 && !ok[i] && a.err != nullptr) {
        const int p = base + i * NT + tid;
        atomicMin(a.err, ((unsigned long long)(unsigned)row << 32) | (unsigned)p);
      }
      m[i] = __ballot(ok[i]);
      if (lane == 0) sWcnt[i * NW + wave] = __popcll(m[i]);
    }
    __syncthreads();
    // slots keep position order: batch i, then wave, then lane
    int off = n_valid;
#pragma unroll
    for (int i = 0; i < kCB; ++i) {
      int before_w = 0, tot = 0;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const int c = sWcnt[i * NW + w];
        before_w += (w < wave) ? c : 0;
        tot += c;
      }
      const int before = __builtin_amdgcn_mbcnt_hi((unsigned)(m[i] >> 32),
                                                   __builtin_amdgcn_mbcnt_lo((unsigned)m[i], 0u));
      if constexpr (BAL) {
        // the split's rank window; the slot list bound holds whatever the counts say
        const int at = off + before_w + before - lo;
        if (ok[i] && at >= 0 && at < hi - lo && at < kCMax) sSlots[at] = slot[i];
      } else {
        if (ok[i]) sSlots[off + before_w + before] = slot[i];
      }
      off += tot;
    }
    n_valid = off;
    __syncthreads();
    if (BAL && off >= hi) break;     // block uniform: the split's share is complete
  }
  if constexpr (BAL) n_valid = min(max(n_valid - lo, 0), min(hi - lo, kCMax));
  // Positions past the valid count repeat the split's first valid slot, so the copies of
  // the last tile and of the tiles past the end need no per-lane selection and bring in
  // finite data (a valid entry of this very split) that meets a masked score, P = 0.
  {
    const int first = n_valid > 0 ? sSlots[0] : 0;
    __syncthreads();
    for (int i = n_valid + tid; i < kSlotLen; i += NT) sSlots[i] = first;
    __syncthreads();
  }
  // land q before the tile copies start, so no wait on them is placed at its first use
  // inside the loop
  wait_vm();

  float m_used = -INFINITY;
  bool have_ref = false;   // some tile has set m_used (block uniform)
  bool careful = false;    // a repeated pass: every tile checks its max before the exps

  // ---- 2. gather (see Cfg for the DMA instruction map).  Every DMA instruction of a
  // tile is issued, also for tokens past the valid count (they read a dummy address in
  // the cache and are zeroed when the tile is finished), so that the number of pending
  // copies per wave is fixed and vmcnt waits can target the oldest tile.  A tile's copy
  // is split in two steps: its slots are read from LDS into registers first (load_slots),
  // and the copies are issued one phase later (issue_dma), so no LDS round trip sits in
  // front of each copy.
  constexpr int LP = C::LP, RP = C::RP;
  constexpr int NDMA = LP + RP + (FMT == 1 ? 1 : 0);   // slot registers (scales last)
  // recomputed from the wave index where needed (cheaper than keeping the flag live)
  auto scale_wave = [&]() { return FMT == 1 && __builtin_amdgcn_readfirstlane(tid >> 6) == NW - 1; };
  auto lat_token = [&](int ins, int ln) { return FMT != 0 ? 2 * ins + (ln >> 5) : ins; };
  // a rope instruction covers 8 tokens (128 bytes each) or, per-tensor FP8, 16 (64 bytes)
  auto rope_token = [&](int ins, int ln) { return FMT == 2 ? 16 * ins + (ln >> 2) : 8 * ins + (ln >> 3); };
  auto load_slots = [&](int tile, int (&sl)[NDMA]) {
    int ln = lane_id;
    asm volatile("" : "+v"(ln));
    const int t0 = tile * kT;
    // positions past the valid count read the split's first valid slot
#pragma unroll
    for (int j = 0; j < LP; ++j) sl[j] = sSlots[t0 + lat_token(min(wave + NW * j, C::NL - 1), ln)];
#pragma unroll
    for (int j = 0; j < RP; ++j) sl[LP + j] = sSlots[t0 + rope_token(min(wave + NW * j, C::RR - 1), ln)];
    // the scale wave copies the scales of the following tile
    if (FMT == 1) sl[LP + RP] = sSlots[t0 + kT + (ln >> 1)];
  };
  // FP8 byte offset of a region of a slot's page: page * (648 << ps_log2) + add, with the
  // 32-bit page stride (at most 648 KB) in one 32 x 32 -> 64-bit multiply-add
  const uint32_t fp8_stride = (uint32_t)kFp8Entry << a.ps_log2;
  auto fp8_off = [&](uint32_t slot, uint32_t add) {
    return (size_t)((uint64_t)(slot >> a.ps_log2) * fp8_stride + add);
  };
  auto fp8_row = [&](uint32_t slot) { return slot & ((1u << a.ps_log2) - 1u); };
  // Copy part j of `tile`: latent parts 0..LP-1, rope parts LP..LP+RP-1, then (scale wave
  // only) the scales of tile + 1.  `ln` is an opaque copy of the lane id: the per-lane
  // address terms are recomputed at each part instead of being hoisted out of the tile loop
  // (which costs registers, then spills whose reloads would wait on the copies).
  // LDS byte addresses of the copy destinations (wave-uniform, in SGPRs)
  const uint32_t lds_k = lds_offset(sK), lds_raw = lds_offset(sRaw), lds_scl = lds_offset(sScl);
  auto issue_part = [&](int tile, int j, const int (&sl)[NDMA], int ln) {
    const int st = C::NS > 0 ? tile % (FMT != 0 ? C::NS : C::NK) : 0;
    const uint32_t K = lds_k + (FMT != 0 ? 0 : st) * (2 * kTile);
    const uint32_t raw = lds_raw + (FMT != 0 ? st : 0) * (20 * 1024);
    if (j < LP) {
      const int ins = wave + NW * j;
      if (ins < C::NL) {
        const int t = lat_token(ins, ln);
        const uint32_t slot = (uint32_t)sl[j];
        size_t off;
        uint32_t dst;
        if (FMT == 1) {
          off = fp8_off(slot, fp8_row(slot) * 512u + 16u * (ln & 31));
          dst = raw + ins * 1024;
        } else if (FMT == 2) {
          off = (size_t)slot * kQK + 16u * (ln & 31);
          dst = raw + ins * 1024;
        } else {
          // lane = chunk of the destination row
          off = (size_t)slot * kBf16Entry + 16u * ln;
          dst = K + lat_row_byte(t);
        }
        dma16_at(a.kv + off, dst);
      }
    } else if (j < LP + RP) {
      const int ins = wave + NW * (j - LP);
      if (ins < C::RR) {
        const int t = rope_token(ins, ln);
        const uint32_t slot = (uint32_t)sl[j];
        size_t off;
        uint32_t dst;
        if (FMT == 1) {
          off = fp8_off(slot, (512u << a.ps_log2) + fp8_row(slot) * 128u + 16u * (ln & 7));
          dst = raw + (16 + ins) * 1024;
        } else if (FMT == 2) {
          off = (size_t)slot * kQK + 512u + 16u * (ln & 3);
          dst = raw + (16 + ins) * 1024;
        } else {
          off = (size_t)slot * kBf16Entry + 1024u + 16u * ((ln & 7) ^ ((t >> 1) & 7));
          dst = K + 2 * kRopeOff + ins * 1024;
        }
        dma16_at(a.kv + off, dst);
      }
    } else if (scale_wave()) {
      // scales of tile + 1: lane l copies 4 bytes of token l/2
      const uint32_t slot = (uint32_t)sl[LP + RP];
      const size_t off = fp8_off(slot, (640u << a.ps_log2) + fp8_row(slot) * 8u + 4u * (ln & 1));
      dma4_at(a.kv + off, lds_scl + ((tile + 1) % (C::NS + 1)) * 256);
    }
  };
  auto issue_dma = [&](int tile, const int (&sl)[NDMA]) {
    int ln = lane_id;
    asm volatile("" : "+v"(ln));
#pragma unroll
    for (int j = 0; j < NDMA; ++j) issue_part(tile, j, sl, ln);
  };
  // The scales of tile 0 (FP8), copied by the scale wave before anything else.
  auto issue_first_scales = [&]() {
    if (!scale_wave()) return;
    int ln = lane_id;
    asm volatile("" : "+v"(ln));
    const uint32_t slot = (uint32_t)sSlots[ln >> 1];
    const size_t off = fp8_off(slot, (640u << a.ps_log2) + fp8_row(slot) * 8u + 4u * (ln & 1));
    dma4_at(a.kv + off, lds_scl);
  };
  // Wait for the oldest tile in flight; the NS - 1 younger ones may stay pending.
  // A wave issues one group of copies per tile (its parts of tile + NS, in issue order).
  // Counting from the newest, at most `keep` groups may stay pending; vmcnt completes in
  // issue order, so everything older has landed.  The scale wave's groups are one copy
  // longer (the scales); waves issuing more than NMIN copies per group wait for a few of
  // their newest copies as well, which is harmless.
  auto wait_groups = [&](auto keep) {
    constexpr int kKeep = decltype(keep)::value;
    if constexpr (kKeep <= 0) {
      wait_vm();
    } else {
      if (scale_wave())
        wait_vm_le<kKeep * (C::NMIN + 1)>();
      else
        wait_vm_le<kKeep * C::NMIN>();
    }
  };
  // After this wave's group for tile + NS is issued: tile + 1 has landed.
  auto wait_oldest = [&]() { wait_groups(std::integral_constant<int, C::NS - 1>{}); };
  // Before this wave's group for tile + NS is issued: tile + 1 has landed.
  auto wait_next = [&]() { wait_groups(std::integral_constant<int, C::NS - 2>{}); };

  auto kbuf_of = [&](int tile) { return C::NK > 1 ? tile % C::NK : 0; };
  // FP8 dequantization of one part is split into a load step (the lane's raw unit and its
  // scale byte from LDS) and a write step, so the parts can be spread over the MFMAs with
  // each load a few MFMAs ahead of its write.  All addresses are a per-tile lane base plus
  // wave-uniform terms: for latent instruction i the unit of token t = 2i + G, dims
  // 16c..16c+15 (c = lane % 32) goes to chunks 2c and 2c + 1 of row t, at byte
  // lat_row_byte(2i + G) + 32c = 1344 G + 32c + U(i) with U(i) = 2560 i + 128 (i % 2) +
  // 16 ((i / 2) % 4) (pad(2i + G) = 8 (i % 2) + 4G + (i / 2) % 4); rope instruction r
  // puts token 8r + lane / 8, chunk lane % 8, at chunk (lane % 8) ^ (lane / 16) ^ 4(r % 2);
  // per-tensor FP8 rope instruction r holds token 16r + lane / 4, codes 16(lane % 4) .. +15,
  // converted to logical chunks 2(lane % 4) and 2(lane % 4) + 1 of the token's rope row.
  // The lanes with bit 2 of c set convert and write the second 16-byte half of their
  // unit first (they load the two 8-byte halves of the raw unit swapped).  A 16-byte LDS
  // write is served eight lanes at a time against 128 bytes of banks: units c and c + 4
  // start 128 bytes apart, so with the swap each group of eight lanes writes eight
  // different 16-byte bank slots.
  struct DqBase {
    int raw;    // byte offset into sRaw of the half of this lane's unit written first
    int scl;    // byte offset into sScl of this lane's scale byte for instruction `wave`
    int lat;    // lane part of the latent write offset (first half)
    int rope;   // lane part of the rope write offset (bits 4..9)
    int kb;     // byte offset of the destination K buffer
  };
  auto dq_base = [&](int tile, int ln) {
    DqBase d;
    const int G_ = ln >> 5, c = ln & 31;
    d.raw = (C::NS > 0 ? tile % C::NS : 0) * (20 * 1024) + wave * 1024 + 16 * ln + 8 * ((c >> 2) & 1);
    d.scl = (tile % (C::NS + 1)) * 256 + 16 * wave + 8 * G_ + (c >> 2);
    d.lat = (kRowB + 64) * G_ + 32 * c + 16 * ((c >> 2) & 1);
    d.rope = FMT == 2 ? 128 * (ln >> 2) + 16 * ((2 * (ln & 3)) ^ ((ln >> 3) & 7))
                      : 128 * (ln >> 3) + 16 * ((ln & 7) ^ (ln >> 4));
    d.kb = 2 * kbuf_of(tile) * kTile;
    return d;
  };
  struct RawUnit {
    u32x4 rv;
    uint32_t e;
  };
  auto finish_load = [&](int j, const DqBase& d) {
    RawUnit u;
    if (j < LP) {
      const u32x2 first = *reinterpret_cast<const u32x2*>(sRaw + d.raw + NW * j * 1024);
      const u32x2 second = *reinterpret_cast<const u32x2*>(sRaw + (d.raw ^ 8) + NW * j * 1024);
      u.rv = u32x4{first[0], first[1], second[0], second[1]};
      u.e = FMT == 1 ? (uint32_t)sScl[d.scl + 16 * NW * j] : 127u;   // per-tensor FP8: scale 1
    } else {
      u.rv = *reinterpret_cast<const u32x4*>(sRaw + (d.raw & ~15) + (16 + NW * (j - LP)) * 1024);
      u.e = 0u;
    }
    return u;
  };
  auto finish_part = [&](int j, const RawUnit& u, const DqBase& d) {
    uint8_t* Kb = reinterpret_cast<uint8_t*>(sK) + d.kb;
    if (j < LP) {
      const int ins = wave + NW * j;
      if (ins < C::NL) {
        const int U = 2 * kRowB * ins + 128 * (ins & 1) + 16 * ((ins >> 1) & 3);
        const float sc = ue8m0_scale(u.e);
        *reinterpret_cast<u32x4*>(Kb + U + d.lat) = dequant8_fp8(u32x2{u.rv[0], u.rv[1]}, sc);
        *reinterpret_cast<u32x4*>(Kb + U + (d.lat ^ 16)) = dequant8_fp8(u32x2{u.rv[2], u.rv[3]}, sc);
      }
    } else if (FMT == 2) {
      const int r = wave + NW * (j - LP);
      if (r < C::RR) {
        uint8_t* dst = Kb + 2 * kRopeOff + 2048 * r;
        *reinterpret_cast<u32x4*>(dst + d.rope) = dequant8_fp8(u32x2{u.rv[0], u.rv[1]}, 1.0f);
        *reinterpret_cast<u32x4*>(dst + (d.rope ^ 16)) = dequant8_fp8(u32x2{u.rv[2], u.rv[3]}, 1.0f);
      }
    } else {
      const int r = wave + NW * (j - LP);
      if (r < 4) *reinterpret_cast<u32x4*>(Kb + 2 * kRopeOff + 1024 * r + (d.rope ^ (64 * (r & 1)))) = u.rv;
    }
  };
  // One quarter q of latent part j: the bf16 pairs of raw dword q go to `half`; after the
  // odd quarters a 16-byte half of the unit is written.
  auto finish_quarter = [&](int j, int q, const RawUnit& u, u32x4& half, const DqBase& d) {
    const int ins = wave + NW * j;
    if (ins < C::NL) {
      const float sc = ue8m0_scale(u.e);
      half[2 * (q & 1)] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(u.rv[q], sc, false));
      half[2 * (q & 1) + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(u.rv[q], sc, true));
      if (q & 1) {
        uint8_t* Kb = reinterpret_cast<uint8_t*>(sK) + d.kb;
        const int U = 2 * kRowB * ins + 128 * (ins & 1) + 16 * ((ins >> 1) & 3);
        *reinterpret_cast<u32x4*>(Kb + U + (q == 3 ? d.lat ^ 16 : d.lat)) = half;
      }
    }
  };
  // After this lane's copies of `tile` have landed: FP8 dequantizes the units it copied
  // into the tile's K buffer.  (BF16 copies land in the K buffer directly.)
  auto finish_tile = [&](int tile) {
    if (FMT != 0) {
      int ln = lane_id;
      asm volatile("" : "+v"(ln));
      const DqBase d = dq_base(tile, ln);
      RawUnit u[LP + RP];
#pragma unroll
      for (int j = 0; j < LP + RP; ++j) u[j] = finish_load(j, d);
#pragma unroll
      for (int j = 0; j < LP + RP; ++j) finish_part(j, u[j], d);
    }
  };

  // Lane parts of the LDS operand addresses.
  //   QK step ks < 32 (bytes): chunk 2ks + G of row hl -> qk_base + 32 ks;
  //   QK rope step 32 + i (bf16 elements): (rope_base ^ 16i);
  //   PV (bytes; see the B-operand note in the loop): row 16 s2 + 8 hh + 4G + j/4, columns
  //   32b + 16 (gamma % 2) + 4 (j % 4) -> pv_base(hh) + 1280 (16 s2 + 8 hh) + 64 b, where the
  //   row's pad 4 (j/4) + (2 hh + G) % 4 depends on hh.
  auto qk_base_of = [&](int ln) {
    const int hl_ = ln & 31, G_ = ln >> 5;
    return lat_row_byte(hl_) + 16 * G_;
  };
  auto rope_base_of = [&](int ln) {
    const int hl_ = ln & 31, G_ = ln >> 5;
    return kRopeOff + hl_ * 64 + ((G_ ^ ((hl_ >> 1) & 7)) << 3);
  };
  auto pv_base_of = [&](int ln, int hh) {
    const int pj = ln & 15, G_ = ln >> 5, jq = pj >> 2, gam = (ln >> 4) & 1;
    return (4 * G_ + jq) * kRowB + 16 * (4 * jq + ((2 * hh + G_) & 3)) + 32 * gam + 8 * (pj & 3);
  };

  // O blocks are accumulated by compiler-scheduled MFMAs in AGPRs.  With three or four
  // waves, block 15 instead lives in VGPRs (a VGPR-form MFMA): that leaves 16 AGPRs for the
  // QK scores, so no O block has to be moved out of the accumulation registers and back each
  // tile.  (Smaller workgroups keep more copy registers live and stay all-AGPR.)  The
  // compiler does not see that MFMA's latency: until mfma_vgpr_drain() after the tile loop
  // no other instruction may name O15's registers.  The library build checks this on the
  // compiled assembly, over every control-flow path, and refuses a build that breaks it.
  constexpr bool kO15V = NW >= 3;
  f32x16 O[kO15V ? 15 : 16];
  f32x16 O15;
  // array slot of an AGPR block (block 15 never reaches it when it lives in VGPRs)
  auto ob_index = [&](int b) { return kO15V ? b % 15 : b; };
  float l_part;
  // O and the row sum times alpha (per head: this lane's column), for a raised reference
  const int ntiles = (n_valid + kT - 1) / kT;
  // The pass over the tiles is repeated only if some head's reference max had to be
  // raised (kRestartLog2); O is dead across the repeat.
  for (;;) {
#pragma unroll
  for (int b = 0; b < (kO15V ? 15 : 16); ++b) O[b] = f32x16{};
  O15 = f32x16{};
  l_part = 0.f;
  if (ntiles > 0) {
    if (FMT == 1) issue_first_scales();
    if (C::NS > 0) {
#pragma unroll
      for (int i = 0; i < C::NS; ++i) {
        int sl[NDMA];
        load_slots(i, sl);
        issue_dma(i, sl);
      }
      wait_oldest();
    } else {
      int sl[NDMA];
      load_slots(0, sl);
      issue_dma(0, sl);
      wait_vm();
    }
    if (FMT == 1) __syncthreads();   // the scale wave's copy of tile 0's scales is visible
    finish_tile(0);
  }
  __syncthreads();

  bool restart = false;
  for (int tile = 0; tile < ntiles; ++tile) {
    const int t0 = tile * kT;
    const int nt = min(kT, n_valid - t0);
    const bool has_next = tile + 1 < ntiles;
    // With two K buffers and FP8, the dequantization of tile + 1 into the other buffer is
    // spread over the QK MFMAs of this tile (QK leaves LDS bandwidth to spare, PV does
    // not); its copies have landed after wait_next (this tile's own group of copies is
    // issued inside QK, after the wait).  Past the last tile this converts the copies of
    // positions past the end into a buffer nobody reads.
    constexpr bool kWeave = FMT != 0 && C::NK > 1;
    constexpr bool kFine = (LP + RP) * 6 <= 36 && (C::NS == 0 || 1 + 6 * (NDMA - 1) < 36);
    if (kWeave) wait_next();
    // slots of the tile copied during this one
    int sl[NDMA];
    if (C::NS > 0) load_slots(tile + C::NS, sl);

    // ---- 3. QK: S^T[token][head]; lane holds head hl, tokens acc_row(r, G) -------------
    // The A operand (K rows) is software pipelined kDepth loads ahead; scheduling fences
    // keep the compiler from hoisting more loads than that into registers.
    f32x16 s = f32x16{};
    {
      int ln = lane_id;
      asm volatile("" : "+v"(ln));
      // byte offsets into sK of the latent and the four rope lane bases of this tile's
      // buffer, opaque to the compiler so each load is one LDS instruction with a constant
      // offset
      const int kbytes = 2 * kbuf_of(tile) * kTile;
      int qoff = kbytes + qk_base_of(ln), roff[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) roff[i] = kbytes + 2 * (rope_base_of(ln) ^ (16 * i));
      asm volatile("" : "+v"(qoff));
#pragma unroll
      for (int i = 0; i < 4; ++i) asm volatile("" : "+v"(roff[i]));
      auto kload = [&](int ks) {
        const int off = ks < 32 ? qoff + 32 * ks : roff[ks - 32];
        return *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint8_t*>(sK) + off);
      };
      u32x4 kq[kDepth];
      RawUnit un;
      u32x4 half;
      const DqBase dq = dq_base(tile + 1, ln);
#pragma unroll
      for (int i = 0; i < kDepth; ++i) kq[i] = kload(i);
#pragma unroll
      for (int ks = 0; ks < 36; ++ks) {
        const u32x4 kv = kq[ks % kDepth];
        if (ks + kDepth < 36) kq[ks % kDepth] = kload(ks + kDepth);
        s = mfma32x32x16(kv, qf[ks], s);
        // the copies of tile + NS are spread over the QK MFMAs, one part every few
        // steps, so that the waves' copies reach the memory pipeline evenly
        if (C::NS > 0) {
#pragma unroll
          for (int j = 0; j < NDMA; ++j)
            if (ks == (kFine ? 1 + 6 * j : 2 + (j * 33) / NDMA)) issue_part(tile + C::NS, j, sl, ln);
        }
        // dequantization part j of tile + 1.  With few parts per wave (kFine) each latent
        // part is loaded at step 6j and converted a quarter per step at 6j+2 .. 6j+5, so
        // no step carries more than two conversions beside its MFMA; the copies sit on the
        // steps between.  Otherwise a part is loaded two MFMAs before it is written.
        if (kWeave) {
#pragma unroll
          for (int j = 0; j < LP + RP; ++j) {
            if constexpr (kFine) {
              if (ks == 6 * j) un = finish_load(j, dq);
              if (j < LP) {
#pragma unroll
                for (int q = 0; q < 4; ++q)
                  if (ks == 6 * j + 2 + q) finish_quarter(j, q, un, half, dq);
              } else if (ks == 6 * j + 2) {
                finish_part(j, un, dq);
              }
            } else {
              if (ks == 3 + (j * 30) / (LP + RP)) un = finish_load(j, dq);
              if (ks == 5 + (j * 30) / (LP + RP)) finish_part(j, un, dq);
            }
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }

    // PV B-operand: dv block b, k-step s2: lane l needs V[acc_row(8*s2 + kk, G)][32b + l%32]
    // for kk = 0..7.  Two transpose reads give kk 0..3 and 4..7: in each 16-lane group
    // (gamma = l/16, j = l%16) lane j addresses row 16*s2 + 8*hh + 4*G + j/4 at columns
    // 32b + 16*(gamma%2) + 4*(j%4) .. +3.
    int pln = lane_id;
    asm volatile("" : "+v"(pln));
    // byte offsets into sK of the two lane bases (hh), opaque as for QK
    int poff[2];
    {
      const int kbytes = 2 * kbuf_of(tile) * kTile;
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) poff[hh] = kbytes + pv_base_of(pln, hh);
#pragma unroll
      for (int i = 0; i < 2; ++i) asm volatile("" : "+v"(poff[i]));
    }
    // PV steps run k-step major: step = 16 * s2 + b
    auto vaddr = [&](int step, int hh) {
      const int b = step & 15, s2 = step >> 4;
      return reinterpret_cast<const uint16_t*>(reinterpret_cast<const uint8_t*>(sK) + poff[hh] +
                                               kRowB * (16 * s2 + 8 * hh) + 64 * b);
    };
    u32x2 vq[kDepthV][2];
#pragma unroll
    for (int i = 0; i < kDepthV; ++i) {
      vq[i][0] = lds_read_tr16(vaddr(i, 0));
      vq[i][1] = lds_read_tr16(vaddr(i, 1));
    }
    // O^T[dv][head] += V^T[dv][token] P^T[token][head]: the V registers are the A operand
    // (rows = dv) and P the B operand (columns = heads), so each lane's accumulator holds
    // one head and runs of four consecutive dv.
    auto pv_step = [&](int step, const u32x4& p) {
      const u32x2 v0 = vq[step % kDepthV][0];
      const u32x2 v1 = vq[step % kDepthV][1];
      if (step + kDepthV < 32) {
        vq[step % kDepthV][0] = lds_read_tr16(vaddr(step + kDepthV, 0));
        vq[step % kDepthV][1] = lds_read_tr16(vaddr(step + kDepthV, 1));
      }
      const u32x4 va = u32x4{v0[0], v0[1], v1[0], v1[1]};
      if (kO15V && (step & 15) == 15)
        mfma32x32x16_vgpr(va, p, O15);
      else
        O[ob_index(step & 15)] = mfma32x32x16(va, p, O[ob_index(step & 15)]);
    };
    auto pack8 = [&](int s2) {
      return u32x4{pack_bf16x2(s[8 * s2 + 0], s[8 * s2 + 1]), pack_bf16x2(s[8 * s2 + 2], s[8 * s2 + 3]),
                   pack_bf16x2(s[8 * s2 + 4], s[8 * s2 + 5]), pack_bf16x2(s[8 * s2 + 6], s[8 * s2 + 7])};
    };

    // ---- 4./5. softmax (exp2 domain) against a per-head reference max m_used, and PV ---
    // P as the PV B operand: k-step s2 uses the lane's tokens acc_row(8*s2 + kk, G).
    // Each probability is exp2(fma(x, ce, -me)).  In the steady state (a full tile, a
    // reference from earlier tiles, a positive scale) x is the raw score, ce the scale
    // and me the reference, and nothing precedes the exps: k-step 0's probabilities come
    // first and the rest of the softmax (k-step 1's probabilities, the row sum, the
    // overflow check) runs inside k-step 0's MFMAs.  A probability above 2^kRestartLog2
    // means a score far beyond the reference: the pass is repeated (see kRestartLog2).
    // Otherwise (the first tile, a partial tile, a repeated pass) the tile's max is taken
    // first and may raise the reference; x is then the scaled, masked score minus the
    // reference, with ce = 1 and me = 0.
    const bool steady = have_ref && !careful && nt == kT && a.scale_log2 > 0.f;   // uniform
    float ce = a.scale_log2, me = m_used;
    if (!steady) {
      float mx;
      const bool full = nt == kT && a.scale_log2 > 0.f;   // wave uniform
      if (full) {
        float m8[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) m8[r] = fmaxf(s[2 * r], s[2 * r + 1]);
        mx = fmaxf(fmaxf(fmaxf(m8[0], m8[1]), fmaxf(m8[2], m8[3])), fmaxf(fmaxf(m8[4], m8[5]), fmaxf(m8[6], m8[7])));
        mx *= a.scale_log2;
      } else {
        mx = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          s[r] = (acc_row(r, G) < nt) ? s[r] * a.scale_log2 : -INFINITY;
          mx = fmaxf(mx, s[r]);
        }
      }
      mx = max_halves(mx);
      if (m_used == -INFINITY) m_used = mx;       // first tile: O and l are still zero
      if (mx > m_used + kRestartLog2) {           // rare: raise the reference and repeat
        m_used = mx;
        sRestart = 1;
      }
      if (full) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[r] = __builtin_fmaf(s[r], a.scale_log2, -m_used);
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[r] = s[r] - m_used;    // -inf stays -inf
      }
      ce = 1.f;
      me = 0.f;
    }
#pragma unroll
    for (int r = 0; r < 8; ++r) s[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], ce, -me));
    const u32x4 p0 = pack8(0);
    u32x4 p1;
    unsigned pbits = 0;
#pragma unroll
    for (int step = 0; step < 16; ++step) {
      pv_step(step, p0);
      if (step < 8) s[8 + step] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[8 + step], ce, -me));
      if (step == 8) p1 = pack8(1);
      if (step == 10) {
        float p8[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) p8[r] = s[2 * r] + s[2 * r + 1];
        l_part += ((p8[0] + p8[1]) + (p8[2] + p8[3])) + ((p8[4] + p8[5]) + (p8[6] + p8[7]));
      }
      if (step == 12) {
        // probabilities are >= 0, so their bit patterns order like their values
#pragma unroll
        for (int r = 0; r < 16; ++r) pbits = max(pbits, __float_as_uint(s[r]));
      }
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int step = 16; step < 32; ++step) {
      pv_step(step, p1);
      __builtin_amdgcn_sched_barrier(0);
    }
    // A head's largest probability above 2^kRestartLog2 repeats the pass, with the
    // reference raised by the probability's exponent (by 128 for +inf).  NaN, whose
    // patterns lie above +inf's, does not: a NaN score must not repeat the pass.
    if (steady) {
      const unsigned hb = umax_halves(pbits);
      if (hb > kRestartBits && hb <= kInfBits) {
        m_used += hb < kInfBits ? (float)((int)(hb >> 23) - 127) : 128.f;
        sRestart = 1;
      }
    }
    have_ref = true;

    // ---- next tile: finish its gather -------------------------------------------------
    if (has_next) {
      if (C::NK > 1) {
        if (!kWeave) {
          wait_oldest();
          finish_tile(tile + 1);
        }
      } else {
        __syncthreads();                 // everyone is done reading the single K tile
        if (C::NS == 0) {
          int sl1[NDMA];
          load_slots(tile + 1, sl1);
          issue_dma(tile + 1, sl1);
          wait_vm();
        } else {
          wait_oldest();
        }
        finish_tile(tile + 1);
      }
    }
    __syncthreads();
    if (sRestart) {  // the same value in every thread: it was written before the barrier
      restart = true;
      careful = true;
      break;
    }
  }
  wait_vm();  // drain the copies issued past the last tile
  if (kO15V) mfma_vgpr_drain();
  if (!restart) break;
  __syncthreads();  // every thread has seen the flag
  if (tid == 0) sRestart = 0;
  }

  // ---- 6. epilogue ----------------------------------------------------------------------
  const float l_tot = sum_halves(l_part);
  if constexpr (NATIVE) {
    if (BAL && sEpi.one_split) {
      // A balanced row of one split: the output itself, sink folded in, straight from the
      // accumulators (lane: head h, dv 32b + 8k + 4G + 0..3 as one 8-byte bf16 piece; the
      // wave's two lane halves complete each 16-byte piece, and its stores whole head rows)
      const EpiArgs e = sEpi;
      const float sink = (e.sinks != nullptr && h_ok) ? e.sinks[h] : -INFINITY;
      const float sig2 = sink * kLog2e;
      const float M = fmaxf(m_used, sig2);
      float factor, lse_v;
      if (m_used == -INFINITY) {
        factor = 0.f;   // no valid entry: out = 0 and the LSE is the sink itself
        lse_v = sink;
      } else {
        const float al = __builtin_amdgcn_exp2f(m_used - M);
        const float z = l_tot * al + __builtin_amdgcn_exp2f(sig2 - M);
        factor = al / z;
        lse_v = (M + __log2f(z)) * kLn2;
      }
      factor *= e.out_scale;
      if (h_ok) {
        uint16_t* dst = e.out + ((size_t)row * a.H + h) * kV + 4 * G;
#pragma unroll
        for (int b = 0; b < 16; ++b) {
          const f32x16 ob = kO15V && b == 15 ? O15 : O[ob_index(b)];
#pragma unroll
          for (int k = 0; k < 4; ++k)
            *reinterpret_cast<u32x2*>(dst + 32 * b + 8 * k) =
                u32x2{pack_bf16x2(ob[4 * k] * factor, ob[4 * k + 1] * factor),
                      pack_bf16x2(ob[4 * k + 2] * factor, ob[4 * k + 3] * factor)};
          __builtin_amdgcn_sched_barrier(0);   // one block's values live at a time
        }
        if (e.lse != nullptr && G == 0) e.lse[(size_t)row * a.H + h] = lse_v;
      }
      return;
    }
    // Split partials for this library's own merge, in the accumulators' own layout: each
    // store is one 1 KB run (register group k of block b, all 64 lanes), with no LDS stage
    // and no normalization; beside them the head's reference max (log2 domain) and its
    // probability sum, from which the merge forms the weights.  A split with no valid entry
    // writes only its pairs (sum 0): the merge gives it no weight and never uses its runs.
    const size_t rs = (size_t)row * a.S + split;
    const int nwh = (a.H + 31) >> 5;
    float* base = a.part_o + (rs * nwh + wave) * (16 * 4 * 64 * 4) + 4 * lane_id;
    if (n_valid > 0)   // block uniform
#pragma unroll
    for (int b = 0; b < 16; ++b) {
      const f32x16 ob = kO15V && b == 15 ? O15 : O[ob_index(b)];
#pragma unroll
      for (int k = 0; k < 4; ++k)
        *reinterpret_cast<f32x4*>(base + (4 * b + k) * (64 * 4)) =
            f32x4{ob[4 * k], ob[4 * k + 1], ob[4 * k + 2], ob[4 * k + 3]};
    }
    if (G == 0 && h_ok) *reinterpret_cast<f32x2*>(a.part_lse + (rs * a.H + h) * 2) = f32x2{m_used, l_tot};
    return;
  } else {
  const bool documented = a.write_partials != 0;
  float factor, lse_v;
  if (documented) {
    if (l_tot > 0.f) {
      factor = 1.0f / l_tot;
      lse_v = (m_used + __log2f(l_tot)) * kLn2;
    } else {
      factor = 0.f;
      lse_v = -INFINITY;
    }
  } else {
    const float sink = (a.sinks != nullptr && h_ok) ? a.sinks[h] : -INFINITY;
    const float sig2 = sink * kLog2e;
    const float M = fmaxf(m_used, sig2);
    if (m_used == -INFINITY) {
      // no valid entry: out = 0 and the LSE is the sink itself
      factor = 0.f;
      lse_v = sink;
    } else {
      const float al = __builtin_amdgcn_exp2f(m_used - M);
      const float z = l_tot * al + __builtin_amdgcn_exp2f(sig2 - M);
      factor = al / z;
      lse_v = (M + __log2f(z)) * kLn2;
    }
  }
  factor *= a.out_scale;   // the per-tensor FP8 value scale (1 otherwise)

  // Accumulator register r of block b holds head h (this lane's) at dv 32b + acc_row(r, G):
  // registers 4k..4k+3 are four consecutive dv, stored as one 8-byte (bf16) or 16-byte
  // (fp32 partial) piece.
  if (documented) {
    // fp32 partials through a per-wave LDS stage, in four quarters of 128 dv: each lane
    // writes its 16-byte runs into rows of 528 bytes (one per head; the 16-byte pad keeps the
    // 32 rows' writes on different banks), then reads back 16-byte chunks along dv, so every
    // global store writes two whole 512-byte row quarters instead of 32-byte pieces of 32 rows.
    // A wave reads back only what it wrote, in order, so no barrier is needed between passes.
    constexpr int kPitchP = 528;
    static_assert(NW * 32 * kPitchP <= (int)sizeof(sK), "partial stage exceeds the K buffers");
    const size_t rs = (size_t)row * a.S + split;
    __syncthreads();   // every wave is past its last read of sK (and its copies drained)
    uint8_t* stage = reinterpret_cast<uint8_t*>(sK) + wave * (32 * kPitchP);
    int ln = lane_id;
    asm volatile("" : "+v"(ln));
    const int w_off = (ln & 31) * kPitchP + 16 * (ln >> 5);        // row = head, +4 dv for G
    const int r_off = (ln >> 5) * kPitchP + 16 * (ln & 31);        // row (ln / 32) + 2i, chunk
#pragma unroll
    for (int qd = 0; qd < 4; ++qd) {
#pragma unroll
      for (int bb = 0; bb < 4; ++bb) {
        const int b = 4 * qd + bb;
        const f32x16 ob = kO15V && b == 15 ? O15 : O[ob_index(b)];
#pragma unroll
        for (int k = 0; k < 4; ++k)
          *reinterpret_cast<f32x4*>(stage + w_off + 128 * bb + 32 * k) =
              f32x4{ob[4 * k] * factor, ob[4 * k + 1] * factor, ob[4 * k + 2] * factor, ob[4 * k + 3] * factor};
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int hr = 32 * wave + 2 * i + (ln >> 5);
        const f32x4 v = *reinterpret_cast<const f32x4*>(stage + r_off + 2 * i * kPitchP);
        if (hr < a.H)
          *reinterpret_cast<f32x4*>(a.part_o + (rs * a.H + hr) * kV + 128 * qd + 4 * (ln & 31)) = v;
        if (i % 4 == 3) __builtin_amdgcn_sched_barrier(0);   // four reads in flight at most
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if (G == 0 && h_ok) a.part_lse[rs * a.H + h] = lse_v;
  } else {
    // bf16 output through a per-wave LDS stage (the K buffers are free now), in two halves
    // of 256 dv: each lane writes its 8-byte runs into rows of 520 bytes (one per head;
    // the 8-byte pad keeps the 32 rows' writes on different banks), then reads back
    // 16-byte chunks along dv, so every global store writes two whole 512-byte row halves.
    constexpr int kPitch = 520;
    static_assert(NW * 32 * kPitch <= (int)sizeof(sK), "output stage exceeds the K buffers");
    __syncthreads();   // every wave is past its last read of sK (and its copies drained)
    uint8_t* stage = reinterpret_cast<uint8_t*>(sK) + wave * (32 * kPitch);
    int ln = lane_id;
    asm volatile("" : "+v"(ln));
    const int w_off = (ln & 31) * kPitch + 8 * (ln >> 5);          // row = head, +4 dv for G
    const int r_off = (ln >> 5) * kPitch + 16 * (ln & 31);         // row (ln / 32) + 2i, chunk
#pragma unroll
    for (int half = 0; half < 2; ++half) {
#pragma unroll
      for (int bb = 0; bb < 8; ++bb) {
        const f32x16 ob = kO15V && 8 * half + bb == 15 ? O15 : O[ob_index(8 * half + bb)];
#pragma unroll
        for (int k = 0; k < 4; ++k)
          *reinterpret_cast<u32x2*>(stage + w_off + 64 * bb + 16 * k) =
              u32x2{pack_bf16x2(ob[4 * k] * factor, ob[4 * k + 1] * factor),
                    pack_bf16x2(ob[4 * k + 2] * factor, ob[4 * k + 3] * factor)};
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int hr = 32 * wave + 2 * i + (ln >> 5);
        const u32x4 v = *reinterpret_cast<const u32x4*>(stage + r_off + 2 * i * kPitch);
        if (hr < a.H)
          *reinterpret_cast<u32x4*>(a.out + ((size_t)row * a.H + hr) * kV + 256 * half + 8 * (ln & 31)) = v;
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if (a.lse != nullptr && G == 0 && h_ok) a.lse[(size_t)row * a.H + h] = lse_v;
  }
  }
}

template <int FMT>
__global__ __launch_bounds__(256) void gather_debug_kernel(const uint8_t* __restrict__ kv, int ps_log2,
                                                           int num_slots, const int* __restrict__ slots,
                                                           int n, uint16_t* __restrict__ out) {
  const long long item = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long e = item / 72;
  const int c = (int)(item % 72);
  if (e >= n) return;
  const int slot = slots[e];
  u32x4 v = u32x4{0u, 0u, 0u, 0u};
  if (slot >= 0 && slot < num_slots) {
    const SlotAddr sa = slot_addr<FMT>(slot, ps_log2);
    v = (c < 64) ? load_latent8<FMT>(kv, sa, c) : load_rope8<FMT>(kv, sa, c - 64);
  }
  *reinterpret_cast<u32x4*>(out + e * kQK + 8 * c) = v;
}

// ---- balanced rows: entry counts per row, per-row split counts and a longest-first job order
constexpr int kOrderBins = 1024;   // classes of the order: 32 entries (one tile) each, the last open
constexpr int kMinJobTiles = 4;    // the shortest target job (128 entries, the planner's least chunk)
// a balanced share (s + 1) * n / S_r is computed in 32 bits: s < S and n <= K <= S * kCMax
static_assert((unsigned long long)SMLA_MAX_SPLITS * SMLA_MAX_SPLITS * kCMax < (1ull << 32),
              "balanced shares overflow 32 bits");

// One wave per row: the number of entries the decode keeps, by the same test as its
// translation (an id >= 0 that names a slot of the pool, through the page table in LOGICAL
// mode), so that the ranks of a balanced split are those of the decode's own list.  A lane
// takes up to eight 16-byte groups of ids per round, all loaded before any is used, then all
// their page-table entries, so a row of 2048 ids costs two memory round trips.
constexpr int kCountUnroll = 8;
__global__ __launch_bounds__(256) void count_rows_kernel(DecodeArgs a, int32_t* __restrict__ counts) {
  const int lane = threadIdx.x & 63;
  // wave-uniform, so the request lookup is a scalar load beside the vector loads of the ids
  const int row = __builtin_amdgcn_readfirstlane((int)blockIdx.x * 4 + (int)(threadIdx.x >> 6));
  if (row >= a.R) return;
  const u32x4* p = reinterpret_cast<const u32x4*>(a.indices + (size_t)row * a.K);
  const int n4 = a.K >> 2;
  u32x4 v[kCountUnroll];
  auto load_round = [&](int i0) {
#pragma unroll
    for (int u = 0; u < kCountUnroll; ++u) {
      const int i = i0 + 64 * u;
      v[u] = i < n4 ? p[i] : u32x4{~0u, ~0u, ~0u, ~0u};   // past the row: -1
    }
  };
  load_round(lane);   // the first round's ids are in flight during the request lookup
  const int* pt = nullptr;
  bool req_ok = true;
  if (a.index_mode == 0) {
    const int req = a.row_req[row];
    req_ok = req >= 0 && req < a.B;
    pt = a.page_table + (size_t)(req_ok ? req : 0) * a.max_pages;
  }
  int c = 0;
  for (int i0 = lane; i0 < n4; i0 += 64 * kCountUnroll) {
    if (i0 != lane) load_round(i0);
    if (a.index_mode == 0) {
      int pg[kCountUnroll][4];
#pragma unroll
      for (int u = 0; u < kCountUnroll; ++u)
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int t = (int)v[u][k];
          const bool ok = req_ok && t >= 0 && (t >> a.ps_log2) < a.max_pages;
          pg[u][k] = ok ? pt[t >> a.ps_log2] : -1;
        }
#pragma unroll
      for (int u = 0; u < kCountUnroll; ++u)
#pragma unroll
        for (int k = 0; k < 4; ++k) c += (pg[u][k] >= 0 && pg[u][k] < a.num_pages) ? 1 : 0;
    } else {
#pragma unroll
      for (int u = 0; u < kCountUnroll; ++u)
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int t = (int)v[u][k];
          c += (t >= 0 && t < a.num_slots) ? 1 : 0;
        }
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) c += __shfl_xor(c, off);
  if (lane == 0) counts[row] = c;
}

// One workgroup: each row's split count and the (row, split) jobs, longest first.  The target
// job length is three quarters of an even share of the slots' work (at least kMinJobTiles
// tiles); a row whose tiles exceed it splits into ceil(tiles / target) chunks, at most S (and
// at least what keeps each chunk within kCMax entries), so that only long rows pay for
// partials and a merge.  The jobs are counting-sorted by their
// tiles (jobs of one class in no particular order: no result depends on it); job_count holds
// their number.
__global__ __launch_bounds__(1024) void schedule_rows_kernel(const int32_t* __restrict__ counts, int R,
                                                             int S, int slots,
                                                             int32_t* __restrict__ row_splits,
                                                             int32_t* __restrict__ jobs,
                                                             int32_t* __restrict__ job_count) {
  __shared__ int sStart[kOrderBins];
  __shared__ int sWave[16];
  __shared__ unsigned long long sTotal;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  sStart[tid] = 0;
  if (tid == 0) sTotal = 0;
  __syncthreads();
  auto tiles = [](int n) { return (n + 31) >> 5; };
  auto cls = [&](int n) { return min(tiles(n), kOrderBins - 1); };
  unsigned long long t = 0;
  for (int r = tid; r < R; r += 1024) t += (unsigned)tiles(max(counts[r], 0));
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) t += __shfl_xor(t, off);
  if (lane == 0) atomicAdd(&sTotal, t);
  __syncthreads();
  const unsigned long long share = (3ull * sTotal + 4ull * slots - 1) / (4ull * slots);
  const int target = (int)min(max(share, (unsigned long long)kMinJobTiles), (unsigned long long)INT_MAX);
  // at least the splits that keep every chunk within a workgroup's kCMax positions
  auto splits_of = [&](int n) {
    return S > 1 ? min(S, max((n + kCMax - 1) / kCMax, max(1, (tiles(n) + target - 1) / target))) : 1;
  };
  auto job_len = [](int n, int sr, int s) {
    // 32-bit products suffice: s < 256 and n <= K <= 256 * kCMax (2^19)
    return (int)((unsigned)(s + 1) * (unsigned)n / (unsigned)sr - (unsigned)s * (unsigned)n / (unsigned)sr);
  };
  for (int r = tid; r < R; r += 1024) {
    const int n = max(counts[r], 0);
    const int sr = splits_of(n);
    row_splits[r] = sr;
    for (int s = 0; s < sr; ++s) atomicAdd(&sStart[cls(job_len(n, sr, s))], 1);
  }
  __syncthreads();
  // exclusive prefix over the classes in descending order: thread t takes class 1023 - t
  const int v = sStart[kOrderBins - 1 - tid];
  int inc = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int u = __shfl_up(inc, off);
    if (lane >= off) inc += u;
  }
  if (lane == 63) sWave[wave] = inc;
  __syncthreads();
  int before = 0;
  for (int w = 0; w < wave; ++w) before += sWave[w];
  sStart[kOrderBins - 1 - tid] = before + inc - v;
  if (tid == 1023) *job_count = before + inc;   // the last class closes the count
  __syncthreads();
  for (int r = tid; r < R; r += 1024) {
    const int n = max(counts[r], 0);
    const int sr = splits_of(n);
    for (int s = 0; s < sr; ++s) jobs[atomicAdd(&sStart[cls(job_len(n, sr, s))], 1)] = r | (s << 24);
  }
}

__global__ void fill_u64_kernel(unsigned long long* p, unsigned long long v) {
  if (threadIdx.x == 0 && blockIdx.x == 0) *p = v;
}

template <int NW, int FMT>
hipError_t launch_nw(const DecodeArgs& a, hipStream_t st) {
  const dim3 grid(a.R, a.S), block(NW * 64);
  if (a.jobs != nullptr) {
    // balanced rows: the split-format instantiation, whose rows of one split write the
    // output directly
    hipLaunchKernelGGL((decode_kernel<NW, FMT, true, true>), grid, block, 0, st, a);
  } else {
    if (a.write_partials == 2)
      hipLaunchKernelGGL((decode_kernel<NW, FMT, true, false>), grid, block, 0, st, a);
    else
      hipLaunchKernelGGL((decode_kernel<NW, FMT, false, false>), grid, block, 0, st, a);
  }
  return hipGetLastError();
}

template <int FMT>
hipError_t launch_fmt(const DecodeArgs& a, int nw, hipStream_t st) {
  switch (nw) {
    case 1: return launch_nw<1, FMT>(a, st);
    case 2: return launch_nw<2, FMT>(a, st);
    case 3: return launch_nw<3, FMT>(a, st);
    case 4: return launch_nw<4, FMT>(a, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int max_chunk_positions() { return kCMax; }

hipError_t launch_decode(const DecodeArgs& a, int kv_format, hipStream_t st) {
  const int nw = (a.H + 31) / 32;
  switch (kv_format) {
    case 1: return launch_fmt<1>(a, nw, st);
    case 2: return launch_fmt<2>(a, nw, st);
    default: return launch_fmt<0>(a, nw, st);
  }
}

hipError_t launch_gather_debug(const uint8_t* kv, int kv_format, int ps_log2, int num_slots,
                               const int* slots, int n, uint16_t* out, hipStream_t st) {
  const long long items = (long long)n * 72;
  const unsigned blocks = (unsigned)((items + 255) / 256);
  if (kv_format == 1)
    hipLaunchKernelGGL(gather_debug_kernel<1>, dim3(blocks), dim3(256), 0, st, kv, ps_log2, num_slots,
                       slots, n, out);
  else if (kv_format == 2)
    hipLaunchKernelGGL(gather_debug_kernel<2>, dim3(blocks), dim3(256), 0, st, kv, ps_log2, num_slots,
                       slots, n, out);
  else
    hipLaunchKernelGGL(gather_debug_kernel<0>, dim3(blocks), dim3(256), 0, st, kv, ps_log2, num_slots,
                       slots, n, out);
  return hipGetLastError();
}

hipError_t launch_balance(const DecodeArgs& a, int slots, int32_t* counts, int32_t* row_splits,
                          int32_t* jobs, int32_t* job_count, hipStream_t st) {
  hipLaunchKernelGGL(count_rows_kernel, dim3((unsigned)((a.R + 3) / 4)), dim3(256), 0, st, a, counts);
  hipLaunchKernelGGL(schedule_rows_kernel, dim3(1), dim3(1024), 0, st, counts, a.R, a.S, slots,
                     row_splits, jobs, job_count);
  return hipGetLastError();
}

hipError_t launch_fill_u64(unsigned long long* p, unsigned long long v, hipStream_t st) {
  hipLaunchKernelGGL(fill_u64_kernel, dim3(1), dim3(64), 0, st, p, v);
  return hipGetLastError();
}

}  // namespace smla
