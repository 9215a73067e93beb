// LSE merge of split-KV partials with the attention sink applied once.
//
// The split decode on prhub sglang#24692 ("SM120 support for DeepSeek-V4", key files:
// the Triton decode module with its merge of partial attention and its sink step)
// produces per-chunk results that are merged afterwards; here one kernel does both:
//   M = max(max_c lse_c, sigma), w_c = exp(lse_c - M), w_s = exp(sigma - M),
//   out = sum_c w_c o_c / (sum_c w_c + w_s), lse = M + ln(sum_c w_c + w_s).
// One 64-lane wave per (row, head); each lane owns 8 of the 512 output dims.  The partial
// rows of the first sixteen chunks and all chunk LSEs are loaded together, later chunks
// sixteen at a time, so a merge costs one memory round trip per sixteen chunks.
#include "sparse_mla.h"
#include "smla_device.h"
#include "smla_kernels.h"

namespace smla {

namespace {

constexpr int kMaxChunks = 256;   // the largest split count a plan allows
static_assert(kMaxChunks >= SMLA_MAX_SPLITS, "merge chunk capacity below the plan limit");
constexpr int kBatch = 16;        // partial rows loaded together

__global__ __launch_bounds__(64) void merge_kernel(const float* __restrict__ po,
                                                   const float* __restrict__ pl, int R, int S,
                                                   int H, const float* __restrict__ sinks,
                                                   uint16_t* __restrict__ out, float* __restrict__ lse) {
  // chunk weights, shared by the wave (S <= kMaxChunks)
  __shared__ float sw[kMaxChunks];
  const long long rh = blockIdx.x;
  const int r = (int)(rh / H);
  const int h = (int)(rh % H);
  const int lane = threadIdx.x;
  const float sink = (sinks != nullptr) ? sinks[h] : -INFINITY;
  const float sig2 = sink * kLog2e;
  const float* plr = pl + (size_t)r * S * H + h;
  // lane owns output dims 8l..8l+7; the partial rows of the first kBatch chunks are loaded
  // together with the chunk LSEs (before the weights are known), so a merge of up to kBatch
  // chunks costs one memory round trip
  const float* src0 = po + ((size_t)r * S * H + h) * kV + 8 * lane;
  const size_t cstride = (size_t)H * kV;
  f32x4 x[kBatch][2];
#pragma unroll
  for (int j = 0; j < kBatch; ++j) {
    if (j < S) {   // wave-uniform; rows past S are never read (their weight is 0)
      const float* src = src0 + j * cstride;
      x[j][0] = *reinterpret_cast<const f32x4*>(src);
      x[j][1] = *reinterpret_cast<const f32x4*>(src + 4);
    }
  }
  // every chunk's LSE at once: lane l holds chunks l, l + 64, ... (log2 domain)
  float l2[kMaxChunks / 64];
  float mc = -INFINITY;
#pragma unroll
  for (int i = 0; i < kMaxChunks / 64; ++i) {
    const int c = lane + 64 * i;
    l2[i] = c < S ? plr[(size_t)c * H] * kLog2e : -INFINITY;
    mc = fmaxf(mc, l2[i]);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) mc = fmaxf(mc, __shfl_xor(mc, off));
  const float M = fmaxf(mc, sig2);
  u32x4 res = u32x4{0u, 0u, 0u, 0u};
  float lse_v = sink;  // every chunk empty: out = 0, LSE = the sink (or -inf)
  if (mc != -INFINITY) {
    // w_c = 2^(l2_c - M); an empty chunk (LSE -inf) has weight 0 and is skipped below
    float zs = 0.f;
#pragma unroll
    for (int i = 0; i < kMaxChunks / 64; ++i) {
      const int c = lane + 64 * i;
      const float w = l2[i] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(l2[i] - M);
      if (c < S) sw[c] = w;
      zs += w;
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) zs += __shfl_xor(zs, off);
    const float z = zs + ((sig2 == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(sig2 - M));
    __syncthreads();
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int c0 = 0; c0 < S; c0 += kBatch) {
      if (c0 > 0) {   // later batches: their loads, all before any use
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
          if (c0 + j < S) {
            const float* src = src0 + (c0 + j) * cstride;
            x[j][0] = *reinterpret_cast<const f32x4*>(src);
            x[j][1] = *reinterpret_cast<const f32x4*>(src + 4);
          }
        }
      }
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        const float w = (c0 + j < S) ? sw[c0 + j] : 0.f;   // wave-uniform
        if (w > 0.f) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            acc[i] += w * x[j][0][i];
            acc[4 + i] += w * x[j][1][i];
          }
        }
      }
    }
    const float inv = 1.0f / z;
    res = u32x4{pack_bf16x2(acc[0] * inv, acc[1] * inv), pack_bf16x2(acc[2] * inv, acc[3] * inv),
                pack_bf16x2(acc[4] * inv, acc[5] * inv), pack_bf16x2(acc[6] * inv, acc[7] * inv)};
    lse_v = (M + __log2f(z)) * kLn2;
  }
  *reinterpret_cast<u32x4*>(out + ((size_t)r * H + h) * kV + 8 * lane) = res;
  if (lse != nullptr && lane == 0) lse[(size_t)r * H + h] = lse_v;
}

// The same merge over the decode's own split format (write_partials == 2): per (row, split)
// and group of 32 heads, 16 blocks of 32 dv as 4 runs of 64 lanes x 4 floats (lane l: head
// 32g + l%32, dv 32b + 8k + 4(l/32) + 0..3), unnormalized, beside (m, l) per head: the
// head's reference max in the log2 domain and its probability sum.  With sigma the sink in
// the log2 domain:
//   M = max(max_c m_c, sigma), w_c = 2^(m_c - M),
//   out = sum_c w_c O_c / (sum_c w_c l_c + 2^(sigma - M)),  lse = (M + log2 z) ln 2,
// the same result as normalizing each chunk first; out is then multiplied by out_scale (the
// per-tensor FP8 value scale, 1 otherwise).  One wave merges one (row, head group, block),
// each lane 16 outputs of one head.  NB splits' runs and NM splits' (m, l) pairs are loaded
// together; the launch takes the smallest NB that covers S (up to 8), so a merge of few
// splits holds few registers, and below 8 splits the runs of a split that is empty for all
// of the wave's heads are not read.  STAGE (grids of many rows): one workgroup of four waves
// per (row, head group, quarter of dv), whose bf16 results pass through LDS so that every
// store writes whole 256-byte pieces of head rows (a wave's own 32 dv of 32 heads are
// 64-byte pieces, half a cache line each); otherwise one single-wave workgroup per block,
// which spreads a merge of few rows over more CUs, or (KR = 2: more than eight splits over
// very few rows) per half block, whose lanes hold 8 outputs each so that sixteen splits load
// in one round trip.
constexpr int kStagePitch = 272;   // bytes per head row of the stage: 128 dv + 16 bytes of pad
constexpr int kStageMinGroups = 128;   // (row, head group) pairs from which the stage is used
constexpr int kHalfMaxGroups = 16;     // (row, head group) pairs up to which half blocks are used

template <int NB, int NM, bool STAGE, int KR>
__global__ __launch_bounds__(STAGE ? 256 : 64) void merge_native_kernel(
    const float* __restrict__ po, const float* __restrict__ pml, int R, int S, int H,
    const float* __restrict__ sinks, float out_scale, uint16_t* __restrict__ out,
    float* __restrict__ lse, const int32_t* __restrict__ row_splits) {
  __shared__ __attribute__((aligned(16))) uint8_t sStage[STAGE ? 32 * kStagePitch : 16];
  const int nwh = (H + 31) >> 5;
  const long long id = blockIdx.x;
  static_assert(KR == 4 || (KR == 2 && !STAGE), "half blocks only without the stage");
  constexpr int kPer = STAGE ? 4 : 16 * (4 / KR);     // workgroups per (row, head group)
  const int part = (int)(id % kPer);
  const int g = (int)((id / kPer) % nwh);
  const int r = (int)(id / (kPer * nwh));
  const int wave = STAGE ? (int)(threadIdx.x >> 6) : 0;
  const int b = STAGE ? 4 * part + wave : (KR == 4 ? part : part >> 1);
  const int k0 = KR == 4 ? 0 : 2 * (part & 1);       // the wave's first run of the block
  const int lane = threadIdx.x & 63;
  // chunks of this row: all S, or (balanced rows) the row's own count; a row of one chunk
  // was written by the decode itself (uniform over the workgroup: one row)
  int Sr = S;
  if (row_splits != nullptr) {
    Sr = min(max(row_splits[r], 1), S);
    if (Sr == 1) return;
  }
  const int h = 32 * g + (lane & 31);
  const bool h_ok = h < H;
  const int hc = h_ok ? h : H - 1;                  // padded heads read a real head's pair
  const float sink = (sinks != nullptr) ? sinks[hc] : -INFINITY;
  const float sig2 = sink * kLog2e;
  const f32x2* ml = reinterpret_cast<const f32x2*>(pml) + (size_t)r * S * H + hc;
  const float* src0 = po + ((size_t)r * S * nwh + g) * (16 * 4 * 64 * 4) + (4 * b + k0) * (64 * 4) + 4 * lane;
  const size_t cstride = (size_t)nwh * (16 * 4 * 64 * 4);
  // one memory round trip for the pairs of the first NM splits and the runs of the first NB
  // (all issued before any use; the runs do not depend on the weights)
  static_assert(NM >= NB, "the first batch's weights come from the pairs loaded with it");
  f32x2 v[NM];
  f32x4 x[NB][KR];
#pragma unroll
  for (int j = 0; j < NM; ++j)
    if (j < Sr) v[j] = ml[(size_t)j * H];
#pragma unroll
  for (int j = 0; j < NB; ++j)
    if (j < Sr && (NB > 4 || __ballot(v[j][1] > 0.f) != 0)) {
      const float* src = src0 + j * cstride;
#pragma unroll
      for (int k = 0; k < KR; ++k) x[j][k] = *reinterpret_cast<const f32x4*>(src + k * (64 * 4));
    }
  // pass 1: the head's largest reference over the non-empty chunks (and the sink)
  float M = sig2;
  bool any = false;                                  // a non-empty chunk
#pragma unroll
  for (int j = 0; j < NM; ++j)
    if (j < Sr && v[j][1] > 0.f) {
      M = fmaxf(M, v[j][0]);
      any = true;
    }
  for (int c0 = NM; c0 < Sr; c0 += 16) {
    f32x2 u[16];
#pragma unroll
    for (int j = 0; j < 16; ++j)
      if (c0 + j < Sr) u[j] = ml[(size_t)(c0 + j) * H];
#pragma unroll
    for (int j = 0; j < 16; ++j)
      if (c0 + j < Sr && u[j][1] > 0.f) {
        M = fmaxf(M, u[j][0]);
        any = true;
      }
  }
  float acc[4 * KR];
#pragma unroll
  for (int i = 0; i < 4 * KR; ++i) acc[i] = 0.f;
  float z = 0.f;
  if (any) {
    // pass 2: weights and the weighted sum; the first batch is already in registers
    for (int c0 = 0; c0 < Sr; c0 += NB) {
      f32x2 w2[NB];
      if (c0 > 0) {
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          if (c0 + j < Sr) {
            w2[j] = ml[(size_t)(c0 + j) * H];
            const float* src = src0 + (c0 + j) * cstride;
#pragma unroll
            for (int k = 0; k < KR; ++k) x[j][k] = *reinterpret_cast<const f32x4*>(src + k * (64 * 4));
          }
        }
      } else {
#pragma unroll
        for (int j = 0; j < NB; ++j) w2[j] = v[j];
      }
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        if (c0 + j < Sr && w2[j][1] > 0.f) {
          const float w = __builtin_amdgcn_exp2f(w2[j][0] - M);
          z += w * w2[j][1];
#pragma unroll
          for (int k = 0; k < KR; ++k)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[4 * k + i] += w * x[j][k][i];
        }
      }
    }
    z += sig2 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sig2 - M);
  }
  // every chunk empty: z = 0, so out = 0 and the LSE is the sink itself (or -inf)
  const float inv = z > 0.f ? out_scale / z : 0.f;
  const float lse_v = z > 0.f ? (M + __log2f(z)) * kLn2 : sink;
  if constexpr (!STAGE) {
    if (h_ok) {
      uint16_t* dst = out + ((size_t)r * H + h) * kV + 32 * b + 8 * k0 + 4 * (lane >> 5);
#pragma unroll
      for (int k = 0; k < KR; ++k)
        *reinterpret_cast<u32x2*>(dst + 8 * k) =
            u32x2{pack_bf16x2(acc[4 * k] * inv, acc[4 * k + 1] * inv),
                  pack_bf16x2(acc[4 * k + 2] * inv, acc[4 * k + 3] * inv)};
      if (lse != nullptr && b == 0 && k0 == 0 && lane < 32) lse[(size_t)r * H + h] = lse_v;
    }
    return;
  }
  // lane: head row lane % 32 of the stage, dv 32 * wave + 8k + 4 (lane / 32) + 0..3
  uint8_t* srow = sStage + (lane & 31) * kStagePitch + 64 * wave + 8 * (lane >> 5);
#pragma unroll
  for (int k = 0; k < 4; ++k)
    *reinterpret_cast<u32x2*>(srow + 16 * k) =
        u32x2{pack_bf16x2(acc[4 * k] * inv, acc[4 * k + 1] * inv),
              pack_bf16x2(acc[4 * k + 2] * inv, acc[4 * k + 3] * inv)};
  if (h_ok && lse != nullptr && b == 0 && lane < 32) lse[(size_t)r * H + h] = lse_v;
  __syncthreads();
  // 32 heads x 256 bytes: thread t stores 16-byte pieces t and t + 256 (head piece / 16)
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int c = threadIdx.x + 256 * i;
    const int hr = c >> 4;
    const int piece = c & 15;
    const u32x4 v = *reinterpret_cast<const u32x4*>(sStage + hr * kStagePitch + 16 * piece);
    if (32 * g + hr < H)
      *reinterpret_cast<u32x4*>(out + ((size_t)r * H + 32 * g + hr) * kV + 128 * part + 8 * piece) = v;
  }
}

}  // namespace

hipError_t launch_merge_native(const float* part_o, const float* part_ml, int R, int S, int H,
                               const float* sinks, float out_scale, uint16_t* out, float* lse,
                               const int32_t* row_splits, hipStream_t st) {
  // the staged layout once there are enough (row, head group) pairs to fill the chip with
  // four-wave workgroups
  const long long groups = (long long)R * ((H + 31) / 32);
  const bool stage = groups >= kStageMinGroups;
  const dim3 block(stage ? 256 : 64);
  if (!stage && S > 8 && groups <= kHalfMaxGroups) {
    // half blocks for very few rows: sixteen splits' runs in one round trip, and twice the
    // waves (b2_h128_bf16_split16: 27.6 -> 27.1 us; 64 groups at 16 splits measured 2 % slower)
    hipLaunchKernelGGL((merge_native_kernel<16, 16, false, 2>), dim3((unsigned)(groups * 32)), block, 0,
                       st, part_o, part_ml, R, S, H, sinks, out_scale, out, lse, row_splits);
    return hipGetLastError();
  }
  const dim3 grid((unsigned)(groups * (stage ? 4 : 16)));
#define SMLA_MERGE_NATIVE(NB, NM)                                                                    \
  do {                                                                                               \
    if (stage)                                                                                       \
      hipLaunchKernelGGL((merge_native_kernel<NB, NM, true, 4>), grid, block, 0, st, part_o, part_ml, \
                         R, S, H, sinks, out_scale, out, lse, row_splits);                           \
    else                                                                                             \
      hipLaunchKernelGGL((merge_native_kernel<NB, NM, false, 4>), grid, block, 0, st, part_o,         \
                         part_ml, R, S, H, sinks, out_scale, out, lse, row_splits);                  \
  } while (0)
  if (S <= 2)
    SMLA_MERGE_NATIVE(2, 2);
  else if (S <= 4)
    SMLA_MERGE_NATIVE(4, 4);
  else
    SMLA_MERGE_NATIVE(8, 16);
#undef SMLA_MERGE_NATIVE
  return hipGetLastError();
}

hipError_t launch_merge(const float* part_o, const float* part_lse, int R, int S, int H,
                        const float* sinks, uint16_t* out, float* lse, hipStream_t st) {
  const long long blocks = (long long)R * H;
  hipLaunchKernelGGL(merge_kernel, dim3((unsigned)blocks), dim3(64), 0, st, part_o, part_lse, R, S,
                     H, sinks, out, lse);
  return hipGetLastError();
}

}  // namespace smla
