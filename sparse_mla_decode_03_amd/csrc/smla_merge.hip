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

}  // namespace

hipError_t launch_merge(const float* part_o, const float* part_lse, int R, int S, int H,
                        const float* sinks, uint16_t* out, float* lse, hipStream_t st) {
  const long long blocks = (long long)R * H;
  hipLaunchKernelGGL(merge_kernel, dim3((unsigned)blocks), dim3(64), 0, st, part_o, part_lse, R, S,
                     H, sinks, out, lse);
  return hipGetLastError();
}

}  // namespace smla
