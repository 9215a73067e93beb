// LSE merge of split-KV partials with the attention sink applied once.
//
// The split decode on prhub sglang#24692 ("SM120 support for DeepSeek-V4", key files:
// the Triton decode module with its merge of partial attention and its sink step)
// produces per-chunk results that are merged afterwards; here one kernel does both:
//   M = max(max_c lse_c, sigma), w_c = exp(lse_c - M), w_s = exp(sigma - M),
//   out = sum_c w_c o_c / (sum_c w_c + w_s), lse = M + ln(sum_c w_c + w_s).
// One 64-lane wave per (row, head); each lane owns 8 of the 512 output dims.
#include "smla_device.h"
#include "smla_kernels.h"

namespace smla {

namespace {

__global__ __launch_bounds__(64) void merge_kernel(const float* __restrict__ po,
                                                   const float* __restrict__ pl, int R, int S,
                                                   int H, const float* __restrict__ sinks,
                                                   uint16_t* __restrict__ out, float* __restrict__ lse) {
  const long long rh = blockIdx.x;
  const int r = (int)(rh / H);
  const int h = (int)(rh % H);
  const int lane = threadIdx.x;
  const float sink = (sinks != nullptr) ? sinks[h] : -INFINITY;
  const float sig2 = sink * kLog2e;
  const float* plr = pl + (size_t)r * S * H + h;
  float mc = -INFINITY;
  for (int c = 0; c < S; ++c) mc = fmaxf(mc, plr[(size_t)c * H] * kLog2e);
  const float M = fmaxf(mc, sig2);
  u32x4 res = u32x4{0u, 0u, 0u, 0u};
  float lse_v = sink;  // every chunk empty: out = 0, LSE = the sink (or -inf)
  if (mc != -INFINITY) {
    float z = (sig2 == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(sig2 - M);
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int c = 0; c < S; ++c) {
      const float l2 = plr[(size_t)c * H] * kLog2e;
      if (l2 == -INFINITY) continue;
      const float w = __builtin_amdgcn_exp2f(l2 - M);
      z += w;
      const float* src = po + (((size_t)r * S + c) * H + h) * kV + 8 * lane;
      const f32x4 x0 = *reinterpret_cast<const f32x4*>(src);
      const f32x4 x1 = *reinterpret_cast<const f32x4*>(src + 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[i] += w * x0[i];
        acc[4 + i] += w * x1[i];
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
