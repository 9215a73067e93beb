// Cache store for gfx950: new tokens' latent and rope rows into the paged cache.
//
// The FP8 format is e4m3fn codes with one UE8M0 scale byte per 64 latent elements and
// the 64 rope values kept in bf16 (the UE8M0 paged cache named on prhub vllm#43827,
// motivation and key code excerpts), laid out in region-split pages (latent | rope |
// scales) addressed inside the page (prhub sglang#24692, implementation breakdown 2).
// The scale of a group is the smallest power of two 2^(e-127) with 448 * 2^(e-127) >= the
// group's largest magnitude, so every code is finite; codes are rounded to nearest, ties
// to even.  One 64-lane wave stores one token: lane l converts latent dims 8l..8l+7, the
// eight lanes of a 64-element group reduce its maximum, lanes 0..7 copy the rope.
#include "smla_device.h"
#include "smla_kernels.h"

namespace smla {

namespace {

// UE8M0 byte for a group maximum `amax` (a non-negative float holding a bf16 value):
// amax = f * 2^(E - 127) with f in [1, 2) needs 448 * 2^k >= amax, i.e. k = E - 135 when
// f <= 1.75 (448 = 1.75 * 2^8) and one more otherwise; e = k + 127, clamped to [0, 254].
// amax = 0 gives 127.
__device__ __forceinline__ uint32_t ue8m0_for_amax(float amax) {
  const uint32_t b = __float_as_uint(amax);
  if (b == 0u) return 127u;
  const int e = (int)(b >> 23) - 8 + ((b & 0x7FFFFFu) > 0x600000u ? 1 : 0);
  return (uint32_t)min(max(e, 0), 254);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Tokens per wave.  A wave issues its tokens' slot, latent and rope loads together, before
// the slot is checked, so it waits for one memory round trip instead of two (slot, then
// data).  More tokens per wave leave fewer waves to cover the latency: 2 and 4 were slower.
constexpr int kTokPerWave = 1;

template <int FMT>
__global__ __launch_bounds__(256) void store_kernel(const uint16_t* __restrict__ latent,
                                                    const uint16_t* __restrict__ rope,
                                                    const int32_t* __restrict__ slots, int n,
                                                    int ps_log2, int num_slots, uint8_t* __restrict__ kv) {
  const int tok0 = (blockIdx.x * 4 + (threadIdx.x >> 6)) * kTokPerWave;
  const int lane = threadIdx.x & 63;
  if (tok0 >= n) return;                      // the whole wave
  int slot[kTokPerWave];
  u32x4 w[kTokPerWave], rv[kTokPerWave];
#pragma unroll
  for (int i = 0; i < kTokPerWave; ++i) {
    const int tok = tok0 + i;
    const bool ok = tok < n;                  // wave uniform
    slot[i] = ok ? slots[tok] : -1;
    w[i] = ok ? *reinterpret_cast<const u32x4*>(latent + (size_t)tok * 512 + 8 * lane) : u32x4{};
    rv[i] = ok && lane < 8 ? *reinterpret_cast<const u32x4*>(rope + (size_t)tok * 64 + 8 * lane) : u32x4{};
  }
#pragma unroll
  for (int i = 0; i < kTokPerWave; ++i) {
    if (slot[i] < 0 || slot[i] >= num_slots) continue;   // the whole wave: token skipped
    const SlotAddr sa = slot_addr<FMT>(slot[i], ps_log2);
    if (lane < 8) *reinterpret_cast<u32x4*>(kv + sa.rope + 16 * lane) = rv[i];
    if (FMT == 1) {
      float x[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        x[2 * j] = bf16_lo(w[i][j]);
        x[2 * j + 1] = bf16_hi(w[i][j]);
      }
      float am = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) am = fmaxf(am, fabsf(x[j]));
      // the group's eight lanes are lanes 8g .. 8g+7
      am = fmaxf(am, __shfl_xor(am, 1));
      am = fmaxf(am, __shfl_xor(am, 2));
      am = fmaxf(am, __shfl_xor(am, 4));
      const uint32_t e = ue8m0_for_amax(am);
      // x * 2^sh is exact and at most 448 in magnitude; the hardware conversion rounds it to
      // the nearest e4m3fn value, ties to even (subnormal codes included), in the default
      // round-to-nearest mode
      const int sh = 127 - (int)e;
      float y[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) y[j] = __builtin_amdgcn_ldexpf(x[j], sh);
      int w0 = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
      w0 = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], w0, true);
      int w1 = __builtin_amdgcn_cvt_pk_fp8_f32(y[4], y[5], 0, false);
      w1 = __builtin_amdgcn_cvt_pk_fp8_f32(y[6], y[7], w1, true);
      *reinterpret_cast<u32x2*>(kv + sa.latent + 8 * lane) = u32x2{(uint32_t)w0, (uint32_t)w1};
      if ((lane & 7) == 0) kv[sa.scales + (lane >> 3)] = (uint8_t)e;
    } else {
      *reinterpret_cast<u32x4*>(kv + sa.latent + 16 * lane) = w[i];
    }
  }
}

}  // namespace

hipError_t launch_store(const uint16_t* latent, const uint16_t* rope, const int32_t* slots, int n,
                        int kv_format, int ps_log2, int num_slots, uint8_t* kv, hipStream_t st) {
  const unsigned blocks = (unsigned)((n + 4 * kTokPerWave - 1) / (4 * kTokPerWave));
  if (kv_format == 1)
    hipLaunchKernelGGL(store_kernel<1>, dim3(blocks), dim3(256), 0, st, latent, rope, slots, n, ps_log2,
                       num_slots, kv);
  else
    hipLaunchKernelGGL(store_kernel<0>, dim3(blocks), dim3(256), 0, st, latent, rope, slots, n, ps_log2,
                       num_slots, kv);
  return hipGetLastError();
}

}  // namespace smla
