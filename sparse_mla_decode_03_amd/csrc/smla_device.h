// Device-side helpers shared by the gfx950 kernels of the sparse MLA decode library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace smla {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;

constexpr int kQK = 576;      // latent 512 + rope 64
constexpr int kV = 512;       // value width = latent
constexpr int kRope = 64;
constexpr int kFp8Entry = 648;
constexpr int kBf16Entry = 1152;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;

__device__ __forceinline__ f32x16 mfma32x32x16(const u32x4& a, const u32x4& b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
// The same MFMA with its accumulator in VGPRs, accumulating in place.  The compiler does not
// see its latency: the s_nop in front covers a VALU write of an operand just before it, and
// mfma_vgpr_drain() must run before any other instruction reads `c` after the last one.
__device__ __forceinline__ void mfma32x32x16_vgpr(const u32x4& a, const u32x4& b, f32x16& c) {
  asm volatile("s_nop 2\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "v"(b));
}
// Wait states for the result of a VGPR-form 32x32x16 MFMA (8 passes) to be readable.
__device__ __forceinline__ void mfma_vgpr_drain() {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
}

// LDS transpose read of four 16-bit values.  Within each group of 16 lanes, lane i
// receives element i%4 of the 8-byte blocks addressed by lanes 4k + i/4, k = 0..3.
__device__ __forceinline__ u32x2 lds_read_tr16(const uint16_t* p) {
  const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(p));
  return __builtin_bit_cast(u32x2, v);
}

__device__ __forceinline__ f32x4 mfma16x16x32(const u32x4& a, const u32x4& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Two floats -> packed bf16 pair (round to nearest even, hardware conversion).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v;
  v[0] = (__bf16)lo;
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

// UE8M0 byte e -> the fp32 scale 2^(e-127) (exponent field e, zero mantissa).
__device__ __forceinline__ float ue8m0_scale(uint32_t e) {
  return __builtin_bit_cast(float, e << 23);
}

// Eight OCP e4m3fn codes (two dwords, code of dim i in byte i) -> eight bf16 values of
// code * scale, packed as four bf16 pairs.  Exact whenever the product is a normal bf16.
__device__ __forceinline__ u32x4 dequant8_fp8(u32x2 raw, float scale) {
  u32x4 o;
  o[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw[0], scale, false));
  o[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw[0], scale, true));
  o[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw[1], scale, false));
  o[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw[1], scale, true));
  return o;
}

// Byte offsets of one cache slot's regions.  FP8 page = latent [ps][512] | rope bf16
// [ps][64] | scales [ps][8]; BF16 page = bf16 [ps][576]; per-tensor FP8 (FMT 2) page =
// e4m3fn [ps][576], one scale for the whole cache applied outside the gather.
struct SlotAddr {
  size_t latent;  // FP8: 512 codes; BF16: the 1152-byte row
  size_t rope;    // FP8 only
  size_t scales;  // FP8 only
};

template <int FMT>
__device__ __forceinline__ SlotAddr slot_addr(int slot, int ps_log2) {
  const size_t page = (size_t)((uint32_t)slot >> ps_log2);
  const size_t row = (size_t)((uint32_t)slot & ((1u << ps_log2) - 1u));
  SlotAddr a;
  if (FMT == 1) {
    const size_t base = page * ((size_t)kFp8Entry << ps_log2);
    a.latent = base + row * 512;
    a.rope = base + ((size_t)512 << ps_log2) + row * 128;
    a.scales = base + ((size_t)640 << ps_log2) + row * 8;
  } else if (FMT == 2) {
    a.latent = ((page << ps_log2) + row) * kQK;
    a.rope = a.latent + 512;
    a.scales = 0;
  } else {
    a.latent = (page << ps_log2) * kBf16Entry + row * kBf16Entry;
    a.rope = a.latent + 1024;
    a.scales = 0;
  }
  return a;
}

// Load and dequantize dims [8c, 8c+8) of a latent row (c in 0..63) as 8 bf16 values.
template <int FMT>
__device__ __forceinline__ u32x4 load_latent8(const uint8_t* __restrict__ kv, const SlotAddr& a, int c) {
  if (FMT == 1) {
    const u32x2 raw = *reinterpret_cast<const u32x2*>(kv + a.latent + 8 * c);
    const uint32_t e = kv[a.scales + (c >> 3)];
    return dequant8_fp8(raw, ue8m0_scale(e));
  } else if (FMT == 2) {
    return dequant8_fp8(*reinterpret_cast<const u32x2*>(kv + a.latent + 8 * c), 1.0f);
  } else {
    return *reinterpret_cast<const u32x4*>(kv + a.latent + 16 * c);
  }
}

// Load rope dims [512 + 8j, 512 + 8j + 8) (j in 0..7) as 8 bf16 values.
template <int FMT>
__device__ __forceinline__ u32x4 load_rope8(const uint8_t* __restrict__ kv, const SlotAddr& a, int j) {
  if (FMT == 2) return dequant8_fp8(*reinterpret_cast<const u32x2*>(kv + a.rope + 8 * j), 1.0f);
  return *reinterpret_cast<const u32x4*>(kv + a.rope + 16 * j);
}


// Copy 16 (or 4) bytes per lane from global memory into LDS at dst + lane*size
// (global_load_lds; dst is the same for the whole wave).  Written as inline asm so that
// the compiler does not track these LDS writes: it would otherwise wait for every copy in
// flight (vmcnt(0)) before any read of the staging area, exposing the full memory latency
// once per tile.  The kernel orders the copies itself with explicit vmcnt waits (wait_vm,
// wait_vm_le) before reading what they wrote.
__device__ __forceinline__ uint32_t lds_offset(const void* p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)(p));
}
__device__ __forceinline__ void dma16(const void* src, const void* lds_wave_base) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :: "v"(src), "s"(lds_offset(lds_wave_base)) : "memory");
}
__device__ __forceinline__ void dma4(const void* src, const void* lds_wave_base) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
               :: "v"(src), "s"(lds_offset(lds_wave_base)) : "memory");
}
// The same copies to an LDS byte address already in an SGPR (an LDS array's address from
// lds_offset plus wave-uniform integer offsets), which spares the generic-to-LDS pointer
// conversion and its null test at every copy.
__device__ __forceinline__ void dma16_at(const void* src, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :: "v"(src), "s"(lds_addr) : "memory");
}
__device__ __forceinline__ void dma4_at(const void* src, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
               :: "v"(src), "s"(lds_addr) : "memory");
}
// Wait until at most N of this wave's global loads (LDS copies included) are pending.
// The builtin lets the compiler's own wait insertion see the wait; the empty asm with a
// memory clobber keeps LDS reads of the copied data below it.
template <int N>
__device__ __forceinline__ void wait_vm_le() {
  static_assert(N >= 0 && N < 64, "vmcnt is six bits");
  // vmcnt is split over bits 3:0 and 15:14; expcnt and lgkmcnt stay at their maxima
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x70 | 0xF00);
  asm volatile("" ::: "memory");
}
__device__ __forceinline__ void wait_vm() { wait_vm_le<0>(); }

}  // namespace smla
