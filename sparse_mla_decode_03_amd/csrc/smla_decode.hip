// Fused top-k sparse MLA decode kernel for gfx950.
//
// One workgroup handles one (query row, split) pair with all H query heads, as H/16
// waves of 16 heads each.  Steps, in the order of the Triton decode path described on
// prhub sglang#24692 ("SM120 support for DeepSeek-V4", implementation breakdown 2-3):
//   1. index translation + compaction: the row's top-k positions of this split are
//      turned into cache slots through the page table (the block-table translation of
//      prhub vllm#43477, key code excerpts: forward_mqa); -1 and out-of-range entries
//      are dropped, the surviving slots are packed densely into LDS (order kept);
//   2. per tile of 32 slots: gather the entries from HBM, dequantize FP8+UE8M0 (or take
//      BF16) into bf16, store them in LDS twice - row-major K [32][576] for QK and
//      transposed V^T [512][32] for PV;
//   3. QK: S^T[32 tokens][16 heads] per wave on bf16 MFMA 16x16x32 with q in registers;
//   4. online softmax in the exp2 domain with a lazily raised running max (rescaling O
//      only when the tile max exceeds the max in use by more than 2^8);
//   5. PV: O[16 heads][512] += P[16][32] V[32][512] on bf16 MFMA, O in registers;
//   6. epilogue: final output with the sink folded in, or the sink-free split partial.
#include "smla_device.h"
#include "smla_kernels.h"

namespace smla {

namespace {

constexpr int kT = 32;        // tokens per tile
constexpr int kKStr = 584;    // bf16 per K row in LDS: 576 + 8 pad -> 1168 B, staggers banks
constexpr int kCMax = 2048;   // positions per split handled by one workgroup
constexpr float kRescaleLog2 = 8.0f;

// V^T element (d, p) for tile position p in 0..31: rows of 32 bf16 (64 B) split into
// four 16-byte chunks, the chunk index XOR-swizzled by d so that 8 consecutive rows
// read at the same chunk hit 8 different bank groups.
__device__ __forceinline__ int vt_off(int d, int p) {
  const int sw = ((d >> 1) ^ (d >> 3)) & 3;
  return d * kT + ((((p >> 3) ^ sw) & 3) << 3) + (p & 7);
}

template <int NW, int FMT>
__global__ __launch_bounds__(NW * 64) void decode_kernel(DecodeArgs a) {
  constexpr int NT = NW * 64;
  __shared__ __attribute__((aligned(16))) uint16_t sK[kT * kKStr];
  __shared__ __attribute__((aligned(16))) uint16_t sVT[kV * kT];
  __shared__ int sSlots[kCMax];
  __shared__ int sWcnt[NW];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int row = blockIdx.x;
  const int split = blockIdx.y;
  const int p0 = split * a.chunk;
  const int p1 = min(p0 + a.chunk, a.K);
  const int ps_mask = (1 << a.ps_log2) - 1;

  // ---- 1. translate and compact the split's indices --------------------------------
  int req = 0;
  bool req_ok = true;
  if (a.index_mode == 0) {
    req = a.row_req[row];
    req_ok = req >= 0 && req < a.B;
  }
  int n_valid = 0;
  for (int base = p0; base < p1; base += NT) {
    const int p = base + tid;
    bool ok = false;
    int slot = 0;
    if (p < p1) {
      const int t = a.indices[(size_t)row * a.K + p];
      if (t != -1) {
        if (a.index_mode == 0) {
          if (req_ok && t >= 0 && (t >> a.ps_log2) < a.max_pages) {
            const int pg = a.page_table[(size_t)req * a.max_pages + (t >> a.ps_log2)];
            if (pg >= 0 && pg < a.num_pages) {
              slot = (pg << a.ps_log2) | (t & ps_mask);
              ok = true;
            }
          }
        } else if (t >= 0 && t < a.num_slots) {
          slot = t;
          ok = true;
        }
        if (!ok && a.err != nullptr)
          atomicMin(a.err, ((unsigned long long)(unsigned)row << 32) | (unsigned)p);
      }
    }
    const unsigned long long m = __ballot(ok);
    const int before = __builtin_amdgcn_mbcnt_hi((unsigned)(m >> 32),
                                                 __builtin_amdgcn_mbcnt_lo((unsigned)m, 0u));
    if (lane == 0) sWcnt[wave] = __popcll(m);
    __syncthreads();
    int off = n_valid, tot = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const int c = sWcnt[w];
      off += (w < wave) ? c : 0;
      tot += c;
    }
    if (ok) sSlots[off + before] = slot;
    n_valid += tot;
    __syncthreads();
  }

  // ---- q fragments: lane holds head 16*wave + lane%16, dims 32*ks + 8*(lane/16) + 0..7
  const int g = lane >> 4;
  const int hl = lane & 15;
  const int h = wave * 16 + hl;
  u32x4 qf[18];
  {
    const uint16_t* qp = a.q + ((size_t)row * a.H + h) * kQK + 8 * g;
#pragma unroll
    for (int ks = 0; ks < 18; ++ks) qf[ks] = *reinterpret_cast<const u32x4*>(qp + 32 * ks);
  }

  f32x4 O[32];
#pragma unroll
  for (int b = 0; b < 32; ++b) O[b] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_used = -INFINITY;
  float l_part = 0.f;

  for (int t0 = 0; t0 < n_valid; t0 += kT) {
    const int nt = min(kT, n_valid - t0);

    // ---- 2. gather + dequantize: latent items (token quad, 8-dim chunk) -------------
    for (int it = tid; it < (kT / 4) * 64; it += NT) {
      const int qd = it >> 6;
      const int c = it & 63;
      u32x4 v[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int tau = 4 * qd + k;
        if (tau < nt) {
          const SlotAddr sa = slot_addr<FMT>(sSlots[t0 + tau], a.ps_log2);
          v[k] = load_latent8<FMT>(a.kv, sa, c);
        } else {
          v[k] = u32x4{0u, 0u, 0u, 0u};
        }
        *reinterpret_cast<u32x4*>(sK + tau * kKStr + 8 * c) = v[k];
      }
      // tile position of token tau = 16*sub + 4*gq + r is 8*gq + 4*sub + r, so the
      // PV k-slice of lane group gq (tokens 4gq..4gq+3 and 16+4gq..16+4gq+3) is one chunk
      const int phys = 8 * (qd & 3) + 4 * (qd >> 2);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int w = i >> 1;
        uint32_t x0, x1;
        if (i & 1) {
          x0 = (v[0][w] >> 16) | (v[1][w] & 0xffff0000u);
          x1 = (v[2][w] >> 16) | (v[3][w] & 0xffff0000u);
        } else {
          x0 = (v[0][w] & 0xffffu) | (v[1][w] << 16);
          x1 = (v[2][w] & 0xffffu) | (v[3][w] << 16);
        }
        *reinterpret_cast<u32x2*>(sVT + vt_off(8 * c + i, phys)) = u32x2{x0, x1};
      }
    }
    // rope items (token, 8-dim chunk)
    for (int it = tid; it < kT * 8; it += NT) {
      const int tau = it >> 3;
      const int j = it & 7;
      u32x4 v = u32x4{0u, 0u, 0u, 0u};
      if (tau < nt) {
        const SlotAddr sa = slot_addr<FMT>(sSlots[t0 + tau], a.ps_log2);
        v = load_rope8<FMT>(a.kv, sa, j);
      }
      *reinterpret_cast<u32x4*>(sK + tau * kKStr + kV + 8 * j) = v;
    }
    __syncthreads();

    // ---- 3. QK: S^T[token][head], lane holds head hl, tokens 16*sub + 4g + r --------
    f32x4 s0 = f32x4{0.f, 0.f, 0.f, 0.f};
    f32x4 s1 = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 18; ++ks) {
      const u32x4 k0 = *reinterpret_cast<const u32x4*>(sK + hl * kKStr + 32 * ks + 8 * g);
      const u32x4 k1 = *reinterpret_cast<const u32x4*>(sK + (16 + hl) * kKStr + 32 * ks + 8 * g);
      s0 = mfma16x16x32(k0, qf[ks], s0);
      s1 = mfma16x16x32(k1, qf[ks], s1);
    }

    // ---- 4. online softmax (exp2 domain) ---------------------------------------------
    float t[8];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      t[r] = (4 * g + r < nt) ? s0[r] * a.scale_log2 : -INFINITY;
      t[4 + r] = (16 + 4 * g + r < nt) ? s1[r] * a.scale_log2 : -INFINITY;
    }
    float mx = t[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) mx = fmaxf(mx, t[i]);
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const bool need = mx > m_used + kRescaleLog2;
    if (__ballot(need)) {
      const float m_new = need ? mx : m_used;
      const float alpha = need ? __builtin_amdgcn_exp2f(m_used - m_new) : 1.0f;
      m_used = m_new;
      l_part *= alpha;
      float ar[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) ar[r] = __shfl(alpha, 4 * g + r);
#pragma unroll
      for (int b = 0; b < 32; ++b) {
#pragma unroll
        for (int r = 0; r < 4; ++r) O[b][r] *= ar[r];
      }
    }
    float p[8];
    float ls = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      p[i] = (t[i] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(t[i] - m_used);
      ls += p[i];
    }
    l_part += ls;
    const u32x4 pa = u32x4{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]),
                           pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7])};

    // ---- 5. PV: O[head][dv] += P[head][token] V[token][dv] --------------------------
#pragma unroll
    for (int b = 0; b < 32; ++b) {
      const u32x4 vb = *reinterpret_cast<const u32x4*>(sVT + vt_off(16 * b + hl, 8 * g));
      O[b] = mfma16x16x32(pa, vb, O[b]);
    }
    __syncthreads();
  }

  // ---- 6. epilogue ----------------------------------------------------------------------
  float l_tot = l_part + __shfl_xor(l_part, 16);
  l_tot += __shfl_xor(l_tot, 32);
  float factor, lse_v;
  if (a.write_partials) {
    if (l_tot > 0.f) {
      factor = 1.0f / l_tot;
      lse_v = (m_used + __log2f(l_tot)) * kLn2;
    } else {
      factor = 0.f;
      lse_v = -INFINITY;
    }
  } else {
    const float sink = (a.sinks != nullptr) ? a.sinks[h] : -INFINITY;
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
  float fr[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) fr[r] = __shfl(factor, 4 * g + r);

  if (a.write_partials) {
    const size_t rs = (size_t)row * a.S + split;
    float* po = a.part_o + (rs * a.H + 16 * wave) * kV;
#pragma unroll
    for (int b = 0; b < 32; ++b) {
#pragma unroll
      for (int r = 0; r < 4; ++r) po[(4 * g + r) * kV + 16 * b + hl] = O[b][r] * fr[r];
    }
    if (g == 0) a.part_lse[rs * a.H + h] = lse_v;
  } else {
    __bf16* ob = reinterpret_cast<__bf16*>(a.out) + ((size_t)row * a.H + 16 * wave) * kV;
#pragma unroll
    for (int b = 0; b < 32; ++b) {
#pragma unroll
      for (int r = 0; r < 4; ++r) ob[(4 * g + r) * kV + 16 * b + hl] = (__bf16)(O[b][r] * fr[r]);
    }
    if (a.lse != nullptr && g == 0) a.lse[(size_t)row * a.H + h] = lse_v;
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

__global__ void fill_u64_kernel(unsigned long long* p, unsigned long long v) {
  if (threadIdx.x == 0 && blockIdx.x == 0) *p = v;
}

template <int NW, int FMT>
hipError_t launch_nw(const DecodeArgs& a, hipStream_t st) {
  hipLaunchKernelGGL((decode_kernel<NW, FMT>), dim3(a.R, a.S), dim3(NW * 64), 0, st, a);
  return hipGetLastError();
}

template <int FMT>
hipError_t launch_fmt(const DecodeArgs& a, int nw, hipStream_t st) {
  switch (nw) {
    case 1: return launch_nw<1, FMT>(a, st);
    case 2: return launch_nw<2, FMT>(a, st);
    case 3: return launch_nw<3, FMT>(a, st);
    case 4: return launch_nw<4, FMT>(a, st);
    case 5: return launch_nw<5, FMT>(a, st);
    case 6: return launch_nw<6, FMT>(a, st);
    case 7: return launch_nw<7, FMT>(a, st);
    case 8: return launch_nw<8, FMT>(a, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int max_chunk_positions() { return kCMax; }

hipError_t launch_decode(const DecodeArgs& a, int kv_format, hipStream_t st) {
  const int nw = a.H / 16;
  return kv_format == 1 ? launch_fmt<1>(a, nw, st) : launch_fmt<0>(a, nw, st);
}

hipError_t launch_gather_debug(const uint8_t* kv, int kv_format, int ps_log2, int num_slots,
                               const int* slots, int n, uint16_t* out, hipStream_t st) {
  const long long items = (long long)n * 72;
  const unsigned blocks = (unsigned)((items + 255) / 256);
  if (kv_format == 1)
    hipLaunchKernelGGL(gather_debug_kernel<1>, dim3(blocks), dim3(256), 0, st, kv, ps_log2, num_slots,
                       slots, n, out);
  else
    hipLaunchKernelGGL(gather_debug_kernel<0>, dim3(blocks), dim3(256), 0, st, kv, ps_log2, num_slots,
                       slots, n, out);
  return hipGetLastError();
}

hipError_t launch_fill_u64(unsigned long long* p, unsigned long long v, hipStream_t st) {
  hipLaunchKernelGGL(fill_u64_kernel, dim3(1), dim3(64), 0, st, p, v);
  return hipGetLastError();
}

}  // namespace smla
