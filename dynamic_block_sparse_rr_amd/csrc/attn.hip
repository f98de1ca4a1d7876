// Stage 2 of RRAttention on gfx950: block-sparse flash attention over the
// compacted per-row block lists ("computing only half of the attention
// blocks", abstract of "RRAttention: Dynamic Block Sparse Attention via
// Per-Head Round-Robin Shifts for Long-Context Inference").
//
// bfloat16 path (the hot kernel)
//   transpose_v  V [L][Hkv][d] -> Vt [Hkv][nb][d][B]: each key block becomes a
//                contiguous 2*B*d-byte tile whose rows are head-dim channels
//                and whose columns are the block's keys (permuted inside every
//                group of 16, see key_of_pos). One HBM pass over V.
//   attn_bf16    one workgroup of B/32 waves per (query head h, query block i);
//                wave w owns 32 query rows. Per selected key block j:
//                  K tile and Vt tile staged in LDS (16-byte chunks, XOR
//                  swizzled by row so the MFMA operand reads are conflict-free);
//                  S^T = K Q^T on v_mfma_f32_32x32x16_bf16: each lane ends up
//                  owning one query and 64 of its keys (the other lane half
//                  owns the other 64), so the online softmax (running max and
//                  sum, base-2 with the 1/sqrt(d) scale folded in) needs one
//                  cross-half exchange per tile;
//                  P is rounded to bf16 straight from that register layout,
//                  which is exactly the B-operand layout of O^T += Vt P^T, so
//                  O^T accumulates in registers with no shuffles.
//                Grid order: query blocks with the most candidate blocks
//                first, the G query heads sharing a KV head adjacent and on
//                the same XCD (dispatch is round-robin over the 8 XCDs), so
//                K/V tiles are reused from that XCD's L2.
// float32 path: a plain kernel (one thread per query row, K/V tiles in LDS,
// online softmax in registers).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rr_kernels.h"

namespace rr {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float exp2_approx(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)lo) |
         ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)hi) << 16);
}

// Position p (0..15) inside a 16-key group of a Vt row holds key key_of_pos(p)
// of that group. This matches the order in which a lane holds its
// probabilities after S^T = K Q^T (lane half hf, register v: key 8*(v/4) +
// 4*hf + v%4), so that eight consecutive Vt entries form one MFMA A operand.
__host__ __device__ __forceinline__ int key_of_pos(int p) {
  return 8 * ((p & 7) >> 2) + 4 * (p >> 3) + (p & 3);
}

// ------------------------------------------------------------------ V re-layout

template <int D, int BLK>
__global__ void __launch_bounds__(256) transpose_v_kernel(const __bf16* __restrict__ v,
                                                          __bf16* __restrict__ vt, int Hkv, int nb) {
  // one workgroup per (g, key block j); tile BLK keys x D channels
  __shared__ uint16_t tile[BLK][D + 2];
  const int j = blockIdx.x % nb;
  const int g = blockIdx.x / nb;
  const uint16_t* src = reinterpret_cast<const uint16_t*>(v);
  constexpr int CH = D / 8;  // 16-byte chunks per key row
  for (int n = threadIdx.x; n < BLK * CH; n += 256) {
    const int key = n / CH, c = n % CH;
    const u32x4 w = *reinterpret_cast<const u32x4*>(src + ((size_t)(j * BLK + key) * Hkv + g) * D + c * 8);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      tile[key][c * 8 + 2 * e] = (uint16_t)(w[e] & 0xffffu);
      tile[key][c * 8 + 2 * e + 1] = (uint16_t)(w[e] >> 16);
    }
  }
  __syncthreads();
  uint16_t* dst = reinterpret_cast<uint16_t*>(vt) + ((size_t)g * nb + j) * D * BLK;
  constexpr int OCH = BLK / 8;  // 16-byte chunks per channel row
  for (int n = threadIdx.x; n < D * OCH; n += 256) {
    const int e = n / OCH, c = n % OCH;
    u32x4 w;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int p0 = c * 8 + 2 * t, p1 = p0 + 1;
      const int k0 = (p0 & ~15) + key_of_pos(p0 & 15), k1 = (p1 & ~15) + key_of_pos(p1 & 15);
      w[t] = (uint32_t)tile[k0][e] | ((uint32_t)tile[k1][e] << 16);
    }
    *reinterpret_cast<u32x4*>(dst + (size_t)e * BLK + c * 8) = w;
  }
}

// ------------------------------------------------------------------ bf16 attention

// Maps the launch index to (query head, query block): query blocks in
// decreasing order (causal rows get longer with i), the G heads of one KV
// head on one XCD in consecutive dispatch slots.
__device__ __forceinline__ void work_item(int x, int Hq, int Hkv, int nb, int& h, int& i) {
  const int G = Hq / Hkv;
  const int nunits = Hkv * nb;
  int u, hh;
  if ((nunits & 7) == 0) {
    const int xcd = x & 7, t = x >> 3;
    hh = t % G;
    u = (t / G) * 8 + xcd;
  } else {
    u = x / G;
    hh = x % G;
  }
  i = nb - 1 - u / Hkv;
  h = (u % Hkv) * G + hh;
}

template <int D, int BLK>
__global__ void __launch_bounds__(BLK * 2) __attribute__((amdgpu_waves_per_eu(2, 2))) attn_bf16_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ vt,
    const int32_t* __restrict__ row_count, const int32_t* __restrict__ col_idx, __bf16* __restrict__ out,
    int Hq, int Hkv, int nb, int causal, float cscale) {
  constexpr int NTHR = BLK * 2;  // BLK/32 waves
  constexpr int KCH = D / 8;     // 16-byte chunks per K row
  constexpr int VCH = BLK / 8;   // 16-byte chunks per Vt row
  constexpr int MT = BLK / 32;   // 32-key tiles
  constexpr int NT = D / 32;     // 32-channel tiles of O
  constexpr int DK = D / 16;     // MFMA k-steps over d
  __shared__ __attribute__((aligned(16))) uint8_t lds_k[BLK * D * 2];
  __shared__ __attribute__((aligned(16))) uint8_t lds_v[D * BLK * 2];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n32 = lane & 31, half = lane >> 5;
  int h, i;
  work_item(blockIdx.x, Hq, Hkv, nb, h, i);
  const int G = Hq / Hkv;
  const int g = h / G;
  const int qr = wave * 32 + n32;  // query row inside the block
  const int x = i * BLK + qr;

  bf16x8 qf[DK];
  {
    const bf16x8* src = reinterpret_cast<const bf16x8*>(q + ((size_t)x * Hq + h) * D);
#pragma unroll
    for (int c = 0; c < DK; ++c) qf[c] = src[2 * c + half];
  }

  f32x16 oacc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) oacc[t] = f32x16{};
  float mrow = -INFINITY, lrow = 0.0f;

  const size_t row = (size_t)h * nb + i;
  const int cnt = min(max(row_count[row], 0), nb);
  const int32_t* lst = col_idx + row * nb;
  const uint8_t* kbase = reinterpret_cast<const uint8_t*>(k);
  const uint8_t* vbase = reinterpret_cast<const uint8_t*>(vt);

  for (int c = 0; c < cnt; ++c) {
    const int j = min(max(lst[c], 0), nb - 1);
    if (causal && j > i) continue;
    __syncthreads();  // previous tile fully consumed
#pragma unroll
    for (int it = 0; it < (BLK * KCH) / NTHR; ++it) {
      const int n = threadIdx.x + it * NTHR;
      const int r = n / KCH, ch = n % KCH;
      const u32x4 w = *reinterpret_cast<const u32x4*>(kbase + (((size_t)(j * BLK + r) * Hkv + g) * D + ch * 8) * 2);
      *reinterpret_cast<u32x4*>(lds_k + r * D * 2 + ((ch ^ (r & (KCH - 1))) << 4)) = w;
    }
#pragma unroll
    for (int it = 0; it < (D * VCH) / NTHR; ++it) {
      const int n = threadIdx.x + it * NTHR;
      const int r = n / VCH, ch = n % VCH;
      const u32x4 w = *reinterpret_cast<const u32x4*>(vbase + ((((size_t)g * nb + j) * D + r) * BLK + ch * 8) * 2);
      *reinterpret_cast<u32x4*>(lds_v + r * BLK * 2 + ((ch ^ (r & (VCH - 1))) << 4)) = w;
    }
    __syncthreads();

    // S^T = K Q^T
    f32x16 sacc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      sacc[mt] = f32x16{};
      const int r = mt * 32 + n32;
#pragma unroll
      for (int cc = 0; cc < DK; ++cc) {
        const int ch = 2 * cc + half;
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(lds_k + r * D * 2 + ((ch ^ (r & (KCH - 1))) << 4));
        sacc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[cc], sacc[mt], 0, 0, 0);
      }
    }

    // online softmax in base 2
    const bool diag = causal && (j == i);
    float tmax = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int key = mt * 32 + 8 * (v >> 2) + 4 * half + (v & 3);
        if (diag && key > qr) sacc[mt][v] = -INFINITY;
        tmax = fmaxf(tmax, sacc[mt][v]);
      }
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    const float mnew = fmaxf(mrow, tmax * cscale);
    const float alpha = exp2_approx(mrow - mnew);
    float psum = 0.0f;
    bf16x8 pf[MT][2];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
      for (int p2 = 0; p2 < 2; ++p2) {
        u32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p0 = exp2_approx(__builtin_fmaf(sacc[mt][8 * p2 + 2 * e], cscale, -mnew));
          const float p1 = exp2_approx(__builtin_fmaf(sacc[mt][8 * p2 + 2 * e + 1], cscale, -mnew));
          psum += p0 + p1;
          w[e] = pack_bf16x2(p0, p1);
        }
        pf[mt][p2] = __builtin_bit_cast(bf16x8, w);
      }
    }
    lrow = lrow * alpha + psum;
    mrow = mnew;
#pragma unroll
    for (int t = 0; t < NT; ++t) oacc[t] *= alpha;

    // O^T += Vt P^T
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int r = t * 32 + n32;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
        for (int p2 = 0; p2 < 2; ++p2) {
          const int ch = mt * 4 + 2 * p2 + half;
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(lds_v + r * BLK * 2 + ((ch ^ (r & (VCH - 1))) << 4));
          oacc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[mt][p2], oacc[t], 0, 0, 0);
        }
      }
    }
  }

  const float ltot = lrow + __shfl_xor(lrow, 32);
  const float inv = ltot > 0.0f ? 1.0f / ltot : 0.0f;
  uint16_t* dst = reinterpret_cast<uint16_t*>(out) + ((size_t)x * Hq + h) * D;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
#pragma unroll
    for (int v4 = 0; v4 < 4; ++v4) {
      const int e = t * 32 + 8 * v4 + 4 * half;
      u32x2 w;
      w[0] = pack_bf16x2(oacc[t][4 * v4] * inv, oacc[t][4 * v4 + 1] * inv);
      w[1] = pack_bf16x2(oacc[t][4 * v4 + 2] * inv, oacc[t][4 * v4 + 3] * inv);
      *reinterpret_cast<u32x2*>(dst + e) = w;
    }
  }
}

// ------------------------------------------------------------------ fp32 attention

template <int D, int BLK>
__global__ void __launch_bounds__(BLK) attn_f32_kernel(const float* __restrict__ q, const float* __restrict__ k,
                                                       const float* __restrict__ v,
                                                       const int32_t* __restrict__ row_count,
                                                       const int32_t* __restrict__ col_idx,
                                                       float* __restrict__ out, int Hq, int Hkv, int nb,
                                                       int causal, float cscale) {
  extern __shared__ float smem[];
  float* ks = smem;             // [BLK][D]
  float* vs = smem + BLK * D;   // [BLK][D]
  const int h = blockIdx.x % Hq;
  const int i = nb - 1 - blockIdx.x / Hq;
  const int g = h / (Hq / Hkv);
  const int qr = threadIdx.x;
  const int x = i * BLK + qr;
  float qv[D], o[D];
#pragma unroll
  for (int e = 0; e < D; ++e) {
    qv[e] = q[((size_t)x * Hq + h) * D + e] * cscale;
    o[e] = 0.0f;
  }
  float m = -INFINITY, l = 0.0f;
  const size_t row = (size_t)h * nb + i;
  const int cnt = min(max(row_count[row], 0), nb);
  for (int c = 0; c < cnt; ++c) {
    const int j = min(max(col_idx[row * nb + c], 0), nb - 1);
    if (causal && j > i) continue;
    __syncthreads();
    for (int n = threadIdx.x; n < BLK * D; n += BLK) {
      const int r = n / D, e = n % D;
      const size_t src = ((size_t)(j * BLK + r) * Hkv + g) * D + e;
      ks[n] = k[src];
      vs[n] = v[src];
    }
    __syncthreads();
    const int ylast = (causal && j == i) ? qr : BLK - 1;
    for (int y = 0; y <= ylast; ++y) {
      float s = 0.0f;
#pragma unroll
      for (int e = 0; e < D; ++e) s += qv[e] * ks[y * D + e];
      if (s > m) {
        const float a = exp2_approx(m - s);
        l *= a;
#pragma unroll
        for (int e = 0; e < D; ++e) o[e] *= a;
        m = s;
      }
      const float p = exp2_approx(s - m);
      l += p;
#pragma unroll
      for (int e = 0; e < D; ++e) o[e] += p * vs[y * D + e];
    }
  }
  const float inv = l > 0.0f ? 1.0f / l : 0.0f;
#pragma unroll
  for (int e = 0; e < D; ++e) out[((size_t)x * Hq + h) * D + e] = o[e] * inv;
}

}  // namespace

hipError_t launch_transpose_v(const Geometry& g, const void* v, void* vt, hipStream_t st) {
  const dim3 grid((unsigned)(g.Hkv * g.nb));
  const __bf16* vv = static_cast<const __bf16*>(v);
  __bf16* out = static_cast<__bf16*>(vt);
  if (g.d == 128 && g.B == 128) transpose_v_kernel<128, 128><<<grid, 256, 0, st>>>(vv, out, g.Hkv, g.nb);
  else if (g.d == 128 && g.B == 64) transpose_v_kernel<128, 64><<<grid, 256, 0, st>>>(vv, out, g.Hkv, g.nb);
  else if (g.d == 64 && g.B == 128) transpose_v_kernel<64, 128><<<grid, 256, 0, st>>>(vv, out, g.Hkv, g.nb);
  else transpose_v_kernel<64, 64><<<grid, 256, 0, st>>>(vv, out, g.Hkv, g.nb);
  return hipGetLastError();
}

hipError_t launch_attention(const Geometry& g, const void* q, const void* k, const void* v,
                            const void* vt, const int32_t* row_count, const int32_t* col_idx,
                            void* out, hipStream_t st) {
  const float cscale = (1.0f / sqrtf((float)g.d)) * 1.4426950408889634f;
  const dim3 grid((unsigned)(g.Hq * g.nb));
  if (g.bf16) {
    const __bf16* qq = static_cast<const __bf16*>(q);
    const __bf16* kk = static_cast<const __bf16*>(k);
    const __bf16* vv = static_cast<const __bf16*>(vt);
    __bf16* oo = static_cast<__bf16*>(out);
#define RR_ATTN_CASE(DV, BV)                                                                      \
  if (g.d == DV && g.B == BV) {                                                                   \
    attn_bf16_kernel<DV, BV><<<grid, BV * 2, 0, st>>>(qq, kk, vv, row_count, col_idx, oo, g.Hq,    \
                                                      g.Hkv, g.nb, g.causal, cscale);            \
    return hipGetLastError();                                                                     \
  }
    RR_ATTN_CASE(128, 128)
    RR_ATTN_CASE(128, 64)
    RR_ATTN_CASE(64, 128)
    RR_ATTN_CASE(64, 64)
#undef RR_ATTN_CASE
    return hipErrorInvalidValue;
  }
  const float* qq = static_cast<const float*>(q);
  const float* kk = static_cast<const float*>(k);
  const float* vv = static_cast<const float*>(v);
  float* oo = static_cast<float*>(out);
#define RR_F32_CASE(DV, BV)                                                                       \
  if (g.d == DV && g.B == BV) {                                                                   \
    const size_t lds = 2 * (size_t)BV * DV * sizeof(float);                                       \
    hipError_t fe = hipFuncSetAttribute(reinterpret_cast<const void*>(&attn_f32_kernel<DV, BV>),    \
                                        hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);     \
    if (fe != hipSuccess) return fe;                                                              \
    attn_f32_kernel<DV, BV><<<grid, BV, lds, st>>>(qq, kk, vv, row_count, col_idx, oo, g.Hq, g.Hkv, \
                                                   g.nb, g.causal, cscale);                     \
    return hipGetLastError();                                                                     \
  }
  RR_F32_CASE(128, 128)
  RR_F32_CASE(128, 64)
  RR_F32_CASE(64, 128)
  RR_F32_CASE(64, 64)
#undef RR_F32_CASE
  return hipErrorInvalidValue;
}

}  // namespace rr
