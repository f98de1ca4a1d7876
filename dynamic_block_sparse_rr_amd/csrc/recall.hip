// Mass recall of a block selection against full attention: for every row
// (head h, query block i), the mean over the row's queries (B, or fewer in a
// short last block) of the share of
// each query's full-attention softmax mass that lies on keys of the row's
// selected blocks. This puts a number on what the Figure 4 and Figure 5
// captions of "RRAttention: Dynamic Block Sparse Attention via Per-Head
// Round-Robin Shifts for Long-Context Inference" show as pictures (the
// full-attention ground truth next to the selected blocks).
//
// Per query x with logits a_y = Q[x,h] . K[y,g] / sqrt(d) over every
// admissible key y (y <= x under the causal flag):
//   r(x) = sum_{y in selected blocks} exp(a_y - m) / sum_{y admissible} exp(a_y - m)
// computed in one pass over all candidate key blocks with a running maximum m
// shared by the two sums (both are rescaled together when m grows).
//
// bfloat16: one workgroup of B/32 waves per row, each wave 32 queries; the
// key tile is copied to LDS with buffer loads (double-buffered, one LDS object
// per stage so the next copy overlaps the current block) and S^T = K Q^T runs
// on v_mfma_f32_32x32x16_bf16 (lane = one query, 64 of the block's keys per
// lane half). float32: one thread per query, the key tile in LDS.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rr_kernels.h"

namespace rr {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

template <int D, int BLK>
struct RecallCfg {
  static constexpr int NW = BLK / 32;              // waves, 32 queries each
  static constexpr int NTHR = NW * 64;
  static constexpr int MT = BLK / 32;              // 32-key subtiles of a block
  static constexpr int DK = D / 16;                // MFMA k-steps over d
  static constexpr int TILE = BLK * D * 2;         // bytes of one K tile
  static constexpr int KCH = D / 8;                // 16-byte chunks per K row
  static constexpr int RPC = NTHR / KCH;           // tile rows covered by one copy
  static constexpr int NDMA = TILE / (NTHR * 16);  // copies per thread per tile
  static_assert(NTHR % KCH == 0 && NDMA * NTHR * 16 == TILE, "copy geometry");
};

// The key tile lives in LDS as rows of 16-byte chunks, chunk c of row r stored
// at position c ^ (r mod KCH), so the 32 rows an MFMA operand read touches
// fall in distinct banks. Lane l of a wave's copy lands at 16*l past the
// wave's slot, so thread t fetches the source chunk that belongs at its
// position: row n*RPC + t/KCH, chunk (t mod KCH) ^ (row mod KCH), i.e. one
// base offset, a fixed step per copy and an XOR of the copy's phase.
template <int D, int BLK>
__device__ __forceinline__ void recall_copy(__amdgpu_buffer_rsrc_t rsrc, uint32_t off, uint32_t step, int wave,
                                            uint8_t* dst) {
  typedef RecallCfg<D, BLK> C;
#pragma unroll
  for (int n = 0; n < C::NDMA; ++n)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rsrc,
        reinterpret_cast<__attribute__((address_space(3))) void*>(
            reinterpret_cast<uintptr_t>(dst + (n * C::NTHR + wave * 64) * 16)),
        16, (int)(n * step + (off ^ (((n * C::RPC) & (C::KCH - 1)) << 4))), 0, 0, 0);
}

// One key block for one wave: scores, running maximum, and the two sums.
// masked: keys with index > klim inside the block are masked (the causal
// diagonal block: the lane's query row; a short last block: its last key).
template <int D, int BLK>
__device__ __forceinline__ void recall_tile(const uint8_t* lds_k, int kro, const bf16x8 (&qf)[D / 16], int half,
                                            int klim, bool masked, bool sel, float cscale, float& m, float& lall,
                                            float& lsel) {
  typedef RecallCfg<D, BLK> C;
  f32x16 sacc[C::MT];
#pragma unroll
  for (int mt = 0; mt < C::MT; ++mt) {
    f32x16 acc = {};
#pragma unroll
    for (int cc = 0; cc < C::DK; ++cc) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(lds_k + mt * 32 * D * 2 + (kro ^ (cc << 5)));
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[cc], acc, 0, 0, 0);
    }
    sacc[mt] = acc;
  }
  if (masked) {
#pragma unroll
    for (int mt = 0; mt < C::MT; ++mt)
#pragma unroll
      for (int v = 0; v < 16; ++v)
        if (mt * 32 + 8 * (v >> 2) + 4 * half + (v & 3) > klim) sacc[mt][v] = -INFINITY;
  }
  float tmax = -INFINITY;
#pragma unroll
  for (int mt = 0; mt < C::MT; ++mt)
#pragma unroll
    for (int v = 0; v < 16; ++v) tmax = fmaxf(tmax, sacc[mt][v]);
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(tmax), __float_as_uint(tmax), false, false);
  tmax = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
  const float mnew = fmaxf(m, tmax * cscale);  // every query sees at least one key of block 0
  const float alpha = exp2_fast(m - mnew);     // 0 while m is -inf
  lall *= alpha;
  lsel *= alpha;
  m = mnew;
  float s0 = 0.0f, s1 = 0.0f;
#pragma unroll
  for (int mt = 0; mt < C::MT; ++mt)
#pragma unroll
    for (int v = 0; v < 16; v += 2) {
      s0 += exp2_fast(__builtin_fmaf(sacc[mt][v], cscale, -mnew));
      s1 += exp2_fast(__builtin_fmaf(sacc[mt][v + 1], cscale, -mnew));
    }
  const float s = s0 + s1;
  lall += s;
  if (sel) lsel += s;
}

// Mean over the workgroup's queries of r(x), written by thread 0; fixed
// reduction order (lanes 0..31 by a shuffle tree, then the waves in order).
template <int NW>
__device__ __forceinline__ void block_mean(float r, int lane, int wave, float* red, float* dst, float inv_count) {
#pragma unroll
  for (int o = 16; o >= 1; o >>= 1) r += __shfl_xor(r, o);
  if (lane == 0) red[wave] = r;
  __syncthreads();
  if (threadIdx.x == 0) {
    float t = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) t += red[w];
    *dst = t * inv_count;
  }
}

template <int D, int BLK>
__global__ void __launch_bounds__(BLK * 2) recall_bf16_kernel(const __bf16* __restrict__ q,
                                                               const __bf16* __restrict__ k,
                                                               const int32_t* __restrict__ row_count,
                                                               const int32_t* __restrict__ col_idx,
                                                               float* __restrict__ recall, int Hq, int Hkv, int nb,
                                                               int causal, float cscale, int L) {
  typedef RecallCfg<D, BLK> C;
  __shared__ __attribute__((aligned(1024))) uint8_t lds_k0[C::TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t lds_k1[C::TILE];
  __shared__ float red[C::NW];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n32 = lane & 31, half = lane >> 5;
  const int qr = wave * 32 + n32;
  // long causal rows first
  const int h = blockIdx.x % Hq;
  const int i = nb - 1 - (int)(blockIdx.x / Hq);
  const int g = h / (Hq / Hkv);
  const int x = i * BLK + qr;

  bf16x8 qf[C::DK];
  if (x < L) {
    const bf16x8* src = reinterpret_cast<const bf16x8*>(q + ((size_t)x * Hq + h) * D);
#pragma unroll
    for (int c = 0; c < C::DK; ++c) qf[c] = src[2 * c + half];
  } else {  // past the end of a short last block: not counted
#pragma unroll
    for (int c = 0; c < C::DK; ++c) qf[c] = bf16x8{};
  }
  const int kr = tid / C::KCH, kc = (tid % C::KCH) ^ (kr & (C::KCH - 1));
  const uint32_t koff = (uint32_t)((kr * Hkv * D + kc * 8) * 2);
  const uint32_t kstep = (uint32_t)(C::RPC * Hkv * D * 2);
  const int kro = n32 * D * 2 + ((half ^ (n32 & (C::KCH - 1))) << 4);
  const uint8_t* kg = reinterpret_cast<const uint8_t*>(k) + (size_t)g * D * 2;
  const size_t kstride = (size_t)BLK * Hkv * D * 2;
  const uint32_t kbytes = (uint32_t)((BLK - 1) * Hkv * D * 2 + D * 2);
  const size_t k_bytes = (size_t)L * Hkv * D * 2;  // the whole K tensor
  auto copy = [&](int j, uint8_t* dst) {
    // cut where the tensor ends: a short last block reads zeros past L
    const size_t start = (size_t)g * D * 2 + (size_t)j * kstride;
    const uint32_t kb = start + kbytes <= k_bytes ? kbytes : (uint32_t)(k_bytes - start);
    recall_copy<D, BLK>(__builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(kg + (size_t)j * kstride), 0,
                                                          (int)kb, 0x00020000),
                        koff, kstep, wave, dst);
  };
  const int ltail = L - (nb - 1) * BLK;  // keys in the last block

  const size_t row = (size_t)h * nb + i;
  const int cnt = min(max(row_count[row], 0), nb);
  const int32_t* lst = col_idx + row * nb;
  const int jlast = causal ? i : nb - 1;
  int c = 0;  // next unmatched list entry (the list is ascending)
  float m = -INFINITY, lall = 0.0f, lsel = 0.0f;

  constexpr int kWaitAll = 0x0070;  // vmcnt(0) lgkmcnt(0)
  copy(0, lds_k0);
  // block j's tile is in kc_; the copy of block j + 1 goes to kn_
  auto step = [&](int j, const uint8_t* kc_, uint8_t* kn_) {
    __builtin_amdgcn_s_waitcnt(kWaitAll);
    __builtin_amdgcn_s_barrier();
    if (j + 1 <= jlast) copy(j + 1, kn_);
    bool sel = false;
    if (c < cnt && lst[c] == j) {
      sel = true;
      ++c;
    }
    const bool diag = causal && j == i, shortblk = j == nb - 1 && ltail < BLK;
    recall_tile<D, BLK>(kc_, kro, qf, half, diag ? qr : ltail - 1, diag || shortblk, sel, cscale, m, lall, lsel);
  };
  for (int j = 0; j <= jlast; j += 2) {
    step(j, lds_k0, lds_k1);
    if (j + 1 <= jlast) step(j + 1, lds_k1, lds_k0);
  }
  const float ta = lall + __shfl_xor(lall, 32);
  const float ts = lsel + __shfl_xor(lsel, 32);
  // lanes 32..63 hold the same queries; queries past L are not counted
  const float r = (half == 0 && x < L) ? ts / ta : 0.0f;
  block_mean<C::NW>(r, lane, wave, red, recall + row, 1.0f / (float)min(BLK, L - i * BLK));
}

// float32: thread = query; the key tile of each candidate block in LDS.
template <int D, int BLK>
__global__ void __launch_bounds__(BLK) recall_f32_kernel(const float* __restrict__ q, const float* __restrict__ k,
                                                         const int32_t* __restrict__ row_count,
                                                         const int32_t* __restrict__ col_idx,
                                                         float* __restrict__ recall, int Hq, int Hkv, int nb,
                                                         int causal, float cscale, int L) {
  __shared__ float ks[BLK * D];
  __shared__ float red[BLK / 64 > 0 ? BLK / 64 : 1];
  const int h = blockIdx.x % Hq;
  const int i = nb - 1 - (int)(blockIdx.x / Hq);
  const int g = h / (Hq / Hkv);
  const int qr = threadIdx.x;
  const int x = i * BLK + qr;
  float qv[D];
#pragma unroll
  for (int e = 0; e < D; ++e) qv[e] = x < L ? q[((size_t)x * Hq + h) * D + e] * cscale : 0.0f;
  const size_t row = (size_t)h * nb + i;
  const int cnt = min(max(row_count[row], 0), nb);
  const int32_t* lst = col_idx + row * nb;
  const int jlast = causal ? i : nb - 1;
  int c = 0;
  float m = -INFINITY, lall = 0.0f, lsel = 0.0f;
  for (int j = 0; j <= jlast; ++j) {
    bool sel = false;
    if (c < cnt && lst[c] == j) {
      sel = true;
      ++c;
    }
    __syncthreads();
    for (int n = threadIdx.x; n < BLK * D; n += BLK) {
      const int r = n / D, e = n % D;
      ks[n] = j * BLK + r < L ? k[((size_t)(j * BLK + r) * Hkv + g) * D + e] : 0.0f;
    }
    __syncthreads();
    const int ylast = min((causal && j == i) ? qr : BLK - 1, L - 1 - j * BLK);
    for (int y = 0; y <= ylast; ++y) {
      float s = 0.0f;
#pragma unroll
      for (int e = 0; e < D; ++e) s += qv[e] * ks[y * D + e];
      if (s > m) {
        const float a = exp2_fast(m - s);
        lall *= a;
        lsel *= a;
        m = s;
      }
      const float p = exp2_fast(s - m);
      lall += p;
      if (sel) lsel += p;
    }
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float r = x < L ? lsel / lall : 0.0f;  // queries past L are not counted
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) r += __shfl_xor(r, o);
  if (lane == 0) red[wave] = r;
  __syncthreads();
  if (threadIdx.x == 0) {
    float t = 0.0f;
    for (int w = 0; w < BLK / 64; ++w) t += red[w];
    recall[row] = t / (float)min(BLK, L - i * BLK);
  }
}

}  // namespace

hipError_t launch_recall(const Geometry& g, const void* q, const void* k, const int32_t* row_count,
                         const int32_t* col_idx, float* recall, hipStream_t st) {
  const float cscale = (1.0f / sqrtf((float)g.d)) * 1.4426950408889634f;
  const dim3 grid((unsigned)(g.Hq * g.nb));
#define RR_RECALL_CASE(DV, BV)                                                                          \
  if (g.d == DV && g.B == BV) {                                                                         \
    if (g.bf16)                                                                                         \
      recall_bf16_kernel<DV, BV><<<grid, BV * 2, 0, st>>>(static_cast<const __bf16*>(q),               \
                                                          static_cast<const __bf16*>(k), row_count,     \
                                                          col_idx, recall, g.Hq, g.Hkv, g.nb, g.causal, \
                                                          cscale, g.L);                                 \
    else                                                                                                \
      recall_f32_kernel<DV, BV><<<grid, BV, 0, st>>>(static_cast<const float*>(q),                     \
                                                     static_cast<const float*>(k), row_count, col_idx,  \
                                                     recall, g.Hq, g.Hkv, g.nb, g.causal, cscale, g.L); \
    return hipGetLastError();                                                                           \
  }
  RR_RECALL_CASE(128, 128)
  RR_RECALL_CASE(128, 64)
  RR_RECALL_CASE(64, 128)
  RR_RECALL_CASE(64, 64)
#undef RR_RECALL_CASE
  return hipErrorInvalidValue;
}

}  // namespace rr
