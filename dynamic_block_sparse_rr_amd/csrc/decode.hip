// Decode step of RRAttention on gfx950: one new query per head against the
// KV cache. The TL;DR of "RRAttention: Dynamic Block Sparse Attention via
// Per-Head Round-Robin Shifts for Long-Context Inference" names decode-stage
// sparsification as future work; this applies the prefill's pieces with the
// query itself in place of the round-robin samples:
//   decode_scores   workgroup (KV head, chunk of 256 strides): the G query
//                   heads' scores against the pooled cache keys (stride means,
//                   as in prefill) on MFMA, with each chunk's max and exp-sum
//                   and its key blocks' exp-sums;
//   (select)        search.hip's decode_select_kernel, one workgroup per head:
//                   the chunks merged into one softmax over the strides, summed
//                   into block masses, then the Top-tau prefix of the (mass
//                   desc, index asc) order plus the last block;
//   decode_attn     split-K attention over the selected blocks: workgroup
//                   (KV head, equal share of the blocks any of its G query
//                   heads selected) reads each block once for all G heads, with
//                   an online softmax per head, and leaves (max, sum, O)
//                   partials;
//   decode_combine  one workgroup per head merges its partials in split order.
// bf16 with G <= 8 takes the group kernels; other shapes take per-head ones
// with the same results. The step is memory-bound: the K and V of the union of
// each KV head's selections, read once, a few hundred MB at 128K.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "rr_kernels.h"

namespace rr {
namespace {

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float to_float(__bf16 x) { return (float)x; }
__device__ __forceinline__ float to_float(float x) { return x; }

// dot product of a row of D values of T with the float query in LDS, in
// element order, loaded 16 bytes at a time
template <typename T, int D>
__device__ __forceinline__ float row_dot(const T* __restrict__ row, const float* __restrict__ qs) {
  constexpr int E = 16 / sizeof(T);
  typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
  float acc = 0.0f;
#pragma unroll
  for (int c = 0; c < D / E; ++c) {
    const u32x4v w = reinterpret_cast<const u32x4v*>(row)[c];
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc = __builtin_fmaf(qs[c * 8 + 2 * e], __uint_as_float(w[e] << 16), acc);
        acc = __builtin_fmaf(qs[c * 8 + 2 * e + 1], __uint_as_float(w[e] & 0xffff0000u), acc);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) acc = __builtin_fmaf(qs[c * 4 + e], __uint_as_float(w[e]), acc);
    }
  }
  return acc;
}

// Reductions over a workgroup of NTHR threads in a fixed order: the lanes of a
// wave by a shuffle tree, then the waves in order (the result in every thread).
template <int NTHR>
__device__ __forceinline__ float wg_max(float v, float* red) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int w = 1; w < NTHR / 64; ++w) r = fmaxf(r, red[w]);
  return r;
}

template <int NTHR>
__device__ __forceinline__ float wg_sum(float v, float* red) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int w = 1; w < NTHR / 64; ++w) r += red[w];
  return r;
}

// Scores of one head's new query against a chunk of kDecodeChunk pooled
// keys (thread = stride): z_t = q . Kbar_t * cscale (base-2 units); the
// chunk's maximum cm, its sum of exp2(z - cm), and per key block of the chunk
// (r strides; r divides the chunk) bsum_j = sum of exp2(z_t - cm) over its
// strides, so that a block's mass is bsum_j * exp2(cm - M) / (softmax sum).
constexpr int kDecodeChunk = 256;

template <typename T, int D>
__global__ void __launch_bounds__(kDecodeChunk) decode_scores_kernel(const T* __restrict__ q,
                                                                     const T* __restrict__ kbar,
                                                                     float* __restrict__ bsum, float* __restrict__ zpart,
                                                                     int Hq, int Hkv, int ns, int nb, int r,
                                                                     int nchunk, float cscale) {
  __shared__ float qs[D];
  __shared__ float red[kDecodeChunk / 64];
  __shared__ float ps[kDecodeChunk];
  const int h = blockIdx.x / nchunk, ch = blockIdx.x % nchunk, g = h / (Hq / Hkv);
  for (int e = threadIdx.x; e < D; e += kDecodeChunk) qs[e] = to_float(q[(size_t)h * D + e]);
  __syncthreads();
  const int t = ch * kDecodeChunk + threadIdx.x;
  float zt = -INFINITY;
  if (t < ns) zt = row_dot<T, D>(kbar + ((size_t)t * Hkv + g) * D, qs) * cscale;
  const float cm = wg_max<kDecodeChunk>(zt, red);
  const float p = t < ns ? exp2_fast(zt - cm) : 0.0f;
  ps[threadIdx.x] = p;
  const float cs = wg_sum<kDecodeChunk>(p, red);  // its barriers also publish ps
  const int nbc = kDecodeChunk / r;
  if ((int)threadIdx.x < nbc) {
    const int j = ch * nbc + threadIdx.x;
    if (j < nb) {
      float a = 0.0f;
      for (int i = 0; i < r; ++i) a += ps[threadIdx.x * r + i];
      bsum[(size_t)h * nb + j] = a;
    }
  }
  if (threadIdx.x == 0) {
    zpart[((size_t)h * nchunk + ch) * 2] = cm;
    zpart[((size_t)h * nchunk + ch) * 2 + 1] = cs;
  }
}

constexpr int kDecodeThreads = 256;

// Split-K attention of one head's query (shapes without the group kernel) over
// the selected blocks among [sp*kDecodeSplit, sp*kDecodeSplit + kDecodeSplit).
// Per block: thread pairs (2i, 2i+1) score key i over the two halves of d;
// then thread t accumulates channels 8*(t%CG)..+7 of P V over keys
// (t/CG)*KG..+KG-1 with 16-byte loads, and the key groups are summed in LDS
// in a fixed order into the workgroup's O.
template <typename T, int D, int BLK>
__global__ void __launch_bounds__(kDecodeThreads) decode_attn_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, const uint8_t* __restrict__ sel, int nbp,
    float* __restrict__ part, int Hq, int Hkv, int nb, int L, float cscale, int nsplit) {
  constexpr int CG = D / 8;                   // channel groups of 8 (16 bytes of bf16)
  constexpr int NKG = kDecodeThreads / CG;    // key groups
  constexpr int KG = BLK / NKG;               // keys per group
  static_assert(2 * BLK <= kDecodeThreads && KG >= 1, "decode tile shape: a thread pair per key");
  __shared__ float qs[D];
  __shared__ float ps[BLK];
  __shared__ float acc_s[NKG][D];
  __shared__ float red[kDecodeThreads / 64];
  const int h = blockIdx.x / nsplit, sp = blockIdx.x % nsplit, g = h / (Hq / Hkv);
  const int t = threadIdx.x;
  for (int e = t; e < D; e += kDecodeThreads) qs[e] = to_float(q[(size_t)h * D + e]);
  __syncthreads();
  const int j0 = sp * kDecodeSplit, j1 = min(j0 + kDecodeSplit, nb);
  const int cg = t % CG, kgi = t / CG;
  float m = -INFINITY, l = 0.0f;
  float o[8];  // channels 8*cg.. of the key group's partial, merged each block into O (threads t < D own O[t])
  float O = 0.0f;
  for (int j = j0; j < j1; ++j) {
    if (!sel[(size_t)h * nbp + j]) continue;  // the same for the whole workgroup
    const int nkeys = min(BLK, L - j * BLK);
    // scores: thread 2i + hf scores half hf of key i (keys beyond BLK / nkeys idle)
    const int key = t >> 1, hf = t & 1;
    float part_dot = 0.0f;
    if (key < nkeys)
      part_dot = row_dot<T, D / 2>(k + ((size_t)(j * BLK + key) * Hkv + g) * D + hf * (D / 2), qs + hf * (D / 2));
    part_dot += __shfl_xor(part_dot, 1);
    const float sc = (key < nkeys && hf == 0) ? part_dot * cscale : -INFINITY;
    const float mnew = fmaxf(m, wg_max<kDecodeThreads>(sc, red));
    const float alpha = exp2_fast(m - mnew);  // 0 on the first block
    const float p = (key < nkeys && hf == 0) ? exp2_fast(sc - mnew) : 0.0f;
    if (hf == 0 && key < BLK) ps[key] = p;
    l = l * alpha + wg_sum<kDecodeThreads>(p, red);  // its barriers also publish ps
    // P V for this thread's key group and channel group
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = 0.0f;
#pragma unroll
    for (int kk = 0; kk < KG; ++kk) {
      const int y = kgi * KG + kk;
      if (y < nkeys) {
        typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
        const float py = ps[y];
        if constexpr (sizeof(T) == 2) {
          const u32x4v w = *reinterpret_cast<const u32x4v*>(v + ((size_t)(j * BLK + y) * Hkv + g) * D + cg * 8);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            o[2 * e] = __builtin_fmaf(py, __uint_as_float(w[e] << 16), o[2 * e]);
            o[2 * e + 1] = __builtin_fmaf(py, __uint_as_float(w[e] & 0xffff0000u), o[2 * e + 1]);
          }
        } else {
#pragma unroll
          for (int half8 = 0; half8 < 2; ++half8) {
            const u32x4v w =
                *reinterpret_cast<const u32x4v*>(v + ((size_t)(j * BLK + y) * Hkv + g) * D + cg * 8 + half8 * 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) o[half8 * 4 + e] = __builtin_fmaf(py, __uint_as_float(w[e]), o[half8 * 4 + e]);
          }
        }
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) acc_s[kgi][cg * 8 + e] = o[e];
    __syncthreads();
    if (t < D) {
      float sum = 0.0f;
#pragma unroll
      for (int gi = 0; gi < NKG; ++gi) sum += acc_s[gi][t];
      O = O * alpha + sum;
    }
    m = mnew;
    __syncthreads();  // ps and acc_s are rewritten by the next block
  }
  float* dst = part + ((size_t)h * nsplit + sp) * (D + 2);
  if (t < D) dst[t] = O;
  if (t == 0) {
    dst[D] = m;
    dst[D + 1] = l;
  }
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Workgroup barrier for LDS only: global loads stay in flight across it.
#define RR_LDS_SYNC() asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory")

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Group decode attention: workgroup (KV head g, split sp) reads its share of
// the blocks that any of the G query heads of g selected (an equal run of
// them in block order), each once, and serves all G heads from it (heads that
// did not select a block give it probability 0). Per block:
//   QK  on v_mfma_f32_16x16x32_bf16, A = the G queries (rows, zero-padded to
//       16), B = 16 keys of the block (columns); wave w scores keys
//       [w*BLK/4, (w+1)*BLK/4);
//   softmax: wave w keeps the online (max, sum) of heads w, w+4, ..;
//   PV  on the VALU: thread (key group, chunk of 8 channels, 4 when G > 4)
//       accumulates the G heads' outputs over its keys; the key groups are summed once at the
//       end, in a fixed order.
// The next active block's K and V are loaded into a second register set while
// the current one is computed. sel: per-head selection flags [Hq][nbp].
template <int D, int BLK, int G>
__global__ void __launch_bounds__(256, 2) decode_group_attn_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    const uint8_t* __restrict__ sel, int nbp, float* __restrict__ part, int Hkv, int nb, int L, float cscale,
    int nsplit) {
  constexpr int NS = D / 32;        // 32-wide d slices of one MFMA
  constexpr int KT = BLK / 64;      // 16-key tiles per wave
  constexpr int CPT = G > 4 ? 4 : 8;  // channels per thread in the PV phase (G * CPT accumulators)
  constexpr int CG = D / CPT;         // channel chunks of a row
  constexpr int NKG = 256 / CG;       // key groups of the PV phase
  constexpr int KG = BLK / NKG;       // keys per group
  constexpr int HPW = (G + 3) / 4;    // heads per wave in the softmax phase
  typedef uint32_t vword __attribute__((ext_vector_type(CPT / 2)));
  static_assert(G >= 1 && G <= 8 && KT >= 1 && KG >= 1, "group decode shape");
  __shared__ float sc_s[G][BLK];
  __shared__ float ps_s[BLK][G];
  __shared__ float alpha_s[G];
  __shared__ int act_j[64], act_m[64];
  __shared__ int nact_s;
  __shared__ uint32_t wcount[4];
  __shared__ float red_s[4][G][D];

  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int g = blockIdx.x / nsplit, sp = blockIdx.x % nsplit;
  const size_t row = (size_t)Hkv * D;  // elements between consecutive keys

  // active blocks: those any of the G heads selected, ranked in block order;
  // this workgroup takes ranks [sp * per, sp * per + per), per = ceil(total /
  // nsplit) <= cb <= 64, so the work is even over the workgroups of g
  {
    const int c = (nb + 255) / 256;
    const int jlo = min(t * c, nb), jhi = min(jlo + c, nb);
    auto headmask = [&](int j) {
      int hm = 0;
#pragma unroll
      for (int hh = 0; hh < G; ++hh) hm |= (sel[(size_t)(g * G + hh) * nbp + j] != 0) << hh;
      return hm;
    };
    uint32_t own = 0;
    for (int j = jlo; j < jhi; ++j) own += headmask(j) != 0;
    uint32_t inc = own;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t y = __shfl_up(inc, o);
      if (lane >= o) inc += y;
    }
    if (lane == 63) wcount[w] = inc;
    __syncthreads();
    uint32_t rank = inc - own;
    for (int i = 0; i < w; ++i) rank += wcount[i];
    const uint32_t total = wcount[0] + wcount[1] + wcount[2] + wcount[3];
    const uint32_t per = (total + nsplit - 1) / nsplit;
    const uint32_t a0 = min(total, (uint32_t)sp * per), a1 = min(total, a0 + per);
    if (own > 0 && rank < a1 && rank + own > a0) {
      for (int j = jlo; j < jhi; ++j) {
        const int hm = headmask(j);
        if (hm) {
          if (rank >= a0 && rank < a1) {
            act_j[rank - a0] = j;
            act_m[rank - a0] = hm;
          }
          ++rank;
        }
      }
    }
    if (t == 0) nact_s = (int)(a1 - a0);
  }

  // queries: MFMA A operand, row = head lane % 16, d = 32 s + 8 (lane / 16) ..
  bf16x8 qa[NS];
  {
    const int hh = lane & 15;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (hh < G)
        x = *reinterpret_cast<const u32x4*>(q + (size_t)(g * G + hh) * D + 32 * s + 8 * (lane >> 4));
      qa[s] = __builtin_bit_cast(bf16x8, x);
    }
  }
  __syncthreads();
  const int nact = nact_s;

  const int cg = t % CG, kgi = t / CG;
  float o[G][CPT];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < CPT; ++e) o[h][e] = 0.0f;
  float mst[HPW], lst[HPW];
#pragma unroll
  for (int i = 0; i < HPW; ++i) {
    mst[i] = -INFINITY;
    lst[i] = 0.0f;
  }

  // K rows for the MFMA B operand and V chunks for the PV phase of block j;
  // the loads are unconditional (clamped rows) so that the next block's stay
  // in flight while the current one is computed
  auto load_k = [&](int j, u32x4 (&kr)[KT * NS]) {
    const int nkeys = min(BLK, L - j * BLK);
    const __bf16* kb = k + (size_t)j * BLK * row + (size_t)g * D;
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
      const int key = w * (BLK / 4) + kt * 16 + (lane & 15);
      const int kc = min(key, nkeys - 1);  // rows past the cache end: scores masked later
#pragma unroll
      for (int s = 0; s < NS; ++s)
        kr[kt * NS + s] = *reinterpret_cast<const u32x4*>(kb + (size_t)kc * row + 32 * s + 8 * (lane >> 4));
    }
  };
  auto load_v = [&](int j, vword (&vr)[KG]) {
    const int nkeys = min(BLK, L - j * BLK);
    const __bf16* vb = v + (size_t)j * BLK * row + (size_t)g * D;
#pragma unroll
    for (int kk = 0; kk < KG; ++kk) {
      const int y = kgi * KG + kk;
      // keys past the cache end read the last row and get probability 0
      vr[kk] = *reinterpret_cast<const vword*>(vb + (size_t)min(y, nkeys - 1) * row + CPT * cg);
    }
  };

  auto process = [&](int j, int hm, const u32x4 (&kr)[KT * NS], const vword (&vr)[KG]) {
    const int nkeys = min(BLK, L - j * BLK);
    // QK^T for this wave's keys
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
      f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int s = 0; s < NS; ++s)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[s], __builtin_bit_cast(bf16x8, kr[kt * NS + s]), acc, 0, 0,
                                                      0);
      const int key = w * (BLK / 4) + kt * 16 + (lane & 15);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int h = 4 * (lane >> 4) + i;
        if (h < G) sc_s[h][key] = acc[i] * cscale;
      }
    }
    RR_LDS_SYNC();
    // online softmax of heads w, w + 4, ..
#pragma unroll
    for (int hi = 0; hi < HPW; ++hi) {
      const int h = w + 4 * hi;
      if (h < G) {
        if ((hm >> h) & 1) {
          float x[BLK / 64];
          float bm = -INFINITY;
#pragma unroll
          for (int c = 0; c < BLK / 64; ++c) {
            const int key = lane + 64 * c;
            x[c] = key < nkeys ? sc_s[h][key] : -INFINITY;
            bm = fmaxf(bm, x[c]);
          }
          const float mnew = fmaxf(mst[hi], wave_max(bm));
          const float al = exp2_fast(mst[hi] - mnew);  // 0 on the head's first block
          float ls = 0.0f;
#pragma unroll
          for (int c = 0; c < BLK / 64; ++c) {
            const float p = exp2_fast(x[c] - mnew);
            ps_s[lane + 64 * c][h] = p;
            ls += p;
          }
          lst[hi] = lst[hi] * al + wave_sum(ls);
          mst[hi] = mnew;
          if (lane == 0) alpha_s[h] = al;
        } else {
#pragma unroll
          for (int c = 0; c < BLK / 64; ++c) ps_s[lane + 64 * c][h] = 0.0f;
          if (lane == 0) alpha_s[h] = 1.0f;
        }
      }
    }
    RR_LDS_SYNC();
    // P V
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float al = alpha_s[h];
#pragma unroll
      for (int e = 0; e < CPT; ++e) o[h][e] *= al;
    }
#pragma unroll
    for (int kk = 0; kk < KG; ++kk) {
      const int y = kgi * KG + kk;
      float vf[CPT];
#pragma unroll
      for (int e = 0; e < CPT / 2; ++e) {
        vf[2 * e] = __uint_as_float(vr[kk][e] << 16);
        vf[2 * e + 1] = __uint_as_float(vr[kk][e] & 0xffff0000u);
      }
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float p = ps_s[y][h];
#pragma unroll
        for (int e = 0; e < CPT; ++e) o[h][e] = __builtin_fmaf(p, vf[e], o[h][e]);
      }
    }
    // sc_s, ps_s and alpha_s are rewritten only after the next block's first
    // barrier, which every thread reaches after its reads here
  };

  u32x4 ka[KT * NS], kb2[KT * NS];
  vword va[KG], vb2[KG];
  if (nact > 0) {
    load_k(act_j[0], ka);
    load_v(act_j[0], va);
  }
  for (int a = 0; a < nact; a += 2) {
    {  // the next block, or this one again at the end (cache hits, unused)
      const int jn = act_j[a + 1 < nact ? a + 1 : a];
      load_k(jn, kb2);
      load_v(jn, vb2);
    }
    process(act_j[a], act_m[a], ka, va);
    if (a + 1 >= nact) break;
    {
      const int jn = act_j[a + 2 < nact ? a + 2 : a + 1];
      load_k(jn, ka);
      load_v(jn, va);
    }
    process(act_j[a + 1], act_m[a + 1], kb2, vb2);
  }

  // sum the key groups: within a wave by shuffles, then the 4 waves in order
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < CPT; ++e) {
      float x = o[h][e];
#pragma unroll
      for (int off = CG; off < 64; off <<= 1) x += __shfl_xor(x, off);
      o[h][e] = x;
    }
  __syncthreads();
  if (lane < CG) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < CPT; ++e) red_s[w][h][CPT * cg + e] = o[h][e];
  }
  __syncthreads();
  for (int idx = t; idx < G * D; idx += 256) {
    const int h = idx / D, c = idx % D;
    const float sum = ((red_s[0][h][c] + red_s[1][h][c]) + red_s[2][h][c]) + red_s[3][h][c];
    part[((size_t)(g * G + h) * nsplit + sp) * (D + 2) + c] = sum;
  }
  if (lane == 0) {
#pragma unroll
    for (int hi = 0; hi < HPW; ++hi) {
      const int h = w + 4 * hi;
      if (h < G) {
        float* dst = part + ((size_t)(g * G + h) * nsplit + sp) * (D + 2);
        dst[D] = mst[hi];
        dst[D + 1] = lst[hi];
      }
    }
  }
}

// Group decode scores: workgroup (KV head g, chunk of 256 strides) scores the
// G query heads of g against the chunk's pooled keys on
// v_mfma_f32_16x16x32_bf16 (A = the G queries, B = 16 pooled keys; wave w takes
// strides [64 w, 64 w + 64) of the chunk) and leaves, as the per-head kernel
// above, each head's chunk maximum and exp-sum (waves merged in order) and the
// chunk's block sums.
template <int D, int G>
__global__ void __launch_bounds__(256) decode_group_scores_kernel(const __bf16* __restrict__ q,
                                                                  const __bf16* __restrict__ kbar,
                                                                  float* __restrict__ bsum, float* __restrict__ zpart,
                                                                  int Hkv, int ns, int nb, int r, int nchunk,
                                                                  float cscale) {
  constexpr int NS = D / 32;
  __shared__ float wred[4][16];
  __shared__ float ps[G][256];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int g = blockIdx.x / nchunk, ch = blockIdx.x % nchunk;
  const size_t row = (size_t)Hkv * D;
  bf16x8 qa[NS];
  {
    const int hh = lane & 15;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (hh < G)
        x = *reinterpret_cast<const u32x4*>(q + (size_t)(g * G + hh) * D + 32 * s + 8 * (lane >> 4));
      qa[s] = __builtin_bit_cast(bf16x8, x);
    }
  }
  u32x4 kr[4][NS];
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) {
    const int t = ch * 256 + w * 64 + kt * 16 + (lane & 15);
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (t < ns) x = *reinterpret_cast<const u32x4*>(kbar + (size_t)t * row + (size_t)g * D + 32 * s + 8 * (lane >> 4));
      kr[kt][s] = x;
    }
  }
  float z[4][4], mx[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) mx[i] = -INFINITY;
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) {
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int s = 0; s < NS; ++s)
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[s], __builtin_bit_cast(bf16x8, kr[kt][s]), acc, 0, 0, 0);
    const int t = ch * 256 + w * 64 + kt * 16 + (lane & 15);
#pragma unroll
    for (int i = 0; i < 4; ++i) {  // row 4 (lane / 16) + i: a head of the group (or padding)
      z[kt][i] = t < ns ? acc[i] * cscale : -INFINITY;
      mx[i] = fmaxf(mx[i], z[kt][i]);
    }
  }
  // head rows 4 (lane / 16) + i: reduce over the 16 lanes of the row group, then the waves
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int o = 8; o >= 1; o >>= 1) mx[i] = fmaxf(mx[i], __shfl_xor(mx[i], o));
  if ((lane & 15) == 0)
#pragma unroll
    for (int i = 0; i < 4; ++i) wred[w][4 * (lane >> 4) + i] = mx[i];
  __syncthreads();
  float cm[4], sm[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int h = 4 * (lane >> 4) + i;
    cm[i] = fmaxf(fmaxf(wred[0][h], wred[1][h]), fmaxf(wred[2][h], wred[3][h]));
    float a = 0.0f;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      const float p = exp2_fast(z[kt][i] - cm[i]);  // -inf (past ns) gives 0
      if (h < G) ps[h][w * 64 + kt * 16 + (lane & 15)] = p;
      a += p;
    }
    sm[i] = a;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int o = 8; o >= 1; o >>= 1) sm[i] += __shfl_xor(sm[i], o);
  __syncthreads();
  if ((lane & 15) == 0)
#pragma unroll
    for (int i = 0; i < 4; ++i) wred[w][4 * (lane >> 4) + i] = sm[i];
  __syncthreads();
  if (w == 0 && (lane & 15) == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = 4 * (lane >> 4) + i;
      if (h < G) {
        float* zp = zpart + ((size_t)(g * G + h) * nchunk + ch) * 2;
        zp[0] = cm[i];
        zp[1] = ((wred[0][h] + wred[1][h]) + wred[2][h]) + wred[3][h];
      }
    }
  }
  // block sums of the chunk (r strides each, r divides 256; ps is published by the barrier above)
  const int nbc = 256 / r;
  for (int idx = threadIdx.x; idx < G * nbc; idx += 256) {
    const int h = idx / nbc, jb = idx % nbc, j = ch * nbc + jb;
    if (j < nb) {
      float a = 0.0f;
      for (int i = 0; i < r; ++i) a += ps[h][jb * r + i];
      bsum[(size_t)(g * G + h) * nb + j] = a;
    }
  }
}

// out[h] = merge of the head's split partials: the weights exp2(m_s - M) in
// LDS, then thread (channel, split class) sums its splits and the classes are
// added in a fixed order.
template <typename T, int D>
__global__ void __launch_bounds__(256) decode_combine_kernel(const float* __restrict__ part, T* __restrict__ out,
                                                             int nsplit) {
  constexpr int NSUB = 256 / D;
  extern __shared__ float wsplit[];  // nsplit weights
  __shared__ float red[4];
  __shared__ float accs[NSUB][D];
  const int h = blockIdx.x, t = threadIdx.x;
  const float* ph = part + (size_t)h * nsplit * (D + 2);
  float mx = -INFINITY;
  for (int s = t; s < nsplit; s += 256) mx = fmaxf(mx, ph[(size_t)s * (D + 2) + D]);
  const float M = wg_max<256>(mx, red);
  float ls = 0.0f;
  for (int s = t; s < nsplit; s += 256) {
    const float ms = ph[(size_t)s * (D + 2) + D];
    const float w = ms == -INFINITY ? 0.0f : exp2_fast(ms - M);  // a split with no blocks weighs 0
    wsplit[s] = w;
    ls += w * ph[(size_t)s * (D + 2) + D + 1];
  }
  const float lsum = wg_sum<256>(ls, red);  // its barriers also publish wsplit
  const int c = t % D, sub = t / D;
  float acc = 0.0f;
#pragma unroll 8
  for (int s = sub; s < nsplit; s += NSUB) acc = __builtin_fmaf(ph[(size_t)s * (D + 2) + c], wsplit[s], acc);
  accs[sub][c] = acc;
  __syncthreads();
  if (t < D) {
    float a = accs[0][t];
#pragma unroll
    for (int i = 1; i < NSUB; ++i) a += accs[i][t];
    out[(size_t)h * D + t] = (T)(lsum > 0.0f ? a / lsum : 0.0f);
  }
}

// Selection flags sel[h][j] from block lists (entries outside [0, nb) and a
// count outside [0, nb] are clamped away): one workgroup per head.
__global__ void __launch_bounds__(256) lists_to_flags_kernel(const int32_t* __restrict__ row_count,
                                                             const int32_t* __restrict__ col_idx, int nb,
                                                             uint8_t* __restrict__ sel, int nbp) {
  const int h = blockIdx.x;
  uint8_t* srow = sel + (size_t)h * nbp;
  for (int j = threadIdx.x; j < nb; j += 256) srow[j] = 0;
  __syncthreads();
  const int cnt = min(max(row_count[h], 0), nb);
  for (int c = threadIdx.x; c < cnt; c += 256) {
    const int j = col_idx[(size_t)h * nb + c];
    if (j >= 0 && j < nb) srow[j] = 1;
  }
}

}  // namespace

hipError_t launch_lists_to_flags(const Geometry& g, const int32_t* row_count, const int32_t* col_idx, uint8_t* sel,
                                 int nbp, hipStream_t st) {
  lists_to_flags_kernel<<<dim3((unsigned)g.Hq), 256, 0, st>>>(row_count, col_idx, g.nb, sel, nbp);
  return hipGetLastError();
}

int decode_chunks(const Geometry& g) { return (g.ns + kDecodeChunk - 1) / kDecodeChunk; }

bool decode_grouped(const Geometry& g) { return g.bf16 && g.G >= 1 && g.G <= 8; }

// blocks per workgroup of the group path: about 512 workgroups over the cache
int decode_group_cb(const Geometry& g) {
  const long long want = ((long long)g.nb * g.Hkv + 511) / 512;
  return (int)std::min<long long>(64, std::max<long long>(1, want));
}

int decode_splits(const Geometry& g) {
  const int per = decode_grouped(g) ? decode_group_cb(g) : kDecodeSplit;
  return (g.nb + per - 1) / per;
}

hipError_t launch_decode_scores(const Geometry& g, const void* q, const void* kbar, float* bsum, float* zpart,
                                hipStream_t st) {
  const float cscale = (1.0f / sqrtf((float)g.d)) * 1.4426950408889634f;
  const int nchunk = decode_chunks(g);
  if (decode_grouped(g)) {
    const dim3 ggrid((unsigned)(g.Hkv * nchunk));
    bool launched = false;
#define RR_GS(DV, GV)                                                                                           \
  if (!launched && g.d == DV && g.G == GV) {                                                                   \
    decode_group_scores_kernel<DV, GV><<<ggrid, 256, 0, st>>>(static_cast<const __bf16*>(q),                   \
                                                              static_cast<const __bf16*>(kbar), bsum, zpart,    \
                                                              g.Hkv, g.ns, g.nb, g.r, nchunk, cscale);         \
    launched = true;                                                                                           \
  }
#define RR_GS_G(DV) RR_GS(DV, 1) RR_GS(DV, 2) RR_GS(DV, 3) RR_GS(DV, 4) RR_GS(DV, 5) RR_GS(DV, 6) RR_GS(DV, 7) RR_GS(DV, 8)
    RR_GS_G(128) RR_GS_G(64)
#undef RR_GS_G
#undef RR_GS
    if (!launched) return hipErrorInvalidValue;
  } else {
  const dim3 grid((unsigned)(g.Hq * nchunk));
#define RR_DS(TY, DV)                                                                                       \
  decode_scores_kernel<TY, DV><<<grid, kDecodeChunk, 0, st>>>(static_cast<const TY*>(q),                    \
                                                              static_cast<const TY*>(kbar), bsum, zpart,    \
                                                              g.Hq, g.Hkv, g.ns, g.nb, g.r, nchunk, cscale)
  if (g.bf16) {
    if (g.d == 128) RR_DS(__bf16, 128);
    else RR_DS(__bf16, 64);
  } else {
    if (g.d == 128) RR_DS(float, 128);
    else RR_DS(float, 64);
  }
#undef RR_DS
  }
  return hipGetLastError();
}

hipError_t launch_decode_attn(const Geometry& g, const void* q, const void* k, const void* v,
                              const int32_t* row_count, const int32_t* col_idx, const uint8_t* sel, int nbp,
                              float* part, void* out, hipStream_t st) {
  const float cscale = (1.0f / sqrtf((float)g.d)) * 1.4426950408889634f;
  const int nsplit = decode_splits(g);
  bool launched = false;
  if (decode_grouped(g)) {
    const dim3 grid((unsigned)(g.Hkv * nsplit));
#define RR_GA(DV, BV, GV)                                                                                           \
  if (!launched && g.d == DV && g.B == BV && g.G == GV) {                                                          \
    decode_group_attn_kernel<DV, BV, GV><<<grid, 256, 0, st>>>(                                                    \
        static_cast<const __bf16*>(q), static_cast<const __bf16*>(k), static_cast<const __bf16*>(v), sel, nbp, part, \
        g.Hkv, g.nb, g.L, cscale, nsplit);                                                                     \
    launched = true;                                                                                               \
  }
#define RR_GA_G(DV, BV) \
  RR_GA(DV, BV, 1) RR_GA(DV, BV, 2) RR_GA(DV, BV, 3) RR_GA(DV, BV, 4) RR_GA(DV, BV, 5) RR_GA(DV, BV, 6) RR_GA(DV, BV, 7) RR_GA(DV, BV, 8)
    RR_GA_G(128, 128) RR_GA_G(128, 64) RR_GA_G(64, 128) RR_GA_G(64, 64)
#undef RR_GA_G
#undef RR_GA
  } else {
    const dim3 grid((unsigned)(g.Hq * nsplit));
#define RR_DA(TY, DV, BV)                                                                                     \
  if (!launched && g.d == DV && g.B == BV) {                                                                  \
    decode_attn_kernel<TY, DV, BV><<<grid, kDecodeThreads, 0, st>>>(                                          \
        static_cast<const TY*>(q), static_cast<const TY*>(k), static_cast<const TY*>(v), sel, nbp, part,     \
        g.Hq, g.Hkv, g.nb, g.L, cscale, nsplit);                                                              \
    launched = true;                                                                                          \
  }
    if (g.bf16) {
      RR_DA(__bf16, 128, 128) RR_DA(__bf16, 128, 64) RR_DA(__bf16, 64, 128) RR_DA(__bf16, 64, 64)
    } else {
      RR_DA(float, 128, 128) RR_DA(float, 128, 64) RR_DA(float, 64, 128) RR_DA(float, 64, 64)
    }
#undef RR_DA
  }
  if (!launched) return hipErrorInvalidValue;
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (g.bf16) {
    if (g.d == 128)
      decode_combine_kernel<__bf16, 128><<<dim3((unsigned)g.Hq), 256, nsplit * sizeof(float), st>>>(
          part, static_cast<__bf16*>(out), nsplit);
    else
      decode_combine_kernel<__bf16, 64><<<dim3((unsigned)g.Hq), 256, nsplit * sizeof(float), st>>>(
          part, static_cast<__bf16*>(out), nsplit);
  } else {
    if (g.d == 128)
      decode_combine_kernel<float, 128><<<dim3((unsigned)g.Hq), 256, nsplit * sizeof(float), st>>>(
          part, static_cast<float*>(out), nsplit);
    else
      decode_combine_kernel<float, 64><<<dim3((unsigned)g.Hq), 256, nsplit * sizeof(float), st>>>(
          part, static_cast<float*>(out), nsplit);
  }
  return hipGetLastError();
}

}  // namespace rr
