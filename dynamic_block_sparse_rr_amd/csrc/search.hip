// Stage 1 of RRAttention on gfx950: stride pooling of the keys, the head
// round-robin sampled scoring with block-mass accumulation, and the adaptive
// Top-tau block selection with the last query block kept whole.
//
// Method: "RRAttention: Dynamic Block Sparse Attention via Per-Head
// Round-Robin Shifts for Long-Context Inference" -- abstract (sampling
// positions rotated over the heads, keys aggregated per stride, the
// O(L^2/S^2) search cost, the adaptive Top-tau cut), TL;DR (Top-tau block
// selection; the last query block always kept whole), Figure 2 caption
// (stride S, block B, three stages).
//
// Kernels
//   pool_keys   K [L][Hkv][d] -> Kbar [ceil(L/S)][Hkv][d]: float32 sum of the
//               keys of a stride in token order (S of them, fewer in a short
//               last stride), divided by their count, rounded to the input
//               dtype. HBM stream: reads K once, writes Kbar.
//   search      one workgroup per (query block i < nb-1, KV head g, chunk of
//               that group's query heads). Sampled query of head h in stride s
//               is token s*S + (h mod S). Scores are computed transposed,
//               Kbar_tile (32 strides x d) * Qs^T (d x 32 sampled queries), on
//               the 32x32 MFMA so that every lane owns one sampled query and
//               16 strides of it: softmax statistics need no cross-lane work
//               except one exchange between the two lane halves. Pass 1 keeps
//               a running (max, sum) per sampled query, the four waves merge
//               theirs through LDS in a fixed order; pass 2 recomputes the
//               scores, forms probabilities and reduces them into key-block
//               masses with a fixed shuffle tree (deterministic, no atomics).
//   select      one wave per (h, i): the Top-tau cut of the (mass desc, index
//               asc) order found without sorting, by bisection on the bits of
//               the cut mass (see the kernel), then the kept blocks compacted
//               into an ascending list.
#include <hip/hip_runtime.h>

#include <type_traits>
#include <stdint.h>

#include "rr_kernels.h"

namespace rr {
namespace {

struct NoSearchBatch {};
template <bool VARLEN>
using SearchBatchArg = typename std::conditional<VARLEN, SearchBatch, NoSearchBatch>::type;

// Sequence of a packed batch whose range [off[b], off[b + 1]) holds x.
__device__ __forceinline__ int batch_seq(const int* off, int n, long long x) {
  int b = 0;
  while (b + 1 < n && x >= off[b + 1]) ++b;
  return b;
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_bits_to_float(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

__device__ __forceinline__ uint32_t float_to_bf16_bits(float x) {
  // clang lowers this conversion to v_cvt_pk_bf16_f32: round to nearest even
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)x);
}

// ------------------------------------------------------------------ pooling

// Pooled keys, one thread per 16-byte chunk of a pooled row (row_chunks =
// Hkv * d * sizeof(T) / 16 per stride; reads of K coalesced). Layout of kbar:
// row-major [ns][Hkv][d] (CM false: the public pooled-key format), or
// chunk-major [Hkv][d*sizeof(T)/16][ns] of 16-byte chunks (CM true: the
// search's own copy, in which the 32 strides of one MFMA operand load are
// contiguous).
// VARLEN: the threads of a packed batch of sequences (SearchBatch), each
// sequence's pooled keys in a region of their own.
template <typename T, bool CM, bool VARLEN>
__global__ void __launch_bounds__(256) pool_keys_kernel(const T* __restrict__ k_all, T* __restrict__ kbar_all,
                                                        int ns_all, int row_chunks, int S, int L_all,
                                                        const SearchBatchArg<VARLEN> sb) {
  long long n = (long long)blockIdx.x * 256 + threadIdx.x;
  const T* k = k_all;
  T* kbar = kbar_all;
  int ns = ns_all, L = L_all;
  if constexpr (VARLEN) {
    if (n >= sb.pool_off[sb.n]) return;
    const int b = batch_seq(sb.pool_off, sb.n, n);
    n -= sb.pool_off[b];
    k = k_all + (size_t)sb.tok_off[b] * row_chunks * (16 / sizeof(T));
    kbar = kbar_all + sb.kbar_off[b];
    ns = sb.ns[b];
    L = sb.L[b];
  }
  if (n >= (long long)ns * row_chunks) return;
  const int t = (int)(n / row_chunks);
  const int c = (int)(n % row_chunks);
  const u32x4* src = reinterpret_cast<const u32x4*>(k) + (size_t)t * S * row_chunks + c;
  const int cnt = min(S, L - t * S);  // tokens in this stride
  const float fcnt = (float)cnt;      // a division by it (by S: exact scaling)
  u32x4 res;
  if constexpr (sizeof(T) == 2) {
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
    for (int u = 0; u < cnt; ++u) {
      const u32x4 w = src[(size_t)u * row_chunks];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[2 * e] += bf16_bits_to_float(w[e] & 0xffffu);
        acc[2 * e + 1] += bf16_bits_to_float(w[e] >> 16);
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e)
      res[e] = float_to_bf16_bits(acc[2 * e] / fcnt) | (float_to_bf16_bits(acc[2 * e + 1] / fcnt) << 16);
  } else {
    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int u = 0; u < cnt; ++u) {
      const u32x4 w = src[(size_t)u * row_chunks];
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] += __uint_as_float(w[e]);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) res[e] = __float_as_uint(acc[e] / fcnt);
  }
  reinterpret_cast<u32x4*>(kbar)[CM ? (size_t)c * ns + t : (size_t)n] = res;
}

// ------------------------------------------------------------------ scoring

// 16-byte operand chunk and the 32x32 MFMA accumulate for one chunk.
template <typename T>
struct Mfma;

template <>
struct Mfma<__bf16> {
  typedef bf16x8 chunk;
  static __device__ __forceinline__ f32x16 acc(chunk a, chunk b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};

template <>
struct Mfma<float> {
  typedef f32x4 chunk;
  static __device__ __forceinline__ f32x16 acc(chunk a, chunk b, f32x16 c) {
#pragma unroll
    for (int e = 0; e < 4; ++e) c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[e], b[e], c, 0, 0, 0);
    return c;
  }
};

__device__ __forceinline__ float exp2_approx(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ void merge_max_sum(float& m, float& l, float m2, float l2) {
  const float mm = fmaxf(m, m2);
  if (mm == -INFINITY) return;  // both empty
  l = l * exp2_approx(m - mm) + l2 * exp2_approx(m2 - mm);
  m = mm;
}

// Cross-lane sums without LDS round trips (DPP and permlane moves). Every
// step adds two equal-sized partial sums, so all lanes of a group end with
// the same value (float addition commutes), the value an xor butterfly over
// the same lanes gives.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xf, 0xf, false));
}
// x + the value of the lane 32 apart
__device__ __forceinline__ float add_halves(float x) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
}
// sum over aligned groups of N consecutive lanes (N a power of two <= 32)
template <int N>
__device__ __forceinline__ float sum_lane_groups(float x) {
  if constexpr (N >= 2) x += dpp<0xB1>(x);   // quad_perm [1,0,3,2]: lane ^ 1
  if constexpr (N >= 4) x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]: lane ^ 2
  if constexpr (N >= 8) x += dpp<0x141>(x);  // row_half_mirror: the other quad of the 8
  if constexpr (N >= 16) x += dpp<0x140>(x); // row_mirror: the other 8 of the 16
  if constexpr (N >= 32) x += __shfl_xor(x, 16);
  return x;
}

// Lane layout of one 32x32 MFMA output (rows = key strides, cols = sampled
// queries): lane owns column (lane & 31) and rows 8*(v/4) + 4*(lane/32) + v%4.
__device__ __forceinline__ int out_row(int v, int half) { return 8 * (v >> 2) + 4 * half + (v & 3); }

// CT: column tiles of sampled queries the kernel can hold (1 when a
// workgroup's heads times R fit in 32 columns, which keeps the registers of
// the second tile free).
// VARLEN: the workgroups of a packed batch of sequences (SearchBatch); each
// workgroup decodes its sequence and continues as that sequence's own.
template <typename T, int D, int R, int CT, bool VARLEN>
__global__ void __launch_bounds__(256) search_kernel(const T* __restrict__ q_all, const T* __restrict__ kbar_all,
                                                     float* __restrict__ mass_all, int Hq, int Hkv, int S,
                                                     int nb_all, int ns_all, int causal, int hpc, int nchunk,
                                                     float cscale, const SearchBatchArg<VARLEN> sb) {
  int bid = blockIdx.x;
  const T* q = q_all;
  const T* kbar = kbar_all;
  float* mass = mass_all;
  int nb = nb_all, ns = ns_all;
  if constexpr (VARLEN) {  // uniform per workgroup
    const int b = batch_seq(sb.blk_off, sb.n, bid);
    bid -= sb.blk_off[b];
    q = q_all + (size_t)sb.tok_off[b] * Hq * D;
    kbar = kbar_all + sb.kbar_off[b];
    mass = mass_all + sb.mass_off[b];
    nb = sb.nb[b];
    ns = sb.ns[b];
  }
  typedef typename Mfma<T>::chunk chunk_t;
  constexpr int E = 16 / sizeof(T);  // elements per 16-byte chunk
  constexpr int NCH = D / (2 * E);   // chunks per lane per row (two lane halves split d)
  static_assert(R >= 2 && R <= 32 && (R & (R - 1)) == 0, "R = B/S must be a power of two in [2, 32]");

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n32 = lane & 31, half = lane >> 5;

  // work item: long rows first
  const int chunk = bid % nchunk;
  const int rest = bid / nchunk;
  const int g = rest % Hkv;
  const int i = (nb - 2) - rest / Hkv;
  const int G = Hq / Hkv;
  const int h0 = g * G + chunk * hpc;
  const int nh = min(hpc, G - chunk * hpc);
  const int NQ = nh * R;
  const int NCT = min((NQ + 31) >> 5, CT);  // 1 or 2 column tiles of sampled queries
  const int tcnt = causal ? (i + 1) * R : ns;
  const int ntile = (tcnt + 31) >> 5;

  // sampled queries (MFMA B operand, kept in registers) and the last visible stride of each
  chunk_t qf[CT][NCH];
  int lim[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    const int qi = ct * 32 + n32;
    if (ct < NCT && qi < NQ) {
      const int hl = qi / R, a = qi % R;
      const int h = h0 + hl;
      const int s = i * R + a;
      const int pos = s * S + (h % S);  // head round-robin offset
      const chunk_t* src = reinterpret_cast<const chunk_t*>(q + ((size_t)pos * Hq + h) * D);  // row-major query
#pragma unroll
      for (int c = 0; c < NCH; ++c) qf[ct][c] = src[2 * c + half];
      lim[ct] = causal ? s : ns - 1;
    } else {
#pragma unroll
      for (int c = 0; c < NCH; ++c) qf[ct][c] = chunk_t{};
      lim[ct] = -1;
    }
  }

  // pooled keys in the chunk-major layout: chunk cc of stride t of KV head g
  // at (g * 2 * NCH + cc) * ns + t, so one operand load (32 strides, one chunk
  // per lane half) reads two contiguous 512-byte runs
  // (read through a buffer descriptor over this KV head's pooled keys, so
  // every load is a per-lane 32-bit offset plus a uniform one per chunk)
  const chunk_t* kcm = reinterpret_cast<const chunk_t*>(kbar) + (size_t)g * 2 * NCH * ns;
  const __amdgpu_buffer_rsrc_t krs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<chunk_t*>(kcm), 0, 2 * NCH * ns * 16, 0x00020000);

  // a tile all of whose strides every sampled query sees needs no mask (the
  // padding columns past NQ then hold values that are never written)
  const int lim_all = causal ? i * R : ns - 1;

  // ---- pass 1: running max / sum of exp2(scaled score) per sampled query
  float mrun[CT], lrun[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    mrun[ct] = -INFINITY;
    lrun[ct] = 0.0f;
  }
  // pooled-key operands of tile `tile` (one 16-byte chunk per lane and k-step;
  // loading the next tile's during this one's compute measured slower: the
  // extra registers cost a wave per SIMD)
  auto load_tile = [&](chunk_t (&kf)[NCH], int tile) __attribute__((always_inline)) {
    const int trow = min(tile * 32 + n32, ns - 1);
    const int voff = (half * ns + trow) * 16;
#pragma unroll
    for (int c = 0; c < NCH; ++c)
      kf[c] = __builtin_bit_cast(chunk_t, __builtin_amdgcn_raw_buffer_load_b128(krs, voff, 2 * c * ns * 16, 0));
  };
  chunk_t kf[NCH];
  for (int tile = wave; tile < ntile; tile += 4) {
    load_tile(kf, tile);
    const bool whole = tile * 32 + 31 <= lim_all;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      if (ct >= NCT) break;
      f32x16 acc = {};
#pragma unroll
      for (int c = 0; c < NCH; ++c) acc = Mfma<T>::acc(kf[c], qf[ct][c], acc);
      // the maximum on the raw scores (cscale > 0), the scale folded into the exponent's FMA
      float tmax = -INFINITY;
      if (whole) {
#pragma unroll
        for (int v = 0; v < 16; ++v) tmax = fmaxf(tmax, acc[v]);
      } else {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int t = tile * 32 + out_row(v, half);
          if (t > lim[ct]) acc[v] = -INFINITY;
          tmax = fmaxf(tmax, acc[v]);
        }
      }
      if (tmax > -INFINITY) {
        const float mnew = fmaxf(mrun[ct], tmax * cscale);
        float sum = 0.0f;
#pragma unroll
        for (int v = 0; v < 16; ++v) sum += exp2_approx(__builtin_fmaf(acc[v], cscale, -mnew));
        lrun[ct] = lrun[ct] * exp2_approx(mrun[ct] - mnew) + sum;
        mrun[ct] = mnew;
      }
    }
  }

  // merge the two lane halves, then the four waves (fixed order)
  __shared__ float sm_m[4][64], sm_l[4][64];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    const float mo = __shfl_xor(mrun[ct], 32);
    const float lo = __shfl_xor(lrun[ct], 32);
    merge_max_sum(mrun[ct], lrun[ct], mo, lo);
    if (half == 0) {
      sm_m[wave][ct * 32 + n32] = mrun[ct];
      sm_l[wave][ct * 32 + n32] = lrun[ct];
    }
  }
  __syncthreads();
  float mu[CT], invl[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    float m = sm_m[0][ct * 32 + n32], l = sm_l[0][ct * 32 + n32];
#pragma unroll
    for (int w = 1; w < 4; ++w) merge_max_sum(m, l, sm_m[w][ct * 32 + n32], sm_l[w][ct * 32 + n32]);
    mu[ct] = m;
    invl[ct] = l > 0.0f ? 1.0f / l : 0.0f;
  }

  // ---- pass 2: probabilities summed into key blocks of R strides
  const float invR = 1.0f / (float)R;  // exact
  for (int tile = wave; tile < ntile; tile += 4) {
    load_tile(kf, tile);
    const bool whole = tile * 32 + 31 <= lim_all;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      if (ct >= NCT) break;
      f32x16 acc = {};
#pragma unroll
      for (int c = 0; c < NCH; ++c) acc = Mfma<T>::acc(kf[c], qf[ct][c], acc);
      // unnormalised probabilities (the query's 1/sum is applied to the in-lane block sums)
      float p[16];
      if (whole) {
#pragma unroll
        for (int v = 0; v < 16; ++v) p[v] = exp2_approx(acc[v] * cscale - mu[ct]);
      } else {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int t = tile * 32 + out_row(v, half);
          const float e = exp2_approx(acc[v] * cscale - mu[ct]);
          p[v] = (t <= lim[ct]) ? e : 0.0f;
        }
      }
      // in-lane sums over the strides of one key block, then across lane halves
      constexpr int NW = (R == 2) ? 8 : (R == 4 || R == 8) ? 4 : (R == 16) ? 2 : 1;
      float w[NW];
      if constexpr (R == 2) {
#pragma unroll
        for (int k2 = 0; k2 < 8; ++k2) w[k2] = p[2 * k2] + p[2 * k2 + 1];
      } else {
        float w4[4];
#pragma unroll
        for (int k4 = 0; k4 < 4; ++k4) w4[k4] = ((p[4 * k4] + p[4 * k4 + 1]) + p[4 * k4 + 2]) + p[4 * k4 + 3];
        if constexpr (R == 4 || R == 8) {
#pragma unroll
          for (int k4 = 0; k4 < 4; ++k4) w[k4] = w4[k4];
        } else if constexpr (R == 16) {
          w[0] = w4[0] + w4[1];
          w[1] = w4[2] + w4[3];
        } else {
          w[0] = (w4[0] + w4[1]) + (w4[2] + w4[3]);
        }
      }
#pragma unroll
      for (int k = 0; k < NW; ++k) w[k] *= invl[ct];
      if constexpr (R >= 8) {
#pragma unroll
        for (int k = 0; k < NW; ++k) w[k] = add_halves(w[k]);
      }
      // sum over the R sampled queries of the head (R consecutive lanes)
#pragma unroll
      for (int k = 0; k < NW; ++k) w[k] = sum_lane_groups<R>(w[k]);
      const int qi = ct * 32 + n32;
      const int hl = qi / R;
      const bool writer = (qi % R == 0) && hl < nh && (R < 8 || half == 0);
      if (writer) {
        float* mrow = mass + ((size_t)(h0 + hl) * nb + i) * nb;
#pragma unroll
        for (int k = 0; k < NW; ++k) {
          int jl;
          if constexpr (R == 2) jl = 4 * (k >> 1) + 2 * half + (k & 1);
          else if constexpr (R == 4) jl = 2 * k + half;
          else jl = k;
          const int jb = tile * (32 / R) + jl;
          if (jb < nb && (!causal || jb <= i)) mrow[jb] = w[k] * invR;
        }
      }
    }
  }
}

// ------------------------------------------------------------------ selection

// Sum over the 64 lanes in one fixed order (pairs of lanes, then of 2, 4, 8,
// 16 and 32 lanes, by DPP and permlane moves: no LDS round trip), taken from
// lane 0 so every lane holds the same value.
__device__ __forceinline__ float lanes16_swap_add(float x) {  // x + the value of the lane 16 apart
  const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
}
__device__ __forceinline__ float wave_total(float x) {
  x = add_halves(lanes16_swap_add(sum_lane_groups<16>(x)));
  return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, x)));
}

__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp<0xB1>(x));
  x = fmaxf(x, dpp<0x4E>(x));
  x = fmaxf(x, dpp<0x141>(x));
  x = fmaxf(x, dpp<0x140>(x));
  {
    const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
  }
  {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
  }
  return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, x)));
}

// Bits of a non-negative mass, ordered like its value (anything else reads as 0).
__device__ __forceinline__ uint32_t mass_bits(float m) { return m > 0.0f ? __float_as_uint(m) : 0u; }

// Top-tau cut of one row per wave (four rows per workgroup, no workgroup
// barriers). The row's candidate masses are staged in LDS. In the (mass
// descending, index ascending) order, block k is kept while the mass before
// it is < tau * total; equivalently, with theta the largest mass value v such
// that the masses >= v reach tau * total (found by bisection on the bits of
// v, each step one sum over the row): every block heavier than theta is
// kept, no lighter one is, and the blocks of mass exactly theta are kept in
// index order while S(> theta) + (equal ones before) * theta < tau * total.
// Sums run in one fixed order, so the cut is deterministic; it can differ from
// a sequential prefix sum only where the cumulative mass lies within float
// rounding of the threshold. At least one block is kept (the first of the
// order: the heaviest, lowest index) even when every mass is zero. The kept
// blocks are written in ascending order (ballot and prefix count per 64).
// VARLEN: the rows of a packed batch of sequences (SearchBatch; no exported
// masses, one threshold); each wave decodes its row's sequence. pitch: the
// LDS floats per wave (the largest nb of the launch).
template <bool VARLEN>
__global__ void __launch_bounds__(256) select_kernel(float* __restrict__ mass_all, int zero_fill,
                                                     int32_t* __restrict__ rc_all,
                                                     int32_t* __restrict__ ci_all, int nrows, int nb_all,
                                                     int causal, float tau_all, const float* __restrict__ tau_heads,
                                                     int pitch, const SearchBatchArg<VARLEN> sb) {
  extern __shared__ float srow_all[];  // one row of up to pitch masses per wave
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int row = blockIdx.x * 4 + wave;
  float* mass = mass_all;
  int32_t* row_count = rc_all;
  int32_t* col_idx = ci_all;
  int nb = nb_all;
  if constexpr (VARLEN) {  // uniform per wave
    if (row >= sb.row_off[sb.n]) return;
    const int b = batch_seq(sb.row_off, sb.n, row);
    row -= sb.row_off[b];
    mass = mass_all + sb.mass_off[b];
    row_count = rc_all + sb.rc_off[b];
    col_idx = ci_all + sb.ci_off[b];
    nb = sb.nb[b];
  } else {
    if (row >= nrows) return;  // the whole wave; nothing below waits for the other waves
  }
  float* srow = srow_all + wave * pitch;
  const int i = row % nb;
  const int ncand = causal ? i + 1 : nb;
  float* mrow = mass + (size_t)row * nb;
  int32_t* out = col_idx + (size_t)row * nb;
  // a threshold per query head when given; NaN or values outside (0, 1] keep
  // every candidate block (never drops mass)
  float tau = tau_heads ? tau_heads[row / nb] : tau_all;
  if (!(tau > 0.0f && tau < 1.0f)) tau = 1.0f;

  if (zero_fill) {  // exported masses: non-candidates and the unsearched last row are zero
    const int from = (i == nb - 1) ? 0 : ncand;
    for (int j = from + lane; j < nb; j += 64) mrow[j] = 0.0f;
  }
  if (i == nb - 1 || tau >= 1.0f) {  // static last-block protection / tau = 1
    for (int j = lane; j < ncand; j += 64) out[j] = j;
    if (lane == 0) row_count[row] = ncand;
    return;
  }

  float part = 0.0f, mx = 0.0f;
  for (int j = lane; j < ncand; j += 64) {
    const float m = mrow[j];
    srow[j] = m;
    part += m;
    mx = fmaxf(mx, m);
  }
  const float total = wave_total(part);
  const uint32_t vmax = mass_bits(wave_max(mx));
  const float thr = tau * total;
  // theta: the largest v <= the maximum mass with S(>= v) >= thr
  uint32_t v = 0;
  for (int bit = 30; bit >= 0; --bit) {
    const uint32_t cand = v | (1u << bit);
    if (cand > vmax) continue;  // uniform
    float sp = 0.0f;
    for (int j = lane; j < ncand; j += 64) {
      const float m = srow[j];
      sp += mass_bits(m) >= cand ? m : 0.0f;
    }
    if (wave_total(sp) >= thr) v = cand;
  }
  float gp = 0.0f;
  for (int j = lane; j < ncand; j += 64) {
    const float m = srow[j];
    gp += mass_bits(m) > v ? m : 0.0f;
  }
  const float sgt = wave_total(gp);  // S(> theta)
  const float theta = __uint_as_float(v);
  int base = 0, eq_before = 0;
  for (int j0 = 0; j0 < ncand; j0 += 64) {
    const int j = j0 + lane;
    const uint32_t bj = j < ncand ? mass_bits(srow[j]) : 0u;
    const bool eq = j < ncand && bj == v;
    const uint64_t eqmask = __ballot(eq);
    const int c = eq_before + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(eqmask >> 32),
                                                          __builtin_amdgcn_mbcnt_lo((uint32_t)eqmask, 0u));
    const bool keep = j < ncand && (bj > v || (eq && (sgt + (float)c * theta < thr || (c == 0 && sgt == 0.0f))));
    const uint64_t kmask = __ballot(keep);
    const int pos = base + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(kmask >> 32),
                                                          __builtin_amdgcn_mbcnt_lo((uint32_t)kmask, 0u));
    if (keep) out[pos] = j;
    base += __popcll(kmask);
    eq_before += __popcll(eqmask);
  }
  if (lane == 0) row_count[row] = base;
}

// Shared mask per KV head (a variant of the per-head masks, not on the pages:
// the union of the G query heads' selected blocks of one query-block row,
// given to every head of the group, so the heads of a KV head compute the
// same blocks). One workgroup per (KV head g, query block i): the union is a
// bitmap of nb bits in LDS (order-free bit sets), compacted in ascending order
// with a prefix sum of the words' popcounts, and written to every head's row.
__global__ void __launch_bounds__(256) union_lists_kernel(const int32_t* __restrict__ row_count,
                                                          const int32_t* __restrict__ col_idx,
                                                          int32_t* __restrict__ out_count,
                                                          int32_t* __restrict__ out_idx, int nb, int G) {
  extern __shared__ uint32_t smem_u[];
  __shared__ uint32_t wsum[4];
  __shared__ uint32_t carry;
  const int nw = (nb + 31) / 32;  // bitmap words
  uint32_t* bits = smem_u;        // [nw]
  uint32_t* base = smem_u + nw;   // [nw] exclusive prefix of the popcounts
  const int g = blockIdx.x / nb, i = blockIdx.x % nb;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int w = threadIdx.x; w < nw; w += 256) bits[w] = 0u;
  if (threadIdx.x == 0) carry = 0u;
  __syncthreads();
  for (int hh = 0; hh < G; ++hh) {
    const size_t row = (size_t)(g * G + hh) * nb + i;
    const int cnt = min(max(row_count[row], 0), nb);
    for (int c = threadIdx.x; c < cnt; c += 256) {
      const int j = col_idx[row * nb + c];
      if (j >= 0 && j < nb) atomicOr(&bits[j >> 5], 1u << (j & 31));
    }
  }
  __syncthreads();
  // exclusive prefix sum of the popcounts, 256 words per pass plus a carry
  for (int w0 = 0; w0 < nw; w0 += 256) {
    const int w = w0 + threadIdx.x;
    const uint32_t c = w < nw ? (uint32_t)__popc(bits[w]) : 0u;
    uint32_t v = c;  // inclusive scan: in-wave shuffles, then the wave totals in order
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t t = __shfl_up(v, o);
      if (lane >= o) v += t;
    }
    if (lane == 63) wsum[wave] = v;
    __syncthreads();
    uint32_t before = carry;
    for (int k = 0; k < wave; ++k) before += wsum[k];
    if (w < nw) base[w] = before + v - c;
    __syncthreads();
    if (threadIdx.x == 255) carry = before + v;
    __syncthreads();
  }
  const uint32_t total = carry;
  for (int w = threadIdx.x; w < nw; w += 256) {
    uint32_t m = bits[w];
    uint32_t pos = base[w];
    while (m) {
      const int j = w * 32 + (__ffs(m) - 1);
      m &= m - 1;
      for (int hh = 0; hh < G; ++hh) out_idx[((size_t)(g * G + hh) * nb + i) * nb + pos] = j;
      ++pos;
    }
  }
  if ((int)threadIdx.x < G) out_count[(size_t)(g * G + threadIdx.x) * nb + i] = (int32_t)total;
}

// Decode step: per query head, the block masses from the scores' chunk
// partials, then the Top-tau prefix of the (mass desc, index asc) order plus
// the last block, which holds the query itself. Written as the ascending list
// and as flags sel[h][j] in {0, 1}.
//
// No sort: the cut is found by a radix search over the order key ~bits(mass)
// (ascending key = descending mass) in 11-, 11- and 10-bit digits. The masses
// (which sum to 1) are summed as 64-bit fixed point, m_j * 2^40, so every
// partial sum is exact and independent of the summation order. Block j is kept
// when the mass before it in the order is below tau * total: each pass
// histograms the candidates' next digit (count and mass), and the cut bucket is
// the last non-empty one whose preceding mass is still below the threshold;
// the search stops once that bucket holds a single block. Equal masses (one key
// value) are kept in index order while the mass before each stays below it.
constexpr int kRadixBuckets = 2048;
constexpr int kRadixPer = kRadixBuckets / 256;  // buckets per thread in the scans

template <typename U>
__device__ __forceinline__ U wave_scan_incl(U x, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const U y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  return x;
}

__device__ __forceinline__ unsigned long long to_fixed(float m) {
  return (unsigned long long)(m * 1099511627776.0f);  // 2^40
}

__global__ void __launch_bounds__(256) decode_select_kernel(const float* __restrict__ bsum,
                                                            const float* __restrict__ zpart, int r, int nchunk,
                                                            float* __restrict__ mass, int nb, float tau,
                                                            int32_t* __restrict__ row_count,
                                                            int32_t* __restrict__ col_idx,
                                                            uint8_t* __restrict__ sel, int nbp) {
  extern __shared__ float mm[];  // the head's nb block masses
  __shared__ uint32_t cnt[kRadixBuckets];
  __shared__ unsigned long long msum[kRadixBuckets];
  __shared__ unsigned long long wtot[4], wscan[4];
  __shared__ uint32_t wt32[4];
  __shared__ int slot_d[4];
  __shared__ uint32_t slot_n[4];
  __shared__ unsigned long long slot_b[4];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int h = blockIdx.x;
  int32_t* out = col_idx + (size_t)h * nb;
  uint8_t* srow = sel + (size_t)h * nbp;
  const bool all = !(tau > 0.0f && tau < 1.0f);  // every block

  for (int b = tid; b < kRadixBuckets; b += 256) {
    cnt[b] = 0;
    msum[b] = 0;
  }
  // the first block sums are loaded before the chunk partials are used, so
  // that both reads share one round trip
  constexpr int PRE = 4;
  float bpre[PRE];
#pragma unroll
  for (int e = 0; e < PRE; ++e) {
    const int j = tid + 256 * e;
    bpre[e] = j < nb ? bsum[(size_t)h * nb + j] : 0.0f;
  }
  // softmax over all strides from the chunks' (max, exp-sum), every wave alike
  const float* zp = zpart + (size_t)h * nchunk * 2;
  float M = -INFINITY;
  for (int c = lane; c < nchunk; c += 64) M = fmaxf(M, zp[2 * c]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
  float S = 0.0f;
  for (int c = lane; c < nchunk; c += 64) S += zp[2 * c + 1] * __builtin_amdgcn_exp2f(zp[2 * c] - M);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) S += __shfl_xor(S, o);
  const float inv_s = 1.0f / S;
  __syncthreads();  // histogram cleared

  // masses, their fixed-point total and the first digit's histogram
  unsigned long long fsum = 0;
  auto block_mass = [&](int j, float b) {
    const int ch = (j * r) >> 8;
    float m = b * __builtin_amdgcn_exp2f(zp[2 * ch] - M) * inv_s;
    mass[(size_t)h * nb + j] = m;
    m = m > 0.0f ? m : 0.0f;  // NaN and negative count as 0
    mm[j] = m;
    if (!all) {
      const unsigned long long f = to_fixed(m);
      fsum += f;
      const uint32_t d = ~__float_as_uint(m) >> 21;
      atomicAdd(&cnt[d], 1u);
      atomicAdd(&msum[d], f);
    }
  };
#pragma unroll
  for (int e = 0; e < PRE; ++e)
    if (tid + 256 * e < nb) block_mass(tid + 256 * e, bpre[e]);
  for (int j = tid + 256 * PRE; j < nb; j += 256) block_mass(j, bsum[(size_t)h * nb + j]);
  if (all) {
    for (int j = tid; j < nb; j += 256) {
      out[j] = j;
      srow[j] = 1;
    }
    if (tid == 0) row_count[h] = nb;
    return;
  }
  fsum = wave_scan_incl(fsum, lane);
  if (lane == 63) wtot[w] = fsum;
  __syncthreads();
  const unsigned long long TF = wtot[0] + wtot[1] + wtot[2] + wtot[3];
  const double thr = (double)tau * (double)TF;
  const bool none = !(thr > 0.0);  // all masses zero: keep the first block of the order only

  uint32_t prefix = 0;
  unsigned long long base = 0;
  int fshift = 0;     // the cut is (key >> fshift) == prefix
  uint32_t ncut = 0;  // blocks with that key prefix
  if (!none) {
    const int shifts[3] = {21, 10, 0}, widths[3] = {11, 11, 10};
#pragma unroll
    for (int pss = 0; pss < 3; ++pss) {
      const int sh = shifts[pss], wd = widths[pss];
      if (pss > 0) {  // histogram of the candidates' next digit (cleared at the end of the last pass)
        for (int j = tid; j < nb; j += 256) {
          const uint32_t key = ~__float_as_uint(mm[j]);
          if ((key >> (sh + wd)) == prefix) {
            const uint32_t d = (key >> sh) & ((1u << wd) - 1u);
            atomicAdd(&cnt[d], 1u);
            atomicAdd(&msum[d], to_fixed(mm[j]));
          }
        }
        __syncthreads();
      }
      // thread t owns buckets kRadixPer t ..: the mass before each bucket
      uint32_t bc[kRadixPer];
      unsigned long long bm[kRadixPer], loc = 0;
#pragma unroll
      for (int e = 0; e < kRadixPer; ++e) {
        bc[e] = cnt[kRadixPer * tid + e];
        bm[e] = msum[kRadixPer * tid + e];
        loc += bm[e];
      }
      const unsigned long long inc = wave_scan_incl(loc, lane);
      if (lane == 63) wscan[w] = inc;
      __syncthreads();
      unsigned long long ex = base + inc - loc;
      for (int i = 0; i < w; ++i) ex += wscan[i];
      int cand = -1;
      uint32_t ccnt = 0;
      unsigned long long cbase = 0;
#pragma unroll
      for (int e = 0; e < kRadixPer; ++e) {
        if (bc[e] > 0 && (double)ex < thr) {
          cand = kRadixPer * tid + e;
          ccnt = bc[e];
          cbase = ex;
        }
        ex += bm[e];
      }
      // the last qualifying bucket: per wave its highest lane, then the last wave with one
      const unsigned long long q = __ballot(cand >= 0);
      if (q != 0 && lane == 63 - __clzll(q)) {
        slot_d[w] = cand;
        slot_n[w] = ccnt;
        slot_b[w] = cbase;
      } else if (q == 0 && lane == 0) {
        slot_d[w] = -1;
      }
#pragma unroll
      for (int e = 0; e < kRadixPer; ++e) {  // clear for the next pass (this thread's reads are done)
        cnt[kRadixPer * tid + e] = 0;
        msum[kRadixPer * tid + e] = 0;
      }
      __syncthreads();
      int ws = 3;
      while (ws > 0 && slot_d[ws] < 0) --ws;
      // slot_d[ws] >= 0: the candidates' first block has mass before it base < thr
      prefix = (prefix << wd) | (uint32_t)slot_d[ws];
      base = slot_b[ws];
      ncut = slot_n[ws];
      fshift = sh;
      if (ncut == 1) break;
      // the slots and wscan are rewritten only after the next pass's first
      // barrier, which every thread reaches after its reads here
    }
  }

  // ties (one key value, fshift == 0): the first tkeep of them in index order
  const bool tied = !none && ncut > 1;
  uint32_t tkeep = ncut;
  if (tied) {
    const unsigned long long Fs = to_fixed(__uint_as_float(~prefix));
    if (Fs > 0) tkeep = (uint32_t)fmin((double)ncut, ceil((thr - (double)base) / (double)Fs));
  }
  const int seg = (nb + 255) / 256;
  const int jlo = min(tid * seg, nb), jhi = min(jlo + seg, nb);
  uint32_t trank = 0;
  if (tied) {  // rank of this thread's first tie in index order
    uint32_t ties = 0;
    for (int j = jlo; j < jhi; ++j) ties += (~__float_as_uint(mm[j]) >> fshift) == prefix;
    const uint32_t inc = wave_scan_incl(ties, lane);
    __syncthreads();
    if (lane == 63) wt32[w] = inc;
    __syncthreads();
    trank = inc - ties;
    for (int i = 0; i < w; ++i) trank += wt32[i];
  }
  auto kept = [&](int j, uint32_t& rk) -> bool {
    const uint32_t k = ~__float_as_uint(mm[j]) >> fshift;
    const bool tie = tied && k == prefix;
    const bool keep = j == nb - 1 || (none ? j == 0 : (k < prefix || (k == prefix && (!tied || rk < tkeep))));
    rk += tie;
    return keep;
  };
  uint32_t c = 0, rk = trank;
  for (int j = jlo; j < jhi; ++j) c += kept(j, rk);
  const uint32_t inc = wave_scan_incl(c, lane);
  __syncthreads();
  if (lane == 63) wt32[w] = inc;
  __syncthreads();
  uint32_t pos = inc - c;
  for (int i = 0; i < w; ++i) pos += wt32[i];
  rk = trank;
  for (int j = jlo; j < jhi; ++j) {
    const bool kj = kept(j, rk);
    srow[j] = (uint8_t)kj;
    if (kj) out[pos++] = j;
  }
  if (tid == 0) row_count[h] = (int32_t)(wt32[0] + wt32[1] + wt32[2] + wt32[3]);
}

// Query heads per search workgroup and workgroups per (query block, KV head).
inline void search_split(const Geometry& g, int* hpc, int* nchunk) {
  *hpc = min(g.G, 64 / g.r);
  *nchunk = (g.G + *hpc - 1) / *hpc;
}

template <typename T, int D>
hipError_t launch_search_r(const Geometry& g, const void* q, const void* kbar, float* mass,
                           hipStream_t st) {
  int hpc, nchunk;
  search_split(g, &hpc, &nchunk);
  const int nrows = g.nb - 1;
  if (nrows <= 0) return hipSuccess;
  const dim3 grid((unsigned)(nrows * g.Hkv * nchunk));
  const float cscale = (1.0f / sqrtf((float)g.d)) * 1.4426950408889634f;
  const T* qq = static_cast<const T*>(q);
  const T* kk = static_cast<const T*>(kbar);
  const bool one_tile = hpc * g.r <= 32;
#define RR_SEARCH_CASE(RV)                                                                               \
  case RV:                                                                                               \
    if (one_tile)                                                                                        \
      search_kernel<T, D, RV, 1, false><<<grid, 256, 0, st>>>(qq, kk, mass, g.Hq, g.Hkv, g.S, g.nb, g.ns, \
                                                              g.causal, hpc, nchunk, cscale, {});        \
    else                                                                                                 \
      search_kernel<T, D, RV, 2, false><<<grid, 256, 0, st>>>(qq, kk, mass, g.Hq, g.Hkv, g.S, g.nb, g.ns, \
                                                              g.causal, hpc, nchunk, cscale, {});        \
    break;
  switch (g.r) {
    RR_SEARCH_CASE(2)
    RR_SEARCH_CASE(4)
    RR_SEARCH_CASE(8)
    RR_SEARCH_CASE(16)
    RR_SEARCH_CASE(32)
    default:
      return hipErrorInvalidValue;
  }
#undef RR_SEARCH_CASE
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_search_batched_r(const Geometry& g, const SearchBatch& sb, const void* q, const void* kbar,
                                   float* mass, hipStream_t st) {
  int hpc, nchunk;
  search_split(g, &hpc, &nchunk);
  if (sb.blk_off[sb.n] <= 0) return hipSuccess;
  const dim3 grid((unsigned)sb.blk_off[sb.n]);
  const float cscale = (1.0f / sqrtf((float)g.d)) * 1.4426950408889634f;
  const T* qq = static_cast<const T*>(q);
  const T* kk = static_cast<const T*>(kbar);
  const bool one_tile = hpc * g.r <= 32;
#define RR_SEARCH_CASE(RV)                                                                            \
  case RV:                                                                                            \
    if (one_tile)                                                                                     \
      search_kernel<T, D, RV, 1, true><<<grid, 256, 0, st>>>(qq, kk, mass, g.Hq, g.Hkv, g.S, 0, 0,     \
                                                             g.causal, hpc, nchunk, cscale, sb);      \
    else                                                                                              \
      search_kernel<T, D, RV, 2, true><<<grid, 256, 0, st>>>(qq, kk, mass, g.Hq, g.Hkv, g.S, 0, 0,     \
                                                             g.causal, hpc, nchunk, cscale, sb);      \
    break;
  switch (g.r) {
    RR_SEARCH_CASE(2)
    RR_SEARCH_CASE(4)
    RR_SEARCH_CASE(8)
    RR_SEARCH_CASE(16)
    RR_SEARCH_CASE(32)
    default:
      return hipErrorInvalidValue;
  }
#undef RR_SEARCH_CASE
  return hipGetLastError();
}

}  // namespace

void search_batch_counts(const Geometry& g, int nb, int ns, int* pool_threads, int* search_blocks, int* rows) {
  int hpc, nchunk;
  search_split(g, &hpc, &nchunk);
  *pool_threads = ns * (g.Hkv * g.d * (g.bf16 ? 2 : 4) / 16);
  *search_blocks = (nb - 1) * g.Hkv * nchunk;
  *rows = g.Hq * nb;
}

hipError_t launch_pool_keys_batched(const Geometry& g, const SearchBatch& sb, const void* k, void* kbar,
                                    hipStream_t st) {
  const int row_chunks = g.Hkv * g.d * (g.bf16 ? 2 : 4) / 16;
  const dim3 grid((unsigned)((sb.pool_off[sb.n] + 255) / 256));
  if (g.bf16)
    pool_keys_kernel<__bf16, true, true><<<grid, 256, 0, st>>>(static_cast<const __bf16*>(k), static_cast<__bf16*>(kbar),
                                                               0, row_chunks, g.S, 0, sb);
  else
    pool_keys_kernel<float, true, true><<<grid, 256, 0, st>>>(static_cast<const float*>(k), static_cast<float*>(kbar),
                                                              0, row_chunks, g.S, 0, sb);
  return hipGetLastError();
}

hipError_t launch_search_batched(const Geometry& g, const SearchBatch& sb, const void* q, const void* kbar,
                                 float* mass, hipStream_t st) {
  if (g.bf16) return g.d == 128 ? launch_search_batched_r<__bf16, 128>(g, sb, q, kbar, mass, st)
                                : launch_search_batched_r<__bf16, 64>(g, sb, q, kbar, mass, st);
  return g.d == 128 ? launch_search_batched_r<float, 128>(g, sb, q, kbar, mass, st)
                    : launch_search_batched_r<float, 64>(g, sb, q, kbar, mass, st);
}

hipError_t launch_select_batched(const Geometry& g, const SearchBatch& sb, const float* mass, int32_t* row_count,
                                 int32_t* col_idx, hipStream_t st) {
  int pitch = 1;
  for (int b = 0; b < sb.n; ++b) pitch = max(pitch, sb.nb[b]);
  const size_t lds = 4 * (size_t)pitch * sizeof(float);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&select_kernel<true>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  if (sb.row_off[sb.n] <= 0) return hipSuccess;
  select_kernel<true><<<dim3((unsigned)((sb.row_off[sb.n] + 3) / 4)), 256, lds, st>>>(
      const_cast<float*>(mass), 0, row_count, col_idx, 0, 0, g.causal, g.tau, nullptr, pitch, sb);
  return hipGetLastError();
}

hipError_t launch_pool_keys(const Geometry& g, const void* k, void* kbar, bool chunk_major, hipStream_t st) {
  const int esz = g.bf16 ? 2 : 4;
  const int row_chunks = g.Hkv * g.d * esz / 16;
  const long long n = (long long)g.ns * row_chunks;
  const dim3 grid((unsigned)((n + 255) / 256));
#define RR_POOL(TY, CMV)                                                                           \
  pool_keys_kernel<TY, CMV, false><<<grid, 256, 0, st>>>(static_cast<const TY*>(k), static_cast<TY*>(kbar), \
                                                         g.ns, row_chunks, g.S, g.L, {})
  if (g.bf16) {
    if (chunk_major) RR_POOL(__bf16, true);
    else RR_POOL(__bf16, false);
  } else {
    if (chunk_major) RR_POOL(float, true);
    else RR_POOL(float, false);
  }
#undef RR_POOL
  return hipGetLastError();
}

hipError_t launch_search(const Geometry& g, const void* q, const void* kbar, float* mass,
                         hipStream_t st) {
  if (g.bf16) return g.d == 128 ? launch_search_r<__bf16, 128>(g, q, kbar, mass, st)
                                : launch_search_r<__bf16, 64>(g, q, kbar, mass, st);
  return g.d == 128 ? launch_search_r<float, 128>(g, q, kbar, mass, st)
                    : launch_search_r<float, 64>(g, q, kbar, mass, st);
}

hipError_t launch_select(const Geometry& g, const float* mass, int zero_fill, int32_t* row_count,
                         int32_t* col_idx, const float* tau_heads, hipStream_t st) {
  const size_t lds = 4 * (size_t)g.nb * sizeof(float);  // one row per wave
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&select_kernel<false>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  const int nrows = g.Hq * g.nb;
  select_kernel<false><<<dim3((unsigned)((nrows + 3) / 4)), 256, lds, st>>>(
      const_cast<float*>(mass), zero_fill, row_count, col_idx, nrows, g.nb, g.causal, g.tau, tau_heads, g.nb, {});
  return hipGetLastError();
}

hipError_t launch_union_lists(const Geometry& g, const int32_t* row_count, const int32_t* col_idx,
                              int32_t* out_count, int32_t* out_idx, hipStream_t st) {
  const size_t lds = 2 * (size_t)((g.nb + 31) / 32) * sizeof(uint32_t);
  union_lists_kernel<<<dim3((unsigned)(g.Hkv * g.nb)), 256, lds, st>>>(row_count, col_idx, out_count, out_idx,
                                                                      g.nb, g.G);
  return hipGetLastError();
}


hipError_t launch_decode_select(const Geometry& g, const float* bsum, const float* zpart, float* mass,
                                int32_t* row_count, int32_t* col_idx, uint8_t* sel, int nbp, hipStream_t st) {
  decode_select_kernel<<<dim3((unsigned)g.Hq), 256, (size_t)g.nb * sizeof(float), st>>>(
      bsum, zpart, g.r, decode_chunks(g), mass, g.nb, g.tau, row_count, col_idx, sel, nbp);
  return hipGetLastError();
}

}  // namespace rr
