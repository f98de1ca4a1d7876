// Stage 2 of RRAttention on gfx950: block-sparse flash attention over the
// compacted per-row block lists (the abstract of "RRAttention: Dynamic Block
// Sparse Attention via Per-Head Round-Robin Shifts for Long-Context
// Inference" reports about half of the blocks computed).
//
// bfloat16 path (the hot kernel)
//   transpose_v  V [L][Hkv][d] -> Vt [Hkv][nb][B/8][d][8]: each key block
//                becomes a contiguous 2*B*d-byte tile of 16-byte chunks, chunk
//                (c, e) holding channel e at the block's positions 8c..8c+7
//                (keys permuted inside every group of 16, see key_of_pos),
//                chunk-major so that the copy into LDS is a straight copy and
//                every MFMA operand read is one contiguous run. One HBM pass
//                over V.
//   attn_bf16    one workgroup of B/32 waves per (query head h, query block i);
//                wave w owns 32 query rows. Per selected key block j:
//                  K tile and Vt tile staged in LDS (K as 16-byte chunks XOR
//                  swizzled by row, Vt chunk-major as stored, so the MFMA
//                  operand reads are conflict-free);
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
//   attn_bf16_pp B = 128: two query heads of one KV head per workgroup (two
//                waves per SIMD, one per head), walking the merged block
//                list of both heads, so each K/Vt tile is copied once for
//                both (double-buffered); each block is split in two
//                half-steps so that one head's waves issue their MFMAs while
//                the other head's run the softmax (see the kernel). With an
//                odd group (one query head per KV head included) the last
//                head of each KV head pairs with itself over two adjacent
//                query blocks (one per slot), so no slot is left idle.
//                attn_bf16 serves B = 64.
// The kernel is chosen from the problem alone (dtype, B).
// float32 path: attn_f32, on the fp32 matrix cores (see the kernel).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <type_traits>

#include "rr_kernels.h"

namespace rr {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float exp2_approx(float x) { return __builtin_amdgcn_exp2f(x); }

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// two floats to a packed pair of bfloat16 (round to nearest even), one v_cvt_pk_bf16_f32
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
}

// Online softmax of one key block for one wave, in base 2 with the scale
// folded into cscale (the score tiles of S^T = K Q^T: the lane's column is its
// query, rows are keys). The probabilities are first taken against the current
// reference mrow (the largest scaled score seen when it last moved) without
// looking for the block's maximum: only when the block's sum for some query
// exceeds kSumLimit (or is not finite, as on a lane's first block, where the
// reference is the kRefStart sentinel) does the block take the maximum, move
// the reference, rescale O and the sum, and recompute. Probabilities therefore
// stay below kSumLimit, far inside the range of bf16 and fp32. P is rounded to
// bf16 in the B-operand layout of O^T += Vt P^T, and the row sum adds exactly
// the rounded values the MFMA multiplies.
constexpr float kSumLimit = 65536.0f;
constexpr float kRefStart = -1e30f;  // reference before any visible key
template <int MT, int NT>
__device__ __forceinline__ void ref_softmax(float cscale, f32x16 (&sacc)[MT], f32x16 (&oacc)[NT], float& mrow,
                                            float& lrow, bf16x8 (&pf)[MT][2]) {
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  auto probs = [&](float m) __attribute__((always_inline)) {
    float ps[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
      for (int p2 = 0; p2 < 2; ++p2) {
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p0 = exp2_approx(__builtin_fmaf(sacc[mt][8 * p2 + 2 * e], cscale, -m));
          const float p1 = exp2_approx(__builtin_fmaf(sacc[mt][8 * p2 + 2 * e + 1], cscale, -m));
          w[e] = pack_bf16x2(p0, p1);
          ps[e] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w[e]), ones, ps[e], false);
        }
        pf[mt][p2] = __builtin_bit_cast(bf16x8, (u32x4){w[0], w[1], w[2], w[3]});
      }
    }
    return (ps[0] + ps[1]) + (ps[2] + ps[3]);
  };
  float tot = probs(mrow);
  float both;  // the query's block sum: the two lane halves hold different keys
  {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(tot), __float_as_uint(tot), false, false);
    both = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
  }
  if (__builtin_amdgcn_ballot_w64(!(both <= kSumLimit)) != 0) {  // some reference moves
    float tmax = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int v = 0; v < 16; ++v) tmax = fmaxf(tmax, sacc[mt][v]);
    {
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(tmax), __float_as_uint(tmax), false, false);
      tmax = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
    }
    const float mnew = fmaxf(mrow, tmax * cscale);
    const float alpha = exp2_approx(mrow - mnew);
    lrow *= alpha;
#pragma unroll
    for (int t = 0; t < NT; ++t) oacc[t] *= alpha;
    mrow = mnew;
    tot = probs(mrow);
  }
  lrow += tot;
}

// Position p (0..15) inside a 16-key group of a Vt row holds key key_of_pos(p)
// of that group. This matches the order in which a lane holds its
// probabilities after S^T = K Q^T (lane half hf, register v: key 8*(v/4) +
// 4*hf + v%4), so that eight consecutive Vt entries form one MFMA A operand.
__host__ __device__ __forceinline__ int key_of_pos(int p) {
  return 8 * ((p & 7) >> 2) + 4 * (p >> 3) + (p & 3);
}

// The batch table argument of the varlen launches (an empty struct otherwise).
struct NoBatch {};
template <bool VARLEN>
using BatchArg = typename std::conditional<VARLEN, SeqBatch, NoBatch>::type;

// ------------------------------------------------------------------ V re-layout

//
// VARLEN: one launch re-lays out every sequence of a packed batch (SeqBatch):
// workgroup x belongs to the sequence whose tile range holds it.
template <int D, int BLK, bool VARLEN>
__global__ void __launch_bounds__(256) transpose_v_kernel(const __bf16* __restrict__ v_all,
                                                          __bf16* __restrict__ vt_all, int Hkv, int nb_all,
                                                          int L_all, int32_t* __restrict__ queues,
                                                          const BatchArg<VARLEN> sb) {
  // one workgroup per (g, key block j); tile BLK keys x D channels
  __shared__ uint16_t tile[BLK][D + 2];
  if (blockIdx.x == 0 && threadIdx.x < kAttnQueues) queues[threadIdx.x] = 0;  // the attention's work queues
  const __bf16* v = v_all;
  __bf16* vt = vt_all;
  int nb = nb_all, L = L_all, tile_id = (int)blockIdx.x;
  if constexpr (VARLEN) {  // the sequence of this tile (uniform)
    int sq = 0;
    while (sq + 1 < sb.n && tile_id >= sb.tile_off[sq + 1]) ++sq;
    tile_id -= sb.tile_off[sq];
    nb = sb.nb[sq];
    L = sb.L[sq];
    v = v_all + (size_t)sb.tok_off[sq] * Hkv * D;
    vt = reinterpret_cast<__bf16*>(reinterpret_cast<uint8_t*>(vt_all) + sb.vt_off[sq]);
  }
  const int j = tile_id % nb;
  const int g = tile_id / nb;
  const uint16_t* src = reinterpret_cast<const uint16_t*>(v);
  constexpr int CH = D / 8;  // 16-byte chunks per key row
  for (int n = threadIdx.x; n < BLK * CH; n += 256) {
    const int key = n / CH, c = n % CH;
    // keys past the end of a short last block are zero (their probabilities are zero too)
    const u32x4 w = j * BLK + key < L
                        ? *reinterpret_cast<const u32x4*>(src + ((size_t)(j * BLK + key) * Hkv + g) * D + c * 8)
                        : u32x4{0u, 0u, 0u, 0u};
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
    const int e = n % D, c = n / D;  // consecutive threads, consecutive chunks of the tile
    u32x4 w;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int p0 = c * 8 + 2 * t, p1 = p0 + 1;
      const int k0 = (p0 & ~15) + key_of_pos(p0 & 15), k1 = (p1 & ~15) + key_of_pos(p1 & 15);
      w[t] = (uint32_t)tile[k0][e] | ((uint32_t)tile[k1][e] << 16);
    }
    *reinterpret_cast<u32x4*>(dst + ((size_t)c * D + e) * 8) = w;
  }
}

// ------------------------------------------------------------------ bf16 attention

// Maps the launch index to (query head, query block): query blocks in
// decreasing order (causal rows get longer with i), the heads of one KV head
// on one XCD in consecutive dispatch slots. The launch covers heads hbase ..
// hbase + hcount - 1 of every KV head (all G of them, or one).
__device__ __forceinline__ void work_item(int x, int Hq, int Hkv, int nb, int hbase, int hcount, int& h, int& i) {
  const int G = Hq / Hkv;
  const int nunits = Hkv * nb;
  int u, hh;
  if ((nunits & 7) == 0) {
    const int xcd = x & 7, t = x >> 3;
    hh = t % hcount;
    u = (t / hcount) * 8 + xcd;
  } else {
    u = x / hcount;
    hh = x % hcount;
  }
  i = nb - 1 - u / Hkv;
  h = (u % Hkv) * G + hbase + hh;
}

// Shared state of one workgroup of the bf16 kernel.
template <int D, int BLK>
struct AttnCtx {
  static constexpr int NTHR = BLK * 2;               // BLK/32 waves
  static constexpr int MT = BLK / 32;                // 32-key subtiles
  static constexpr int NT = D / 32;                  // 32-channel tiles of O
  static constexpr int DK = D / 16;                  // MFMA k-steps over d
  static constexpr int TILE = BLK * D * 2;           // bytes of one K or Vt tile
  static constexpr int NDMA = TILE / (NTHR * 16);    // 16-byte copies per thread per tile
  static constexpr int KCH = D / 8;                  // 16-byte chunks per K row
  uint8_t* lds_k;
  uint8_t* lds_v;
  uint32_t koff, voff;    // this thread's copy source for copy 0, relative to a tile base
  uint32_t kstep, vstep;  // source distance between consecutive copies (bytes)
  int kro, vro;          // operand read offsets for chunk 0 (K: XOR in the chunk index; Vt: add)
  int wave, qr, half;
  float cscale;
};

// Copy n of a thread fetches row (n * RPC + row0) of the tile, RPC = threads
// per copy / chunks per row. Its swizzled chunk is chunk0 ^ ((n * RPC) mod
// CH) because row0 < RPC, and chunk bits (16-byte units below the row size)
// do not overlap row bits, hence the XOR on the offset.
// Buffer descriptor over `bytes` bytes from p (raw addressing, no stride;
// reads beyond the range return zero).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const uint8_t* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(p), 0, (int)bytes, 0x00020000);
}

template <int D, int BLK, int CH>
__device__ __forceinline__ void copy_tile(const AttnCtx<D, BLK>& cx, __amdgpu_buffer_rsrc_t src, uint32_t off,
                                          uint32_t step, uint8_t* dst) {
  constexpr int RPC = AttnCtx<D, BLK>::NTHR / CH;
#pragma unroll
  for (int n = 0; n < AttnCtx<D, BLK>::NDMA; ++n)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        src,
        reinterpret_cast<__attribute__((address_space(3))) void*>(
            reinterpret_cast<uintptr_t>(dst + (n * AttnCtx<D, BLK>::NTHR + cx.wave * 64) * 16)),
        16, (int)(n * step + (off ^ (((n * RPC) & (CH - 1)) << 4))), 0, 0, 0);
}

// Bytes of a K tile from its first byte at offset tile_start of the K tensor
// (k_bytes long): `full` when the tile lies inside it, else cut where it ends
// (a short last block then reads zeros).
__device__ __forceinline__ uint32_t k_tile_bytes(size_t tile_start, size_t k_bytes, uint32_t full) {
  return tile_start + full <= k_bytes ? full : (uint32_t)(k_bytes - tile_start);
}

// One key block. On entry K (and possibly V) copies of this block are in
// flight; next_k / next_v are the descriptors of the following block's tiles
// (has_next false at the end). masked: keys with index > klim inside the
// block are masked (the causal diagonal block: klim = the lane's query row;
// a short last block: klim = its last key).
template <int D, int BLK>
__device__ __forceinline__ void attn_tile(const AttnCtx<D, BLK>& cx, const bf16x8 (&qf)[D / 16],
                                          f32x16 (&oacc)[D / 32], float& mrow, float& lrow, bool has_next,
                                          __amdgpu_buffer_rsrc_t next_k, __amdgpu_buffer_rsrc_t next_v, bool masked,
                                          int klim) {
  constexpr int MT = AttnCtx<D, BLK>::MT;
  constexpr int NT = AttnCtx<D, BLK>::NT;
  constexpr int DK = AttnCtx<D, BLK>::DK;

  constexpr int NDMA = AttnCtx<D, BLK>::NDMA;
  // K of this block has landed (its V may still be in flight)
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(NDMA) : "memory");
  // S^T = K Q^T: rows are keys, the lane's column is its query
  // operand reads run LA steps ahead of the MFMAs through a register ring
  constexpr int LA = 4;
  constexpr int NQK = MT * DK;
  auto kread = [&](int k) {
    return *reinterpret_cast<const bf16x8*>(cx.lds_k + (k / DK) * 32 * D * 2 + (cx.kro ^ ((k % DK) << 5)));
  };
  f32x16 sacc[MT];
  bf16x8 ring[LA];
#pragma unroll
  for (int k = 0; k < LA; ++k) ring[k] = kread(k);
#pragma unroll
  for (int k = 0; k < NQK; ++k) {
    const bf16x8 a = ring[k % LA];
    if (k + LA < NQK) ring[k % LA] = kread(k + LA);
    const int mt = k / DK, cc = k % DK;
    sacc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[cc], cc ? sacc[mt] : f32x16{}, 0, 0, 0);
  }
  // every wave is done with the K buffer: the next block's K may land in it
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  if (has_next) copy_tile<D, BLK, AttnCtx<D, BLK>::KCH>(cx, next_k, cx.koff, cx.kstep, cx.lds_k);

  // online softmax against the reference (ref_softmax)
  if (masked) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int key = mt * 32 + 8 * (v >> 2) + 4 * cx.half + (v & 3);
        if (key > klim) sacc[mt][v] = -INFINITY;
      }
  }
  bf16x8 pf[MT][2];
  ref_softmax(cx.cscale, sacc, oacc, mrow, lrow, pf);

  // V of this block has landed (the next block's K may still be in flight)
  if (has_next)
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(NDMA) : "memory");
  else
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
  // O^T += Vt P^T, operand reads again LA steps ahead
  constexpr int NPV = NT * MT * 2;
  auto vread = [&](int k) {
    const int t = k / (MT * 2), r = k % (MT * 2);
    return *reinterpret_cast<const bf16x8*>(cx.lds_v + cx.vro + (2 * r * D + t * 32) * 16);
  };
#pragma unroll
  for (int k = 0; k < LA; ++k) ring[k] = vread(k);
#pragma unroll
  for (int k = 0; k < NPV; ++k) {
    const bf16x8 a = ring[k % LA];
    if (k + LA < NPV) ring[k % LA] = vread(k + LA);
    const int t = k / (MT * 2), r = k % (MT * 2);
    oacc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[r >> 1][r & 1], oacc[t], 0, 0, 0);
  }
  // every wave is done with the V buffer: the next block's V may land in it
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  if (has_next) copy_tile<D, BLK, 1>(cx, next_v, cx.voff, cx.vstep, cx.lds_v);
}

template <int D, int BLK>
__global__ void __launch_bounds__(BLK * 2) __attribute__((amdgpu_waves_per_eu(2, 2))) attn_bf16_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ vt,
    const int32_t* __restrict__ row_count, const int32_t* __restrict__ col_idx, __bf16* __restrict__ out,
    int Hq, int Hkv, int nb, int causal, float cscale, int L, int hbase, int hcount) {
  typedef AttnCtx<D, BLK> C;
  constexpr int KCH = C::KCH;
  __shared__ __attribute__((aligned(1024))) uint8_t lds_k[C::TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t lds_v[C::TILE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  C cx;
  cx.lds_k = lds_k;
  cx.lds_v = lds_v;
  cx.wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n32 = lane & 31;
  cx.half = lane >> 5;
  cx.cscale = cscale;
  int h, i;
  work_item(blockIdx.x, Hq, Hkv, nb, hbase, hcount, h, i);
  const int G = Hq / Hkv;
  const int g = h / G;
  cx.qr = cx.wave * 32 + n32;  // query row inside the block
  const int x = i * BLK + cx.qr;

  // K tiles live in LDS as rows of 16-byte chunks, chunk c of row r stored at
  // position c ^ (r mod chunks-per-row), so the 32 rows one MFMA operand read
  // touches fall in distinct banks. Copies write LDS linearly (lane l of a
  // wave's copy lands at 16*l), so each thread fetches the global chunk that
  // belongs at its position: a base offset, a fixed step per copy, and a
  // per-copy XOR of the chunk (see copy_tile). Vt tiles are chunk-major in
  // HBM already: an operand read (32 channels of one chunk column) is one
  // contiguous run, and the copy is straight.
  static_assert(C::NTHR % KCH == 0, "copy rows must advance evenly");
  {
    const int kr = tid / KCH, kc = (tid % KCH) ^ (kr & (KCH - 1));
    cx.koff = (kr * Hkv * D + kc * 8) * 2;
    cx.kstep = (C::NTHR / KCH) * Hkv * D * 2;
    cx.voff = tid * 16;  // Vt tiles are copied as stored
    cx.vstep = C::NTHR * 16;
  }
  // An operand read of chunk c in a row r = 32*m + n32 is at r*rowbytes +
  // 16*(c ^ (n32 mod chunks)); with c = 2*cc + half that is kro ^ (32*cc).
  cx.kro = n32 * D * 2 + (((cx.half) ^ (n32 & (KCH - 1))) << 4);
  cx.vro = (cx.half * D + n32) * 16;

  bf16x8 qf[C::DK];
  if (x < L) {
    const bf16x8* src = reinterpret_cast<const bf16x8*>(q + ((size_t)x * Hq + h) * D);
#pragma unroll
    for (int c = 0; c < C::DK; ++c) qf[c] = src[2 * c + cx.half];
  } else {  // past the end of a short last block: computed, never stored
#pragma unroll
    for (int c = 0; c < C::DK; ++c) qf[c] = bf16x8{};
  }

  const size_t row = (size_t)h * nb + i;
  const int cnt = min(max(row_count[row], 0), nb);
  const int32_t* lst = col_idx + row * nb;
  const int jmax = causal ? i : nb - 1;
  const uint8_t* kg = reinterpret_cast<const uint8_t*>(k) + (size_t)g * D * 2;
  const uint8_t* vg = reinterpret_cast<const uint8_t*>(vt) + (size_t)g * nb * C::TILE;
  const size_t kstride = (size_t)BLK * Hkv * D * 2;  // bytes between consecutive key blocks of K
  const size_t k_bytes = (size_t)L * Hkv * D * 2;    // the whole K tensor
  const uint32_t kfull = (uint32_t)((BLK - 1) * Hkv * D * 2 + D * 2);
  auto krsrc = [&](int jj) {
    return tile_rsrc(kg + (size_t)jj * kstride, k_tile_bytes((size_t)g * D * 2 + (size_t)jj * kstride, k_bytes, kfull));
  };
  auto vrsrc = [&](int jj) { return tile_rsrc(vg + (size_t)jj * C::TILE, C::TILE); };
  const int ltail = L - (nb - 1) * BLK;  // keys in the last block (BLK unless it is short)

  f32x16 oacc[C::NT];
#pragma unroll
  for (int t = 0; t < C::NT; ++t) oacc[t] = f32x16{};
  float mrow = kRefStart, lrow = 0.0f;

  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // queries are in registers
  int j = cnt > 0 ? min(max(lst[0], 0), jmax) : 0;
  if (cnt > 0) {
    copy_tile<D, BLK, KCH>(cx, krsrc(j), cx.koff, cx.kstep, lds_k);
    copy_tile<D, BLK, 1>(cx, vrsrc(j), cx.voff, cx.vstep, lds_v);
  }
  // Lists are ascending, so only the last entry can need a mask (the causal
  // diagonal block, or a short last block): the loop never masks, the peeled
  // last entry may.
  for (int c = 0; c + 1 < cnt; ++c) {
    const int jn = min(max(lst[c + 1], 0), jmax);
    attn_tile<D, BLK>(cx, qf, oacc, mrow, lrow, true, krsrc(jn), vrsrc(jn), false, BLK - 1);
    j = jn;
  }
  if (cnt > 0) {
    const bool diag = causal && j == i;
    const bool shortblk = j == nb - 1 && ltail < BLK;
    attn_tile<D, BLK>(cx, qf, oacc, mrow, lrow, false, krsrc(j), vrsrc(j), diag || shortblk,
                      diag ? cx.qr : ltail - 1);
  }

  const float ltot = lrow + __shfl_xor(lrow, 32);
  const float inv = ltot > 0.0f ? 1.0f / ltot : 0.0f;
  if (x >= L) return;
  uint16_t* dst = reinterpret_cast<uint16_t*>(out) + ((size_t)x * Hq + h) * D;
#pragma unroll
  for (int t = 0; t < C::NT; ++t) {
#pragma unroll
    for (int v4 = 0; v4 < 4; ++v4) {
      const int e = t * 32 + 8 * v4 + 4 * cx.half;
      u32x2 w;
      w[0] = pack_bf16x2(oacc[t][4 * v4] * inv, oacc[t][4 * v4 + 1] * inv);
      w[1] = pack_bf16x2(oacc[t][4 * v4 + 2] * inv, oacc[t][4 * v4 + 3] * inv);
      *reinterpret_cast<u32x2*>(dst + e) = w;
    }
  }
}

// ------------------------------------------------------------------ bf16 attention, head pairs

// Two query heads of one KV head share a workgroup of 2 * B/32 waves (two per
// SIMD, 32 queries each). The workgroup walks the merged, ascending block
// list of both heads: each K/Vt tile is copied once for both, and a wave
// computes only the blocks its own head selected. K and Vt are
// double-buffered (four tiles, 128 KiB at B = d = 128): the copy of the next
// block is issued right after the one barrier per block and has the whole
// block's compute to land.
//
// The copies are buffer loads with an LDS destination, and every stage of
// the double buffer is an LDS object of its own with the stage fixed at
// compile time (the block loop is unrolled by two). Both matter to the
// compiler's wait-count insertion: a flat/global LDS copy in flight makes it
// wait for all LDS traffic (lgkmcnt(0)) before every operand read, and a copy
// into the same LDS object as the operands makes it wait for the copy itself
// (vmcnt(0)) before the first read. With both, the operand reads of block j
// run while the copy of block j + 1 is still in flight.
template <int D, int BLK>
struct PairCtx {
  static constexpr int WPH = BLK / 32;               // waves per head
  static constexpr int NTHR = 2 * WPH * 64;          // threads per workgroup
  static constexpr int MT = BLK / 32;                // 32-key subtiles
  static constexpr int NT = D / 32;                  // 32-channel tiles of O
  static constexpr int DK = D / 16;                  // MFMA k-steps over d
  static constexpr int TILE = BLK * D * 2;           // bytes of one K or Vt tile
  static constexpr int NDMA = TILE / (NTHR * 16);    // 16-byte copies per thread per tile
  static constexpr int KCH = D / 8;                  // 16-byte chunks per K row
  static constexpr int VBIAS = 2 * TILE;             // LDS offset of the first Vt stage (after the K stages)
  uint32_t koff, voff;    // this thread's copy source for copy 0, relative to a tile base
  uint32_t kstep, vstep;  // source distance between consecutive copies (bytes)
  int kro, vro;           // operand read offsets for chunk 0 (K: XOR in the chunk index; Vt: add)
  int vro_hi;             // vro + VBIAS, opaque to the optimizer (see the kernel)
  int wave, qr, half;
  float cscale;
};

// One tile: NDMA buffer loads of 16 bytes per lane straight into LDS (lane l
// of a wave lands at 16*l past the wave's slot), from a descriptor based at
// the tile's first byte.
template <int D, int BLK, int CH>
__device__ __forceinline__ void pair_copy(const PairCtx<D, BLK>& cx, __amdgpu_buffer_rsrc_t rsrc, uint32_t off,
                                          uint32_t step, uint8_t* dst) {
  typedef PairCtx<D, BLK> C;
  constexpr int RPC = C::NTHR / CH;
#pragma unroll
  for (int n = 0; n < C::NDMA; ++n)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rsrc,
        reinterpret_cast<__attribute__((address_space(3))) void*>(
            reinterpret_cast<uintptr_t>(dst + (n * C::NTHR + cx.wave * 64) * 16)),
        16, (int)(n * step + (off ^ (((n * RPC) & (CH - 1)) << 4))), 0, 0, 0);
}

// Online softmax of one key block for one wave of a head pair (ref_softmax).
// MASK: keys with index > klim inside the block get probability zero.
template <int D, int BLK, bool MASK>
__device__ __forceinline__ void pair_softmax(const PairCtx<D, BLK>& cx, f32x16 (&sacc)[BLK / 32],
                                             f32x16 (&oacc)[D / 32], float& mrow, float& lrow,
                                             bf16x8 (&pf)[BLK / 32][2], int klim) {
  constexpr int MT = BLK / 32;
  if (MASK) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int key = mt * 32 + 8 * (v >> 2) + 4 * cx.half + (v & 3);
        if (key > klim) sacc[mt][v] = -INFINITY;
      }
  }
  ref_softmax(cx.cscale, sacc, oacc, mrow, lrow, pf);
}

// Rows (of n) after which the KV head an XCD serves moves on by one: each XCD
// then serves every KV head over the launch, so KV heads whose rows select
// more blocks do not keep one XCD busy after the others, while the rows in
// flight on an XCD at one time (about 16) mostly share one KV head's tiles.
__device__ __forceinline__ int rotation_rows(int n) { return n / 16 > 16 ? n / 16 : 16; }

// Launch index -> (KV head g, query block i, head pair p): query blocks in
// decreasing order, the pairs of one (g, i) on one XCD in consecutive slots;
// for each query block the KV heads rotate over the XCDs (rotation_rows).
__device__ __forceinline__ void pair_item(int x, int Hkv, int nb, int npairs, int& g, int& i, int& p) {
  const int nunits = Hkv * nb;
  int u;
  if ((nunits & 7) == 0) {
    const int xcd = x & 7, t = x >> 3;
    p = t % npairs;
    u = (t / npairs) * 8 + xcd;
  } else {
    u = x / npairs;
    p = x % npairs;
  }
  const int r = u / Hkv;  // rows longest first
  i = nb - 1 - r;
  g = (u % Hkv + r / rotation_rows(nb)) % Hkv;
}

// Work item x of the ping-pong kernel for an odd group size G: unit u = (KV
// head g, query blocks nb-1-2*pb and nb-2-2*pb) holds G items, slot `it`:
// the G/2 head pairs of the upper block, the G/2 head pairs of the lower one,
// and last the group's lone head over both blocks (one block per slot). Units
// run longest rows first and, when their count allows, each XCD takes every
// eighth unit, like pair_item.
__device__ __forceinline__ void odd_item(int x, int Hkv, int npb, int G, int& g, int& pb, int& it) {
  const int nunits = Hkv * npb;
  int u;
  if ((nunits & 7) == 0) {
    const int xcd = x & 7, t = x >> 3;
    it = t % G;
    u = (t / G) * 8 + xcd;
  } else {
    u = x / G;
    it = x % G;
  }
  pb = u / Hkv;
  g = (u % Hkv + pb / rotation_rows(npb)) % Hkv;
}

// ------------------------------------------------------------------ bf16 attention, head pairs in ping-pong

// The head-pair workgroup above runs its two waves per SIMD in step: both
// issue their S = K Q^T MFMAs, then both run the softmax on the VALU while
// the matrix unit idles, then both issue O += P V. Here the block is split
// in two half-steps, each closed by a workgroup barrier, and the two heads
// take opposite roles in them:
//
//   half-step 2n    head A: O += P(n-1) V(n-1), S(n) = K(n) Q^T   (MFMA)
//                   head B: softmax(n-1)                            (VALU)
//   half-step 2n+1  head A: softmax(n)
//                   head B: O += P(n-1) V(n-1), S(n) = K(n) Q^T
//
// so the matrix unit of every SIMD is fed by one of its two waves at a time
// while the other computes exponentials. Tiles: K(n) and V(n-1) are read in
// half-steps 2n and 2n+1; the copies of K(n+1) and V(n) are issued in
// half-step 2n (head B's waves before their softmax, head A's after their
// MFMAs, so that no MFMA phase waits behind the copy issue) into the stages
// that held K(n-1) and V(n-2) (last read in half-step 2n-1) and have landed
// at the end of half-step 2n+1. A head that did not select block n skips its
// MFMAs and softmax for it; the barriers and copies are the same for every
// wave.

template <int V>
struct IntConst {
  static constexpr int value = V;
};

// S^T = K Q^T for one wave: the k-step outer and the key subtile inner, so
// consecutive MFMAs feed different accumulators.
template <int D, int BLK>
__device__ __forceinline__ void pp_qk(const PairCtx<D, BLK>& cx, const uint8_t* lds_k, const bf16x8 (&qf)[D / 16],
                                      f32x16 (&sacc)[BLK / 32]) {
  typedef PairCtx<D, BLK> C;
  constexpr int MT = C::MT;
  constexpr int DK = C::DK;
  constexpr int LA = 4;
  constexpr int NQK = MT * DK;
  auto kread = [&](int k) {
    const int cc = k / MT, mt = k % MT;
    return *reinterpret_cast<const bf16x8*>(lds_k + mt * 32 * D * 2 + (cx.kro ^ (cc << 5)));
  };
  bf16x8 ring[LA];
#pragma unroll
  for (int k = 0; k < LA; ++k) ring[k] = kread(k);
#pragma unroll
  for (int k = 0; k < NQK; ++k) {
    const bf16x8 a = ring[k % LA];
    if (k + LA < NQK) ring[k % LA] = kread(k + LA);
    const int cc = k / MT, mt = k % MT;
    sacc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[cc], cc ? sacc[mt] : f32x16{}, 0, 0, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x100, LA, 0);
#pragma unroll
  for (int k = 0; k < NQK - LA; ++k) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, LA, 0);
}

// O^T += Vt P^T for one wave: the key step outer and the channel tile inner.
template <int D, int BLK>
__device__ __forceinline__ void pp_pv(const PairCtx<D, BLK>& cx, const uint8_t* lds_v, const bf16x8 (&pf)[BLK / 32][2],
                                      f32x16 (&oacc)[D / 32]) {
  typedef PairCtx<D, BLK> C;
  constexpr int MT = C::MT;
  constexpr int NT = C::NT;
  constexpr int LA = 4;
  constexpr int NPV = NT * MT * 2;
  auto vread = [&](int k) {
    const int r = k / NT, t = k % NT;
    return *reinterpret_cast<const bf16x8*>(lds_v + (cx.vro_hi - C::VBIAS) + (2 * r * D + t * 32) * 16);
  };
  bf16x8 ring[LA];
#pragma unroll
  for (int k = 0; k < LA; ++k) ring[k] = vread(k);
#pragma unroll
  for (int k = 0; k < NPV; ++k) {
    const bf16x8 a = ring[k % LA];
    if (k + LA < NPV) ring[k % LA] = vread(k + LA);
    const int r = k / NT, t = k % NT;
    oacc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[r >> 1][r & 1], oacc[t], 0, 0, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x100, LA, 1);
#pragma unroll
  for (int k = 0; k < NPV - LA; ++k) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 1);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, LA, 1);
}

// ODD: the group size is odd and work items are decoded by odd_item (each
// slot then has its own query block); otherwise by pair_item (both slots on
// one query block).
// Work queues of the ping-pong kernel: the nitems items split into nq
// interleaved queues (item x in queue x mod nq; with nq = kAttnQueues this is
// the split of pair_item and odd_item over the XCDs). A workgroup claims the
// next unclaimed item of its own XCD's queue or, once that is empty, of the
// following queues. Returns -1 when every queue is empty. Called by all
// threads of the workgroup (one barrier).
static_assert(kAttnQueues == 8, "pair_item and odd_item spread items over the 8 XCDs");
__device__ __forceinline__ int claim_item(int32_t* queues, int nq, int nitems) {
  __shared__ int claimed;
  if (threadIdx.x == 0) {
    const int per = nitems / nq;
    const int own = blockIdx.x % nq;
    int got = -1;
    for (int s = 0; s < nq && got < 0; ++s) {
      const int qi = (own + s) % nq;
      const int t = __hip_atomic_fetch_add(queues + qi, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (t < per) got = t * nq + qi;
    }
    claimed = got;
  }
  __syncthreads();
  return __builtin_amdgcn_readfirstlane(claimed);
}

// ODD: the group size is odd and work items are decoded by odd_item (each
// slot then has its own query block); otherwise by pair_item (both slots on
// one query block). two == 0: workgroup x runs item x. two == 1: as many
// workgroups as items, each claiming up to two items from the work queues
// (claim_item; counters zero at launch, nitems a multiple of nq). The
// workgroups of an XCD that runs faster then drain its queue two items at a
// time and go on to the other XCDs' items, so the XCDs finish together; each
// counter increment hands out at most one item, so every item runs exactly
// once, and workgroups that find every queue empty exit at once. The two
// items are two straight-line copies of the body: a loop over items makes the
// compiler keep its whole register budget and spill.
//
// VARLEN: the launch covers a packed batch of sequences (SeqBatch): item x
// belongs to the sequence whose item range holds it, and is decoded as that
// sequence's own item; the tensors, lists and lengths are that sequence's.
// Each range starts at a multiple of 16, so a sequence's items keep the XCD
// split of pair_item / odd_item; the padding items past a sequence's own
// count exit at once.
template <int D, int BLK, bool ODD, bool VARLEN>
__global__ void __launch_bounds__(4 * BLK) __attribute__((amdgpu_waves_per_eu(2, 2))) attn_bf16_pp_kernel(
    const __bf16* __restrict__ q_all, const __bf16* __restrict__ k_all, const __bf16* __restrict__ vt_all,
    const int32_t* __restrict__ rc_all, const int32_t* __restrict__ ci_all, __bf16* __restrict__ out_all,
    int Hq, int Hkv, int nb_all, int causal, float cscale, int L_all, int32_t* __restrict__ queues, int nq,
    int nitems, int two, const BatchArg<VARLEN> sb) {
  typedef PairCtx<D, BLK> C;
  constexpr int KCH = C::KCH;
  constexpr int MT = C::MT;
  __shared__ __attribute__((aligned(1024))) uint8_t lds_k0[C::TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t lds_k1[C::TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t lds_v0[C::TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t lds_v1[C::TILE];

  // one work item; returns early (per thread) where the item or a row ends
  auto process = [&](const int item_in) __attribute__((always_inline)) {
    const __bf16* q = q_all;
    const __bf16* k = k_all;
    const __bf16* vt = vt_all;
    const int32_t* row_count = rc_all;
    const int32_t* col_idx = ci_all;
    __bf16* out = out_all;
    int nb = nb_all, L = L_all, item = item_in;
    if constexpr (VARLEN) {  // the sequence of this item, and the item inside it (uniform)
      int sq = 0;
      while (sq + 1 < sb.n && item_in >= sb.item_off[sq + 1]) ++sq;
      item = item_in - sb.item_off[sq];
      nb = sb.nb[sq];
      L = sb.L[sq];
      const size_t tok = (size_t)sb.tok_off[sq];
      q = q_all + tok * Hq * D;
      k = k_all + tok * Hkv * D;
      out = out_all + tok * Hq * D;
      vt = reinterpret_cast<const __bf16*>(reinterpret_cast<const uint8_t*>(vt_all) + sb.vt_off[sq]);
      row_count = rc_all + sb.rc_off[sq];
      col_idx = ci_all + sb.ci_off[sq];
      const int Gs = Hq / Hkv;
      const int own = Gs % 2 ? Hkv * ((nb + 1) / 2) * Gs : Hkv * nb * (Gs / 2);
      if (item >= own) return;  // padding up to the next range (uniform, before any barrier)
    }
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    C cx;
    cx.wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int slot = cx.wave / C::WPH;  // 0: head A (MFMAs in even half-steps), 1: head B
    const int n32 = lane & 31;
    cx.half = lane >> 5;
    cx.qr = (cx.wave % C::WPH) * 32 + n32;
    cx.cscale = cscale;
    const int G = Hq / Hkv;
    // slot 0 runs head hA on query block iA, slot 1 head hB on block iB
    int g, hA, hB, iA, iB;
    bool hasB = true;
    if constexpr (!ODD) {  // G even: heads 2p and 2p+1 of one query block
      int p;
      pair_item(item, Hkv, nb, G / 2, g, iA, p);
      iB = iA;
      hA = g * G + 2 * p;
      hB = hA + 1;
    } else {
      int pb, it;
      odd_item(item, Hkv, (nb + 1) / 2, G, g, pb, it);
      const int i0 = nb - 1 - 2 * pb, i1 = i0 - 1;
      if (it < 2 * (G / 2)) {
        iA = iB = it < G / 2 ? i0 : i1;
        if (iA < 0) return;  // odd nb: the lowest unit has one block (uniform exit, before any barrier)
        hA = g * G + 2 * (it % (G / 2));
        hB = hA + 1;
      } else {  // the lone head, block i0 in slot 0 and i1 (if any) in slot 1
        hA = hB = g * G + G - 1;
        iA = i0;
        iB = i1;
        hasB = i1 >= 0;
      }
    }
    const int h = slot ? hB : hA;
    const int i = slot ? iB : iA;
    const bool active = slot == 0 || hasB;
    const int x = i * BLK + cx.qr;

    static_assert(C::NTHR % KCH == 0, "copy rows must advance evenly");
    {
      const int kr = tid / KCH, kc = (tid % KCH) ^ (kr & (KCH - 1));
      cx.koff = (kr * Hkv * D + kc * 8) * 2;
      cx.kstep = (C::NTHR / KCH) * Hkv * D * 2;
      cx.voff = tid * 16;  // Vt tiles are copied as stored
      cx.vstep = C::NTHR * 16;
    }
    cx.kro = n32 * D * 2 + (((cx.half) ^ (n32 & (KCH - 1))) << 4);
    cx.vro = (cx.half * D + n32) * 16;
    // The Vt stages follow the two K stages in LDS (at 64 and 96 KiB for d =
    // 128), beyond the 16-bit offset field of ds_read_b128. Written as lds_v +
    // vro + offset, every read costs a VALU add (the stage base folds into
    // the constant, which then does not fit); written as lds_v + (vro_hi -
    // VBIAS) + offset with vro_hi opaque, the constants cancel against the
    // base and each read is vro_hi plus an immediate. Either form addresses
    // the same bytes.
    cx.vro_hi = cx.vro + C::VBIAS;
    asm volatile("" : "+v"(cx.vro_hi));

    bf16x8 qf[C::DK];
    if (active && x < L) {
      const bf16x8* src = reinterpret_cast<const bf16x8*>(q + ((size_t)x * Hq + h) * D);
#pragma unroll
      for (int c = 0; c < C::DK; ++c) qf[c] = src[2 * c + cx.half];
    } else {
#pragma unroll
      for (int c = 0; c < C::DK; ++c) qf[c] = bf16x8{};
    }

    // the two block lists, merged on the fly (all values wave-uniform)
    const int ltail = L - (nb - 1) * BLK;   // keys in the last block (BLK unless it is short)
    // largest admissible key block of each slot's row, and of the merged walk (iA >= iB)
    const int jlastA = causal ? iA : nb - 1;
    const int jlastB = causal ? iB : nb - 1;
    const int jlast = jlastA;
    // each slot's masked block, if any: its causal diagonal, else a short last block
    const int jdiagA = causal ? iA : (ltail < BLK ? nb - 1 : nb);
    const int jdiagB = causal ? iB : (ltail < BLK ? nb - 1 : nb);
    const int klim = causal ? cx.qr : ltail - 1;
    const size_t rowA = (size_t)hA * nb + iA, rowB = (size_t)hB * nb + iB;
    const int cntA = min(max(row_count[rowA], 0), nb);
    const int cntB = hasB ? min(max(row_count[rowB], 0), nb) : 0;
    const int32_t* la = col_idx + rowA * nb;
    const int32_t* lb = col_idx + rowB * nb;
    constexpr int kNone = 1 << 30;
    int ia = 0, ib = 0;
    int ja = cntA > 0 ? min(max(la[0], 0), jlastA) : kNone;
    int jb = cntB > 0 ? min(max(lb[0], 0), jlastB) : kNone;

    const uint8_t* kg = reinterpret_cast<const uint8_t*>(k) + (size_t)g * D * 2;
    const uint8_t* vg = reinterpret_cast<const uint8_t*>(vt) + (size_t)g * nb * C::TILE;
    const size_t kstride = (size_t)BLK * Hkv * D * 2;  // bytes between consecutive key blocks of K

    f32x16 oacc[C::NT];
#pragma unroll
    for (int t = 0; t < C::NT; ++t) oacc[t] = f32x16{};
    float mrow = kRefStart, lrow = 0.0f;
    f32x16 sacc[MT];
    bf16x8 pf[MT][2];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) sacc[mt] = f32x16{};
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) pf[mt][0] = pf[mt][1] = bf16x8{};

    constexpr int kWaitAll = 0x0070;  // vmcnt(0) lgkmcnt(0)
    __builtin_amdgcn_s_waitcnt(kWaitAll);
    const uint32_t kbytes = (uint32_t)((BLK - 1) * Hkv * D * 2 + D * 2);
    const size_t k_bytes = (size_t)L * Hkv * D * 2;  // the whole K tensor
    auto copy_k = [&](int jj, uint8_t* dst) {
      const uint32_t kb = k_tile_bytes((size_t)g * D * 2 + (size_t)jj * kstride, k_bytes, kbytes);
      pair_copy<D, BLK, KCH>(cx, tile_rsrc(kg + (size_t)jj * kstride, kb), cx.koff, cx.kstep, dst);
    };
    auto copy_v = [&](int jj, uint8_t* dst) {
      pair_copy<D, BLK, 1>(cx, tile_rsrc(vg + (size_t)jj * C::TILE, C::TILE), cx.voff, cx.vstep, dst);
    };
    int j = min(ja, jb);  // block n of the merged list (> jlast: the list is done)
    if (j <= jlast) copy_k(j, lds_k0);
    __builtin_amdgcn_s_waitcnt(kWaitAll);
    __builtin_amdgcn_s_barrier();

    // Block n with K(n) in kc and V(n-1) in vp; K(n+1) is copied to kn and V(n)
    // to vc. Returns false after the step past the last block (which only
    // finishes the last P V). SLOT is this wave's head: 0 issues its MFMAs in
    // the first half-step, 1 in the second.
    auto run = [&](auto slot_c) __attribute__((always_inline)) {
      constexpr int SLOT = decltype(slot_c)::value;
      bool sel_prev = false;  // this wave's head selected block n-1
      auto mfma_phase = [&](bool sel, bool diag, const uint8_t* kc, const uint8_t* vp) __attribute__((always_inline)) {
        if (sel_prev) pp_pv<D, BLK>(cx, vp, pf, oacc);
        if (sel) {
          pp_qk<D, BLK>(cx, kc, qf, sacc);
          if (diag) {  // keys past the lane's limit get score -inf (probability zero)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
              for (int v = 0; v < 16; ++v) {
                const int key = mt * 32 + 8 * (v >> 2) + 4 * cx.half + (v & 3);
                if (key > klim) sacc[mt][v] = -INFINITY;
              }
          }
        }
      };
      auto step = [&](const uint8_t* kc, uint8_t* kn, const uint8_t* vp, uint8_t* vc) __attribute__((always_inline)) {
        const bool have = j <= jlast;
        const bool selA = have && ja == j, selB = have && jb == j;
        if (selA) {
          ++ia;
          ja = ia < cntA ? min(max(la[ia], 0), jlastA) : kNone;
        }
        if (selB) {
          ++ib;
          jb = ib < cntB ? min(max(lb[ib], 0), jlastB) : kNone;
        }
        const int jn = min(ja, jb);
        const bool sel = SLOT ? selB : selA;
        const bool diag = have && j == (SLOT ? jdiagB : jdiagA);
        // each wave issues its share of the copies of K(n+1) and V(n) in
        // half-step 2n where it is off the critical path: head B before its
        // softmax, head A after its MFMAs
        auto copies = [&]() __attribute__((always_inline)) {
          if (jn <= jlast) copy_k(jn, kn);
          if (have) copy_v(j, vc);
        };
        // half-step 2n
        if (SLOT == 0) {
          mfma_phase(sel, diag, kc, vp);
          copies();
        } else {
          copies();
          if (sel_prev) pair_softmax<D, BLK, false>(cx, sacc, oacc, mrow, lrow, pf, 0);
        }
        __builtin_amdgcn_s_barrier();
        // half-step 2n+1
        if (SLOT == 0) {
          if (sel) pair_softmax<D, BLK, false>(cx, sacc, oacc, mrow, lrow, pf, 0);
        } else {
          mfma_phase(sel, diag, kc, vp);
        }
        // this block's reads are done and the copies issued at its start have landed
        __builtin_amdgcn_s_waitcnt(kWaitAll);
        __builtin_amdgcn_s_barrier();
        sel_prev = sel;
        j = jn;
        return have;
      };
      // two blocks per trip, so that each stage's LDS objects are known at compile time
      while (step(lds_k0, lds_k1, lds_v1, lds_v0) && step(lds_k1, lds_k0, lds_v0, lds_v1)) {
      }
    };
    if (slot == 0)
      run(IntConst<0>{});
    else
      run(IntConst<1>{});

    if (!active || x >= L) return;
    const float ltot = lrow + __shfl_xor(lrow, 32);
    const float inv = ltot > 0.0f ? 1.0f / ltot : 0.0f;
    uint16_t* dst = reinterpret_cast<uint16_t*>(out) + ((size_t)x * Hq + h) * D;
#pragma unroll
    for (int t = 0; t < C::NT; ++t) {
#pragma unroll
      for (int v4 = 0; v4 < 4; ++v4) {
        const int e = t * 32 + 8 * v4 + 4 * cx.half;
        u32x2 w;
        w[0] = pack_bf16x2(oacc[t][4 * v4] * inv, oacc[t][4 * v4 + 1] * inv);
        w[1] = pack_bf16x2(oacc[t][4 * v4 + 2] * inv, oacc[t][4 * v4 + 3] * inv);
        *reinterpret_cast<u32x2*>(dst + e) = w;
      }
    }
  };

  const int item0 = two ? claim_item(queues, nq, nitems) : (int)blockIdx.x;
  if (item0 < 0) return;  // uniform
  process(item0);
  if (!two) return;
  __syncthreads();  // this item's LDS reads and the claimed index are done
  const int item1 = claim_item(queues, nq, nitems);
  if (item1 < 0) return;
  process(item1);
}

// ------------------------------------------------------------------ fp32 attention

// float32 path on the fp32 matrix cores (v_mfma_f32_16x16x4f32). A workgroup of
// f32_waves(D) waves serves one query head and one tile of 16 queries (so even a
// 1K-token layer spreads over a few hundred workgroups); the row's selected
// blocks are cut into 16-key subtiles and wave w takes subtiles w, w + waves,
// ... Lane (i = lane % 16, grp = lane / 16) keeps its own running maximum, sum
// and O for query i; the waves' parts are merged at the end (each rescaled to
// the common maximum). The operands come from global memory straight into
// registers in the matrix layout, the next subtile's while the current one is
// computed; no staging through LDS:
//   S^T = K Q^T, D/4 MFMAs: step s takes channel grp * D/4 + s from every lane
//     group (the sum over channels may run in any order), so A = K[key i]
//     and B = Q[query i] are each D/4 contiguous floats of the lane; the lane
//     then holds the scores of keys 4 grp + r, r < 4, for query i;
//   online softmax in base 2 on those 4 scores (maximum across the 4 groups);
//   O^T += V^T P^T, 4 * D/16 MFMAs: step r pairs key 4 grp + r across the
//     groups, exactly the key of the lane's P register r, so P is the B
//     operand as it stands; row i of output tile c is channel i * D/16 + c,
//     so A = V[key 4 grp + r][i * D/16 + c], D/16 contiguous floats per key.
// After the loop the lane holds O^T for channels grp * D/4 ... grp * D/4 +
// D/4 - 1 of query i, in order (4 rows per output tile, D/16 tiles).
// Waves per workgroup: 8, two per SIMD (16 at d = 64, four per SIMD within
// 128 VGPRs, ran the 1K-token layer 13% slower: twice the parts to merge).
__host__ __device__ constexpr int f32_waves(int) { return 8; }
typedef float f32x4 __attribute__((ext_vector_type(4)));

// The larger of x and the value of the lane 16 (32) apart, by one permlane
// swap (no LDS round trip).
__device__ __forceinline__ float max_lane16(float x) {
  const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
}
__device__ __forceinline__ float max_lane32(float x) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
}
// x plus the value of the lane 16 (32) apart
__device__ __forceinline__ float add_lane16(float x) {
  const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
}
__device__ __forceinline__ float add_lane32(float x) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
}

template <int D>
struct F32Lds {
  static constexpr int OP = D + 4;                 // padded row of a wave's O part (floats)
  static constexpr int PER_WAVE = 16 * OP + 32;    // O [16][OP], maximum [16], sum [16]
  static constexpr size_t BYTES = (size_t)f32_waves(D) * PER_WAVE * sizeof(float);
};

template <int D, int BLK>
__global__ void __launch_bounds__(f32_waves(D) * 64) attn_f32_kernel(const float* __restrict__ q,
                                                                 const float* __restrict__ k,
                                                                 const float* __restrict__ v,
                                                                 const int32_t* __restrict__ row_count,
                                                                 const int32_t* __restrict__ col_idx,
                                                                 float* __restrict__ out, int Hq, int Hkv, int nb,
                                                                 int causal, float cscale, int L, int ntiles) {
  typedef F32Lds<D> Lds;
  constexpr int KQ = D / 4;    // channels of a lane in S^T (one quarter)
  constexpr int VC = D / 16;   // channels of a lane per key in O^T += V^T P^T, and output tiles
  constexpr int NST = BLK / 16;
  constexpr int W = f32_waves(D);
  extern __shared__ float smem[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, grp = lane >> 4;
  // longest rows first: query tiles in decreasing order, heads adjacent
  const int qt = ntiles - 1 - (int)blockIdx.x / Hq;
  const int h = (int)blockIdx.x % Hq;
  const int g = h / (Hq / Hkv);
  const int q0 = qt * 16;
  const int i = q0 / BLK;        // query block of this tile
  const int x = q0 + li;         // this lane's query

  // queries past L (the last tile of a ragged layer) read row L - 1, replaced
  // by zeros after the load (a load under a branch would leave it in flight
  // into the loop, where the wait counts then cover every load)
  float qf[KQ];
  {
    const f32x4* src = reinterpret_cast<const f32x4*>(q + ((size_t)min(x, L - 1) * Hq + h) * D + grp * KQ);
    const bool qin = x < L;
#pragma unroll
    for (int c = 0; c < KQ / 4; ++c) {
      f32x4 t = src[c];
      if (!qin) t = f32x4{0.f, 0.f, 0.f, 0.f};
      qf[4 * c] = t[0]; qf[4 * c + 1] = t[1]; qf[4 * c + 2] = t[2]; qf[4 * c + 3] = t[3];
    }
  }

  const size_t row = (size_t)h * nb + i;
  const int cnt = min(max(row_count[row], 0), nb);
  const int32_t* lst = col_idx + row * nb;
  const int jmax = causal ? i : nb - 1;
  const int total = cnt * NST;  // subtiles of the row's blocks
  const int qlast = min(q0 + 15, L - 1);
  const int klim = causal ? min(x, L - 1) : L - 1;  // last key the lane's query sees

  // first key of subtile t of the row (any t: past the list it reads entry 0,
  // unused); t is the same in every lane, and so is the key
  auto key_of = [&](int t) {
    const int c = t < total ? t / NST : 0;
    return __builtin_amdgcn_readfirstlane(min(max(lst[c], 0), jmax) * BLK + (t % NST) * 16);
  };
  // K rows key0 + li (quarter grp) and V rows key0 + 4 grp + r (D/16 channels)
  // through buffer descriptors that start at row key0 and end at row L or 16
  // rows on, so rows past L read as zeros with no branch and no select on the
  // loaded values: nothing waits for the loads until the subtile is computed.
  // A subtile past the row's list gets an empty range: its loads are issued
  // all the same, with no memory access, since a load under a branch would make
  // every later wait cover the loads of both sides.
  const uint32_t rowb = (uint32_t)(Hkv * D * 4);
  auto load = [&](int t, int key0, float (&kr)[KQ], float (&vr)[4][VC]) {
    const size_t base = ((size_t)key0 * Hkv + g) * D;
    // the range ends where row key0 + rows begins (rows = the subtile's keys
    // before L; 32-bit scalar arithmetic): every load of a row below it lies
    // inside, every load of a row past it outside
    const int rows = t < total ? min(L - key0, 16) : 0;
    const uint32_t nbytes = rows <= 0 ? 0u : (uint32_t)rows * rowb - (uint32_t)(g * D * 4);
    const __amdgpu_buffer_rsrc_t kr_rs = tile_rsrc(reinterpret_cast<const uint8_t*>(k + base), nbytes);
    const __amdgpu_buffer_rsrc_t vr_rs = tile_rsrc(reinterpret_cast<const uint8_t*>(v + base), nbytes);
    const uint32_t koff = li * rowb + grp * KQ * 4;
#pragma unroll
    for (int c = 0; c < KQ / 4; ++c) {
      const f32x4 t = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(kr_rs, koff + 16 * c, 0, 0));
      kr[4 * c] = t[0]; kr[4 * c + 1] = t[1]; kr[4 * c + 2] = t[2]; kr[4 * c + 3] = t[3];
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const uint32_t voff = (4 * grp + r) * rowb + li * VC * 4;
#pragma unroll
      for (int c = 0; c < VC / 4; ++c) {
        const f32x4 t = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(vr_rs, voff + 16 * c, 0, 0));
        vr[r][4 * c] = t[0]; vr[r][4 * c + 1] = t[1]; vr[r][4 * c + 2] = t[2]; vr[r][4 * c + 3] = t[3];
      }
    }
  };

  f32x4 oacc[VC];
#pragma unroll
  for (int c = 0; c < VC; ++c) oacc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  float mrow = -INFINITY, lrow = 0.0f;

  // one subtile: scores, online softmax, O^T += V^T P^T
  auto compute = [&](int key0, const float (&kr)[KQ], const float (&vr)[4][VC]) {
    // subtiles with no key visible to any query of the tile are skipped (wave-uniform)
    if (key0 >= L || (causal && key0 > qlast)) return;
    f32x4 sacc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KQ; ++s) sacc = __builtin_amdgcn_mfma_f32_16x16x4f32(kr[s], qf[s], sacc, 0, 0, 0);
    float tmax = -INFINITY;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if (key0 + 4 * grp + r > klim) sacc[r] = -INFINITY;
      tmax = fmaxf(tmax, sacc[r]);
    }
    tmax = max_lane32(max_lane16(tmax));
    const float mnew = fmaxf(mrow, tmax * cscale);
    const float mref = mnew == -INFINITY ? 0.0f : mnew;  // a query with nothing visible yet stays at zero
    const float alpha = exp2_approx(mrow - mref);
    lrow *= alpha;
#pragma unroll
    for (int c = 0; c < VC; ++c) oacc[c] *= alpha;
    mrow = mnew;
    float pv[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      pv[r] = exp2_approx(__builtin_fmaf(sacc[r], cscale, -mref));
      lrow += pv[r];
    }
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int c = 0; c < VC; ++c) oacc[c] = __builtin_amdgcn_mfma_f32_16x16x4f32(vr[r][c], pv[r], oacc[c], 0, 0, 0);
  };

  // Two register sets in turn: while one subtile is computed the next one's
  // K and V are in flight, and the list entry of the one after that.
  float ka[KQ], va[4][VC], kb[KQ], vb[4][VC];
  int t = __builtin_amdgcn_readfirstlane(wave);
  int keya = key_of(t);
  int keyb = key_of(t + W);
  load(t, keya, ka, va);
  while (t < total) {
    load(t + W, keyb, kb, vb);
    const int keyc = key_of(t + 2 * W);
    compute(keya, ka, va);
    t += W;
    if (t >= total) break;
    load(t + W, keyc, ka, va);
    const int keyd = key_of(t + 2 * W);
    compute(keyb, kb, vb);
    t += W;
    keya = keyc;  // set A now holds subtile t
    keyb = keyd;
  }

  // merge the waves' parts: O [16][OP], the maximum and the sum per query
  float* ob = smem + wave * Lds::PER_WAVE;
  {
    // output tile c, row 4 grp + rr is channel (4 grp + rr) * VC + c
    float* dst = ob + li * Lds::OP + grp * KQ;
#pragma unroll
    for (int rr = 0; rr < 4; ++rr)
#pragma unroll
      for (int c = 0; c < VC; ++c) dst[rr * VC + c] = oacc[c][rr];
  }
  const float ltot = add_lane32(add_lane16(lrow));
  if (grp == 0) {
    ob[16 * Lds::OP + li] = mrow;
    ob[16 * Lds::OP + 16 + li] = ltot;
  }
  __syncthreads();
  constexpr int TPQ = W * 64 / 16;  // threads per query
  constexpr int CPT = D / TPQ;              // channels per thread
  static_assert(CPT >= 1 && D % TPQ == 0, "channels split evenly over a query's threads");
  const int qq = tid / TPQ, part = tid % TPQ;
  const int xo = q0 + qq;
  float mw[W], m = -INFINITY;
#pragma unroll
  for (int w = 0; w < W; ++w) {
    mw[w] = smem[w * Lds::PER_WAVE + 16 * Lds::OP + qq];
    m = fmaxf(m, mw[w]);
  }
  const float mr = m == -INFINITY ? 0.0f : m;
  float aw[W], l = 0.0f;
#pragma unroll
  for (int w = 0; w < W; ++w) {
    aw[w] = exp2_approx(mw[w] - mr);
    l += aw[w] * smem[w * Lds::PER_WAVE + 16 * Lds::OP + 16 + qq];
  }
  const float inv = l > 0.0f ? 1.0f / l : 0.0f;
  if (xo >= L) return;
#pragma unroll
  for (int e = 0; e < CPT; ++e) {
    const int ch = part * CPT + e;
    float o = 0.0f;
#pragma unroll
    for (int w = 0; w < W; ++w) o += aw[w] * smem[w * Lds::PER_WAVE + qq * Lds::OP + ch];
    out[((size_t)xo * Hq + h) * D + ch] = o * inv;
  }
}

}  // namespace

// Compute units of the device that runs `st`, looked up once per device (the
// count never changes while the process runs).
static hipError_t stream_cu_count(hipStream_t st, int* ncu) {
  static std::atomic<int> cached[64];
  int dev = 0;
  hipError_t e = hipStreamGetDevice(st, &dev);
  if (e != hipSuccess) return e;
  if (dev >= 0 && dev < 64) {
    const int c = cached[dev].load(std::memory_order_relaxed);
    if (c > 0) {
      *ncu = c;
      return hipSuccess;
    }
  }
  int n = 0;
  e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  if (n <= 0) return hipErrorInvalidDevice;
  if (dev >= 0 && dev < 64) cached[dev].store(n, std::memory_order_relaxed);
  *ncu = n;
  return hipSuccess;
}

hipError_t launch_transpose_v(const Geometry& g, const void* v, void* vt, int32_t* queues, hipStream_t st) {
  const dim3 grid((unsigned)(g.Hkv * g.nb));
  const __bf16* vv = static_cast<const __bf16*>(v);
  __bf16* out = static_cast<__bf16*>(vt);
  const NoBatch nob{};
#define RR_TV(DV, BV) transpose_v_kernel<DV, BV, false><<<grid, 256, 0, st>>>(vv, out, g.Hkv, g.nb, g.L, queues, nob)
  if (g.d == 128 && g.B == 128) RR_TV(128, 128);
  else if (g.d == 128 && g.B == 64) RR_TV(128, 64);
  else if (g.d == 64 && g.B == 128) RR_TV(64, 128);
  else RR_TV(64, 64);
#undef RR_TV
  return hipGetLastError();
}

hipError_t attn_cu_count(hipStream_t st, int* ncu) { return stream_cu_count(st, ncu); }

bool attn_pair_shape(const Geometry& g) { return g.bf16 && g.B == 128; }

int attn_items(const Geometry& g) {
  const int G = g.Hq / g.Hkv;
  return G % 2 ? g.Hkv * ((g.nb + 1) / 2) * G : g.Hkv * g.nb * (G / 2);
}

hipError_t launch_transpose_v_batched(const Geometry& g, const SeqBatch& sb, const void* v, void* vt,
                                      int32_t* queues, hipStream_t st) {
  if (!attn_pair_shape(g) || sb.n < 1 || sb.n > kMaxSeqPerLaunch) return hipErrorInvalidValue;
  const dim3 grid((unsigned)sb.tile_off[sb.n]);
  const __bf16* vv = static_cast<const __bf16*>(v);
  __bf16* out = static_cast<__bf16*>(vt);
  if (g.d == 128) transpose_v_kernel<128, 128, true><<<grid, 256, 0, st>>>(vv, out, g.Hkv, 0, 0, queues, sb);
  else transpose_v_kernel<64, 128, true><<<grid, 256, 0, st>>>(vv, out, g.Hkv, 0, 0, queues, sb);
  return hipGetLastError();
}

hipError_t launch_attention(const Geometry& g, const void* q, const void* k, const void* v,
                            const void* vt, int32_t* queues, const int32_t* row_count,
                            const int32_t* col_idx, void* out, hipStream_t st) {
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
                                                      g.Hkv, g.nb, g.causal, cscale, g.L, 0,     \
                                                      g.Hq / g.Hkv);                              \
    return hipGetLastError();                                                                     \
  }
    const int G = g.Hq / g.Hkv;
    if (g.B == 128) {
      // Even group: G/2 head pairs per (KV head, query block). Odd group
      // (G = 1 included): G items per (KV head, two query blocks), the lone
      // head of the group paired with itself over the two blocks (odd_item).
      // With G = 1 every item is such a lone head: 13-17% faster than one
      // head per workgroup on 4K-32K MHA layers.
      const int nunits = G % 2 ? g.Hkv * ((g.nb + 1) / 2) : g.Hkv * g.nb;
      const int nitems = G % 2 ? nunits * G : nunits * (G / 2);
      // Two items per workgroup from per-XCD queues where the items map onto
      // the XCDs and each CU has more than 16 of them; below that the claims'
      // atomic round trips cost more than the balance gains.
      const int nq = nunits % kAttnQueues == 0 ? kAttnQueues : 1;
      int ncu = 0;
      const hipError_t e = stream_cu_count(st, &ncu);
      if (e != hipSuccess) return e;
      const int two = nq == kAttnQueues && nitems > 16 * ncu ? 1 : 0;
      const dim3 fgrid((unsigned)nitems);
      const NoBatch nob{};
#define RR_PP_LAUNCH(DV, ODD)                                                                             \
  attn_bf16_pp_kernel<DV, 128, ODD, false><<<fgrid, 512, 0, st>>>(qq, kk, vv, row_count, col_idx, oo, g.Hq, g.Hkv, \
                                                                  g.nb, g.causal, cscale, g.L, queues, nq, nitems, two, \
                                                                  nob)
      if (g.d == 128) {
        if (G % 2) RR_PP_LAUNCH(128, true); else RR_PP_LAUNCH(128, false);
      } else {
        if (G % 2) RR_PP_LAUNCH(64, true); else RR_PP_LAUNCH(64, false);
      }
#undef RR_PP_LAUNCH
      return hipGetLastError();
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
    const size_t lds = F32Lds<DV>::BYTES;                                                         \
    hipError_t fe = hipFuncSetAttribute(reinterpret_cast<const void*>(&attn_f32_kernel<DV, BV>),    \
                                        hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);     \
    if (fe != hipSuccess) return fe;                                                              \
    attn_f32_kernel<DV, BV><<<f32grid, f32_waves(DV) * 64, lds, st>>>(qq, kk, vv, row_count, col_idx, oo, \
                                                                 g.Hq, g.Hkv, g.nb, g.causal, cscale, \
                                                                 g.L, ntiles);                    \
    return hipGetLastError();                                                                     \
  }
  const int ntiles = (g.L + 15) / 16;
  const dim3 f32grid((unsigned)(g.Hq * ntiles));
  RR_F32_CASE(128, 128)
  RR_F32_CASE(128, 64)
  RR_F32_CASE(64, 128)
  RR_F32_CASE(64, 64)
#undef RR_F32_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_attention_batched(const Geometry& g, const SeqBatch& sb, const void* q, const void* k,
                                    const void* vt, int32_t* queues, const int32_t* row_count,
                                    const int32_t* col_idx, void* out, hipStream_t st) {
  if (!attn_pair_shape(g) || sb.n < 1 || sb.n > kMaxSeqPerLaunch) return hipErrorInvalidValue;
  const float cscale = (1.0f / sqrtf((float)g.d)) * 1.4426950408889634f;
  const int G = g.Hq / g.Hkv;
  const int nitems = sb.item_off[sb.n];  // a multiple of 16: every range starts on one
  int ncu = 0;
  const hipError_t e = stream_cu_count(st, &ncu);
  if (e != hipSuccess) return e;
  // One item per workgroup in launch order: claiming two items per workgroup
  // from the per-XCD queues (as the single-sequence launch does at 128K-class
  // sizes) made the eight-sequence 128K-token batch 6% slower, the static
  // order 1% faster than one launch per sequence.
  (void)ncu;
  const int two = 0;
  const dim3 fgrid((unsigned)nitems);
  const __bf16* qq = static_cast<const __bf16*>(q);
  const __bf16* kk = static_cast<const __bf16*>(k);
  const __bf16* vv = static_cast<const __bf16*>(vt);
  __bf16* oo = static_cast<__bf16*>(out);
#define RR_PPB_LAUNCH(DV, ODD)                                                                            \
  attn_bf16_pp_kernel<DV, 128, ODD, true><<<fgrid, 512, 0, st>>>(qq, kk, vv, row_count, col_idx, oo, g.Hq, g.Hkv, \
                                                                 0, g.causal, cscale, 0, queues, kAttnQueues, nitems, \
                                                                 two, sb)
  if (g.d == 128) {
    if (G % 2) RR_PPB_LAUNCH(128, true); else RR_PPB_LAUNCH(128, false);
  } else {
    if (G % 2) RR_PPB_LAUNCH(64, true); else RR_PPB_LAUNCH(64, false);
  }
#undef RR_PPB_LAUNCH
  return hipGetLastError();
}

}  // namespace rr
