// Measured roofline denominators on one MI355X (gfx950), as a standalone
// program beside bench.py (not part of the library):
//   - bf16 MFMA rate of v_mfma_f32_32x32x16_bf16 with register operands (one
//     and two waves per SIMD) and with one LDS-fed operand per MFMA (one
//     ds_read_b128 per MFMA, two waves per SIMD: the attention's feed), with
//     small-integer operands and with pseudo-random ones (the chip's clock
//     under MFMA load depends on how many multiplier bits toggle);
//   - fp32 MFMA rate of v_mfma_f32_32x32x2f32 with register operands;
//   - HBM: a 1 GiB device copy (read + write) and a 1 GiB stream read;
//   - the decode attention's read pattern over a K/V cache of [L][Hkv][128]
//     bf16 (a grid-stride stream and the per-(KV head, run of blocks) walk).
// Every rate is the best of several timed repetitions (HIP events). Prints
// one JSON line per measurement and a last line {"summary": {...}}.
//   - (chains) the rate of one wave per SIMD with 1, 2, 4 or 8 independent
//     accumulator chains;
//   - (coexec) an LDS-fed MFMA stream beside a softmax-like VALU stream on the
//     same SIMDs, each alone and both together.
// Usage: peak [all|mfma|hbm|cache|chains] [L] [Hkv], or peak coexec [valu rounds]
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#define CHECK(x)                                                                          \
  do {                                                                                    \
    hipError_t e_ = (x);                                                                  \
    if (e_ != hipSuccess) {                                                               \
      fprintf(stderr, "%s:%d %s: %s\n", __FILE__, __LINE__, #x, hipGetErrorString(e_));   \
      exit(1);                                                                            \
    }                                                                                     \
  } while (0)

// ------------------------------------------------------------------ MFMA rate

constexpr int kAcc = 8;          // independent accumulators per wave
constexpr int kLdsSlots = 32;    // 1 KiB operand slots per wave, read round-robin
constexpr int kLdsBytes = 96 * 1024;  // > 80 KiB: one workgroup per CU

// A pseudo-random value in [-2, 2) from (seed, index), by a 32-bit integer
// hash (xorshift-multiply); operands drawn from it toggle every multiplier
// bit the way real activations do, where small-integer operands would not.
__device__ __forceinline__ float hash_value(uint32_t seed, uint32_t i) {
  uint32_t x = seed * 0x9E3779B9u ^ (i + 0x7F4A7C15u);
  x ^= x >> 16;
  x *= 0x85EBCA6Bu;
  x ^= x >> 13;
  x *= 0xC2B2AE35u;
  x ^= x >> 16;
  return (float)(x >> 8) * (4.0f / 16777216.0f) - 2.0f;
}

// Register operands: NACC independent MFMA chains per wave. The operands come
// from the thread index (small integers, or pseudo-random values with RAND),
// and the accumulators are stored at the end, so nothing can be folded away.
template <int THREADS, bool RAND>
__global__ void __launch_bounds__(THREADS) mfma_bf16_reg(int iters, float* out) {
  extern __shared__ uint8_t lds_pad[];  // sized by the launch to force one workgroup per CU
  (void)lds_pad;
  const int t = threadIdx.x;
  const uint32_t gt = blockIdx.x * THREADS + t;
  bf16x8 a, b;
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(RAND ? hash_value(1, gt * 8 + e) : (float)((t + e) & 7));
    b[e] = (__bf16)(RAND ? hash_value(2, gt * 8 + e) : (float)((t * 3 + e) & 7));
  }
  f32x16 acc[kAcc];
  for (int n = 0; n < kAcc; ++n) acc[n] = f32x16{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int n = 0; n < kAcc; ++n) acc[n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[n], 0, 0, 0);
  }
  float s = 0.0f;
  for (int n = 0; n < kAcc; ++n)
    for (int v = 0; v < 16; ++v) s += acc[n][v];
  out[(size_t)blockIdx.x * THREADS + t] = s;
}

// One LDS-fed A operand per MFMA: each wave reads 16 bytes per lane from a
// rotating 1 KiB slot (the address changes every MFMA, so no read can be
// hoisted out of the loop), B stays in registers.
template <int THREADS, bool RAND>
__global__ void __launch_bounds__(THREADS) mfma_bf16_lds(int iters, float* out) {
  extern __shared__ uint8_t lds[];
  const int t = threadIdx.x, lane = t & 63;
  const uint32_t gt = blockIdx.x * THREADS + t;
  // fill the kLdsSlots * 1 KiB operand area (every wave reads the same one)
  for (int i = t; i < kLdsSlots * 64; i += THREADS) {
    bf16x8 x;
    for (int e = 0; e < 8; ++e)
      x[e] = (__bf16)(RAND ? hash_value(3, (blockIdx.x * kLdsSlots * 64 + i) * 8 + e) : (float)((i + e) & 7));
    *reinterpret_cast<bf16x8*>(lds + (size_t)i * 16) = x;
  }
  __syncthreads();
  bf16x8 b;
  for (int e = 0; e < 8; ++e) b[e] = (__bf16)(RAND ? hash_value(4, gt * 8 + e) : (float)((t * 3 + e) & 7));
  f32x16 acc[kAcc];
  for (int n = 0; n < kAcc; ++n) acc[n] = f32x16{};
  // operand reads run kRing MFMAs ahead through a register ring, the issue
  // order pinned (one MFMA, then the read kRing steps ahead), as in the
  // attention kernel's MFMA loops
  constexpr int kRing = 4;
  auto read = [&](int step) {
    return *reinterpret_cast<const bf16x8*>(lds + (step & (kLdsSlots - 1)) * 1024 + lane * 16);
  };
  bf16x8 ring[kRing];
  for (int n = 0; n < kRing; ++n) ring[n] = read(n);
  // 32 MFMAs per trip (four per accumulator), so the wait for the reads in
  // flight across the loop's back edge comes once per 32 MFMAs, as once per
  // 32-MFMA phase in the attention kernel; iters is a multiple of 4
  constexpr int kTrip = 32;
  for (int it = 0; it < iters; it += kTrip / kAcc) {
#pragma unroll
    for (int n = 0; n < kTrip; ++n) {
      const bf16x8 a = ring[n % kRing];
      ring[n % kRing] = read(it * kAcc + n + kRing);
      acc[n % kAcc] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[n % kAcc], 0, 0, 0);
    }
#pragma unroll
    for (int n = 0; n < kTrip; ++n) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
  }
  float s = 0.0f;
  for (int n = 0; n < kAcc; ++n)
    for (int v = 0; v < 16; ++v) s += acc[n][v];
  out[(size_t)blockIdx.x * THREADS + t] = s;
}

// An LDS-fed MFMA stream (waves 0-3, one per SIMD: one ds_read_b128 A operand
// per MFMA, four reads in flight, pseudo-random operands) beside a VALU stream
// like a softmax (waves 4-7: FMA and exp2 over 64 values per lane, viters
// rounds), in one workgroup per CU. MODE bit 0: the MFMA waves run; bit 1:
// the VALU waves run. The time of both together against each alone bounds what
// a kernel that must do both on the same SIMDs can reach.
template <int MODE>
__global__ void __launch_bounds__(512) coexec_kernel(int iters, int viters, float* out) {
  extern __shared__ uint8_t lds[];
  const int t = threadIdx.x, w = t >> 6, lane = t & 63;
  const uint32_t gt = blockIdx.x * 512 + t;
  for (int i = t; i < kLdsSlots * 64; i += 512) {
    bf16x8 x;
    for (int e = 0; e < 8; ++e) x[e] = (__bf16)hash_value(5, (blockIdx.x * kLdsSlots * 64 + i) * 8 + e);
    *reinterpret_cast<bf16x8*>(lds + (size_t)i * 16) = x;
  }
  __syncthreads();
  float s = 0.0f;
  if (w < 4) {
    if (!(MODE & 1)) return;
    bf16x8 b;
    for (int e = 0; e < 8; ++e) b[e] = (__bf16)hash_value(2, gt * 8 + e);
    f32x16 acc[4];
    for (int n = 0; n < 4; ++n) acc[n] = f32x16{};
    auto rd = [&](int step) {
      return *reinterpret_cast<const bf16x8*>(lds + (step & (kLdsSlots - 1)) * 1024 + lane * 16);
    };
    bf16x8 ring[4];
    for (int n = 0; n < 4; ++n) ring[n] = rd(n);
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        const bf16x8 x = ring[n];
        ring[n] = rd(it * 4 + n + 4);
        acc[n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, b, acc[n], 0, 0, 0);
      }
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
    }
    for (int n = 0; n < 4; ++n)
      for (int v = 0; v < 16; ++v) s += acc[n][v];
  } else {
    if (!(MODE & 2)) return;
    float x[64];
    for (int e = 0; e < 64; ++e) x[e] = hash_value(3, gt * 64 + e);
    float m = 0.5f;
    for (int it = 0; it < viters; ++it) {
#pragma unroll
      for (int e = 0; e < 64; ++e) x[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[e], 0.25f, -m));
      m = x[0] * 0.001f;  // a fixed element: a varying index would put x in scratch memory
    }
    for (int e = 0; e < 64; ++e) s += x[e];
  }
  out[gt] = s;
}

// One wave per SIMD, register operands, NACC independent accumulator chains
// (8 MFMAs per loop trip): how many chains one wave needs to keep the matrix
// unit busy.
template <int NACC>
__global__ void __launch_bounds__(256) mfma_bf16_chains(int iters, float* out) {
  extern __shared__ uint8_t lds_pad[];
  (void)lds_pad;
  const int t = threadIdx.x;
  bf16x8 a, b;
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(float)((t + e) & 7);
    b[e] = (__bf16)(float)((t * 3 + e) & 7);
  }
  f32x16 acc[NACC];
  for (int n = 0; n < NACC; ++n) acc[n] = f32x16{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j % NACC] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j % NACC], 0, 0, 0);
  }
  float s = 0.0f;
  for (int n = 0; n < NACC; ++n)
    for (int v = 0; v < 16; ++v) s += acc[n][v];
  out[(size_t)blockIdx.x * 256 + t] = s;
}

template <int THREADS>
__global__ void __launch_bounds__(THREADS) mfma_f32_reg(int iters, float* out) {
  extern __shared__ uint8_t lds_pad[];
  (void)lds_pad;
  const int t = threadIdx.x;
  const float a = (float)(t & 7), b = (float)((t * 3) & 7);
  f32x16 acc[kAcc];
  for (int n = 0; n < kAcc; ++n) acc[n] = f32x16{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int n = 0; n < kAcc; ++n) acc[n] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, acc[n], 0, 0, 0);
  }
  float s = 0.0f;
  for (int n = 0; n < kAcc; ++n)
    for (int v = 0; v < 16; ++v) s += acc[n][v];
  out[(size_t)blockIdx.x * THREADS + t] = s;
}

struct Timer {
  hipEvent_t e0, e1;
  Timer() {
    CHECK(hipEventCreate(&e0));
    CHECK(hipEventCreate(&e1));
  }
  ~Timer() {
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
  }
};

// Best time (ms) of `reps` launches of `launch`, after one untimed launch.
template <class F>
static float best_ms(F launch, int reps) {
  Timer tm;
  launch();
  CHECK(hipGetLastError());
  CHECK(hipDeviceSynchronize());
  float best = 1e30f;
  for (int r = 0; r < reps; ++r) {
    CHECK(hipEventRecord(tm.e0));
    launch();
    CHECK(hipEventRecord(tm.e1));
    CHECK(hipEventSynchronize(tm.e1));
    float ms = 0.0f;
    CHECK(hipEventElapsedTime(&ms, tm.e0, tm.e1));
    if (ms < best) best = ms;
  }
  CHECK(hipGetLastError());
  return best;
}

struct Summary {
  double bf16_reg_1w = 0, bf16_reg_2w = 0, bf16_lds_2w = 0, f32_reg_2w = 0;
  double bf16_reg_2w_rand = 0, bf16_lds_2w_rand = 0, bf16_lds_1w_rand = 0, bf16_lds_valu = 0;
  double copy_GBps = 0, read_GBps = 0;
  double cache_stream_GBps = 0, cache_walk_GBps = 0;
  int ncu = 0, clock_khz = 0;
};

static void run_mfma(Summary& s) {
  const int ncu = s.ncu;
  const int grid = ncu * 4;
  const int iters = 4096;
  float* out = nullptr;
  CHECK(hipMalloc(&out, (size_t)grid * 512 * sizeof(float)));
  CHECK(hipFuncSetAttribute(reinterpret_cast<const void*>(&mfma_bf16_reg<256, false>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes));
  CHECK(hipFuncSetAttribute(reinterpret_cast<const void*>(&mfma_bf16_reg<512, false>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes));
  CHECK(hipFuncSetAttribute(reinterpret_cast<const void*>(&mfma_bf16_reg<512, true>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes));
  CHECK(hipFuncSetAttribute(reinterpret_cast<const void*>(&mfma_bf16_lds<512, false>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes));
  CHECK(hipFuncSetAttribute(reinterpret_cast<const void*>(&mfma_bf16_lds<256, true>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes));
  CHECK(hipFuncSetAttribute(reinterpret_cast<const void*>(&mfma_bf16_lds<512, true>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes));
  CHECK(hipFuncSetAttribute(reinterpret_cast<const void*>(&mfma_f32_reg<512>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes));
  const double f_bf16 = 32.0 * 32 * 16 * 2, f_f32 = 32.0 * 32 * 2 * 2;  // FLOPs per MFMA per wave
  auto rate = [&](double flop_per_mfma, int threads, float ms) {
    return flop_per_mfma * kAcc * iters * (double)grid * (threads / 64) / (ms * 1e-3) / 1e12;
  };
  // about 70 ms of MFMA work first, so that the first timed probe does not see the clock still rising
  (void)best_ms([&] { mfma_bf16_reg<512, false><<<grid, 512, kLdsBytes>>>(iters, out); }, 20);
  float ms = best_ms([&] { mfma_bf16_reg<256, false><<<grid, 256, kLdsBytes>>>(iters, out); }, 5);
  s.bf16_reg_1w = rate(f_bf16, 256, ms);
  printf("{\"probe\": \"mfma_bf16_32x32x16\", \"feed\": \"registers\", \"waves_per_simd\": 1, \"TFLOPs\": %.1f}\n",
         s.bf16_reg_1w);
  ms = best_ms([&] { mfma_bf16_reg<512, false><<<grid, 512, kLdsBytes>>>(iters, out); }, 5);
  s.bf16_reg_2w = rate(f_bf16, 512, ms);
  printf("{\"probe\": \"mfma_bf16_32x32x16\", \"feed\": \"registers\", \"waves_per_simd\": 2, \"TFLOPs\": %.1f}\n",
         s.bf16_reg_2w);
  ms = best_ms([&] { mfma_bf16_reg<512, true><<<grid, 512, kLdsBytes>>>(iters, out); }, 5);
  s.bf16_reg_2w_rand = rate(f_bf16, 512, ms);
  printf("{\"probe\": \"mfma_bf16_32x32x16\", \"feed\": \"registers, pseudo-random operands\", "
         "\"waves_per_simd\": 2, \"TFLOPs\": %.1f}\n",
         s.bf16_reg_2w_rand);
  ms = best_ms([&] { mfma_bf16_lds<512, false><<<grid, 512, kLdsBytes>>>(iters, out); }, 5);
  s.bf16_lds_2w = rate(f_bf16, 512, ms);
  printf("{\"probe\": \"mfma_bf16_32x32x16\", \"feed\": \"one ds_read_b128 A operand per MFMA\", "
         "\"waves_per_simd\": 2, \"TFLOPs\": %.1f}\n",
         s.bf16_lds_2w);
  ms = best_ms([&] { mfma_bf16_lds<512, true><<<grid, 512, kLdsBytes>>>(iters, out); }, 5);
  s.bf16_lds_2w_rand = rate(f_bf16, 512, ms);
  printf("{\"probe\": \"mfma_bf16_32x32x16\", \"feed\": \"one ds_read_b128 A operand per MFMA, pseudo-random "
         "operands\", \"waves_per_simd\": 2, \"TFLOPs\": %.1f}\n",
         s.bf16_lds_2w_rand);
  // the same stream from one wave per SIMD (the feed of each MFMA half-step of the ping-pong attention)
  ms = best_ms([&] { mfma_bf16_lds<256, true><<<grid, 256, kLdsBytes>>>(iters, out); }, 5);
  s.bf16_lds_1w_rand = rate(f_bf16, 256, ms);
  printf("{\"probe\": \"mfma_bf16_32x32x16\", \"feed\": \"one ds_read_b128 A operand per MFMA, pseudo-random "
         "operands\", \"waves_per_simd\": 1, \"TFLOPs\": %.1f}\n",
         s.bf16_lds_1w_rand);
  ms = best_ms([&] { mfma_f32_reg<512><<<grid, 512, kLdsBytes>>>(iters / 2, out); }, 5);
  s.f32_reg_2w = f_f32 * kAcc * (iters / 2) * (double)grid * 8 / (ms * 1e-3) / 1e12;
  printf("{\"probe\": \"mfma_f32_32x32x2\", \"feed\": \"registers\", \"waves_per_simd\": 2, \"TFLOPs\": %.1f}\n",
         s.f32_reg_2w);
  CHECK(hipFree(out));
}

// ------------------------------------------------------------------ HBM

__global__ void __launch_bounds__(256) copy16(const u32x4* __restrict__ src, u32x4* __restrict__ dst, size_t n16) {
  const size_t stride = (size_t)gridDim.x * 256;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += stride) dst[i] = src[i];
}

__global__ void __launch_bounds__(256) stream_read(const u32x4* __restrict__ p, size_t n16, uint32_t* out) {
  const size_t tid = (size_t)blockIdx.x * 256 + threadIdx.x, stride = (size_t)gridDim.x * 256;
  u32x4 acc = {0, 0, 0, 0};
  size_t i = tid;
  for (; i + 3 * stride < n16; i += 4 * stride) acc ^= p[i] ^ p[i + stride] ^ p[i + 2 * stride] ^ p[i + 3 * stride];
  for (; i < n16; i += stride) acc ^= p[i];
  out[tid] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

// workgroup (g, sp) reads key blocks [sp*cb, sp*cb + cb) of KV head g from K
// and V ([L][H][128] bf16: 128 keys of 256 bytes per block, H*256 bytes apart)
__global__ void __launch_bounds__(256) block_walk_read(const u32x4* __restrict__ k, const u32x4* __restrict__ v,
                                                       int H, int nsplit, int cb, uint32_t* out) {
  const int g = blockIdx.x / nsplit, sp = blockIdx.x % nsplit, t = threadIdx.x;
  u32x4 acc = {0, 0, 0, 0};
  for (int jj = 0; jj < cb; ++jj) {
    const int j = sp * cb + jj;
    u32x4 x[16];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = (t + 256 * i) / 16, ch = t % 16;
      const size_t off = ((size_t)(j * 128 + row) * H + g) * 16 + ch;  // 16-byte units
      x[i] = k[off];
      x[8 + i] = v[off];
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) acc ^= x[i];
  }
  out[(size_t)blockIdx.x * 256 + t] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

static void run_hbm(Summary& s) {
  const size_t bytes = (size_t)1 << 30;
  u32x4 *a = nullptr, *b = nullptr;
  uint32_t* out = nullptr;
  const int grid = s.ncu * 16;
  CHECK(hipMalloc(&a, bytes));
  CHECK(hipMalloc(&b, bytes));
  CHECK(hipMalloc(&out, (size_t)grid * 256 * sizeof(uint32_t)));
  CHECK(hipMemset(a, 1, bytes));
  CHECK(hipMemset(b, 2, bytes));
  float ms = best_ms([&] { copy16<<<grid, 256>>>(a, b, bytes / 16); }, 10);
  s.copy_GBps = 2.0 * bytes / (ms * 1e-3) / 1e9;
  printf("{\"probe\": \"hbm_copy\", \"bytes_moved\": %zu, \"us\": %.1f, \"GBps\": %.1f}\n", 2 * bytes, ms * 1e3,
         s.copy_GBps);
  ms = best_ms([&] { stream_read<<<grid, 256>>>(a, bytes / 16, out); }, 10);
  s.read_GBps = (double)bytes / (ms * 1e-3) / 1e9;
  printf("{\"probe\": \"hbm_read\", \"bytes\": %zu, \"us\": %.1f, \"GBps\": %.1f}\n", bytes, ms * 1e3, s.read_GBps);
  CHECK(hipFree(a));
  CHECK(hipFree(b));
  CHECK(hipFree(out));
}

static void run_cache(Summary& s, int L, int H) {
  const size_t bytes = (size_t)L * H * 256;
  const int max_grid = 8192 * 8;
  u32x4 *k = nullptr, *v = nullptr;
  uint32_t* out = nullptr;
  CHECK(hipMalloc(&k, bytes));
  CHECK(hipMalloc(&v, bytes));
  CHECK(hipMalloc(&out, (size_t)max_grid * 256 * sizeof(uint32_t)));
  CHECK(hipMemset(k, 1, bytes));
  CHECK(hipMemset(v, 2, bytes));
  for (int grid : {1024, 2048, 4096}) {
    const float ms = best_ms([&] {
      stream_read<<<grid, 256>>>(k, bytes / 16, out);
      stream_read<<<grid, 256>>>(v, bytes / 16, out);
    }, 10);
    const double gbps = 2.0 * bytes / (ms * 1e-3) / 1e9;
    if (gbps > s.cache_stream_GBps) s.cache_stream_GBps = gbps;
    printf("{\"probe\": \"cache_stream_read\", \"L\": %d, \"Hkv\": %d, \"grid\": %d, \"bytes\": %zu, \"us\": %.2f, "
           "\"GBps\": %.1f}\n", L, H, grid, 2 * bytes, ms * 1e3, gbps);
  }
  const int nb = L / 128;
  for (int cb : {4, 8, 16, 32}) {
    if (nb % cb) continue;
    const int nsplit = nb / cb, grid = H * nsplit;
    if (grid > max_grid) continue;
    const float ms = best_ms([&] { block_walk_read<<<grid, 256>>>(k, v, H, nsplit, cb, out); }, 10);
    const double gbps = 2.0 * bytes / (ms * 1e-3) / 1e9;
    if (gbps > s.cache_walk_GBps) s.cache_walk_GBps = gbps;
    printf("{\"probe\": \"cache_block_walk_read\", \"L\": %d, \"Hkv\": %d, \"blocks_per_workgroup\": %d, "
           "\"grid\": %d, \"bytes\": %zu, \"us\": %.2f, \"GBps\": %.1f}\n", L, H, cb, grid, 2 * bytes, ms * 1e3, gbps);
  }
  CHECK(hipFree(k));
  CHECK(hipFree(v));
  CHECK(hipFree(out));
}

template <int NACC>
static void run_chains_one(int ncu, float* out) {
  const int grid = ncu * 4, iters = 4096;
  CHECK(hipFuncSetAttribute(reinterpret_cast<const void*>(&mfma_bf16_chains<NACC>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes));
  const float ms = best_ms([&] { mfma_bf16_chains<NACC><<<grid, 256, kLdsBytes>>>(iters, out); }, 5);
  const double tf = 32.0 * 32 * 16 * 2 * 8 * iters * (double)grid * 4 / (ms * 1e-3) / 1e12;
  printf("{\"probe\": \"mfma_bf16_32x32x16\", \"feed\": \"registers\", \"waves_per_simd\": 1, \"chains\": %d, "
         "\"TFLOPs\": %.1f}\n", NACC, tf);
}

template <int MODE>
static float coexec_ms(int ncu, float* out, int iters, int viters) {
  CHECK(hipFuncSetAttribute(reinterpret_cast<const void*>(&coexec_kernel<MODE>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes));
  return best_ms([&] { coexec_kernel<MODE><<<ncu * 4, 512, kLdsBytes>>>(iters, viters, out); }, 5);
}

static double run_coexec(int ncu, int viters) {
  const int iters = 8192;  // 32,768 MFMAs per MFMA wave
  float* out = nullptr;
  CHECK(hipMalloc(&out, (size_t)ncu * 4 * 512 * sizeof(float)));
  (void)coexec_ms<1>(ncu, out, iters, viters);  // warm-up
  const float m = coexec_ms<1>(ncu, out, iters, viters);
  const float v = coexec_ms<2>(ncu, out, iters, viters);
  const float b = coexec_ms<3>(ncu, out, iters, viters);
  const double fl = (double)ncu * 4 * 4 * iters * 4 * 32768.0;
  printf("{\"probe\": \"coexec\", \"valu_rounds\": %d, \"mfma_alone_ms\": %.3f, \"valu_alone_ms\": %.3f, "
         "\"both_ms\": %.3f, \"valu_to_mfma_time\": %.2f, \"mfma_alone_TFLOPs\": %.1f, \"both_TFLOPs\": %.1f}\n",
         viters, m, v, b, v / m, fl / (m * 1e-3) / 1e12, fl / (b * 1e-3) / 1e12);
  CHECK(hipFree(out));
  return fl / (b * 1e-3) / 1e12;
}

// VALU rounds of the co-execution probe that match the ping-pong attention's mix:
// per 64 MFMAs the attention issues about 217 other VALU instructions, 64 of them
// exp2 (instruction counters of the 128K layer), i.e. 281 FMA-equivalents with
// exp2 at half rate; 750 rounds give the probe's MFMA waves 93.75 exp2 and 93.75
// FMA per 64 MFMAs, 281.25 FMA-equivalents.
constexpr int kAttnValuRounds = 750;

static void run_chains(int ncu) {
  float* out = nullptr;
  CHECK(hipMalloc(&out, (size_t)ncu * 4 * 256 * sizeof(float)));
  run_chains_one<8>(ncu, out);  // also brings the clock up before the others
  run_chains_one<1>(ncu, out);
  run_chains_one<2>(ncu, out);
  run_chains_one<4>(ncu, out);
  run_chains_one<8>(ncu, out);
  CHECK(hipFree(out));
}

int main(int argc, char** argv) {
  const char* what = argc > 1 ? argv[1] : "all";
  const int L = argc > 2 ? atoi(argv[2]) : 131072, H = argc > 3 ? atoi(argv[3]) : 8;
  const bool all = !strcmp(what, "all");
  if (!all && strcmp(what, "mfma") && strcmp(what, "hbm") && strcmp(what, "cache") && strcmp(what, "chains") &&
      strcmp(what, "coexec")) {
    fprintf(stderr, "usage: peak [all|mfma|hbm|cache|chains|coexec] [L] [Hkv]   (coexec: [valu rounds])\n");
    return 2;
  }
  if (!strcmp(what, "coexec")) {
    int dev0 = 0, ncu0 = 0;
    CHECK(hipGetDevice(&dev0));
    CHECK(hipDeviceGetAttribute(&ncu0, hipDeviceAttributeMultiprocessorCount, dev0));
    const int vr = argc > 2 ? atoi(argv[2]) : 170;
    if (vr < 1 || vr > 10000) {
      fprintf(stderr, "peak coexec: valu rounds in [1, 10000]\n");
      return 2;
    }
    run_coexec(ncu0, vr);
    return 0;
  }
  if (L < 128 || L % 128 != 0 || H < 1 || (long long)L * H > (1ll << 26)) {
    fprintf(stderr, "peak: L must be a positive multiple of 128 and L*Hkv <= 2^26\n");
    return 2;
  }
  Summary s;
  int dev = 0;
  CHECK(hipGetDevice(&dev));
  CHECK(hipDeviceGetAttribute(&s.ncu, hipDeviceAttributeMultiprocessorCount, dev));
  CHECK(hipDeviceGetAttribute(&s.clock_khz, hipDeviceAttributeClockRate, dev));
  if (all || !strcmp(what, "mfma")) {
    run_mfma(s);
    s.bf16_lds_valu = run_coexec(s.ncu, kAttnValuRounds);
  }
  if (all || !strcmp(what, "hbm")) run_hbm(s);
  if (!strcmp(what, "cache")) run_cache(s, L, H);
  if (!strcmp(what, "chains")) run_chains(s.ncu);
  printf("{\"summary\": {\"cus\": %d, \"max_clock_mhz\": %d, \"mfma_bf16_reg_1w_TFLOPs\": %.1f, "
         "\"mfma_bf16_reg_2w_TFLOPs\": %.1f, \"mfma_bf16_lds_2w_TFLOPs\": %.1f, "
         "\"mfma_bf16_reg_2w_random_TFLOPs\": %.1f, \"mfma_bf16_lds_2w_random_TFLOPs\": %.1f, "
         "\"mfma_bf16_lds_1w_random_TFLOPs\": %.1f, \"mfma_bf16_lds_random_with_softmax_valu_TFLOPs\": %.1f, "
         "\"mfma_f32_reg_2w_TFLOPs\": %.2f, "
         "\"hbm_copy_GBps\": %.1f, \"hbm_read_GBps\": %.1f, \"cache_stream_GBps\": %.1f, "
         "\"cache_walk_GBps\": %.1f}}\n",
         s.ncu, s.clock_khz / 1000, s.bf16_reg_1w, s.bf16_reg_2w, s.bf16_lds_2w, s.bf16_reg_2w_rand,
         s.bf16_lds_2w_rand, s.bf16_lds_1w_rand, s.bf16_lds_valu, s.f32_reg_2w, s.copy_GBps,
         s.read_GBps, s.cache_stream_GBps, s.cache_walk_GBps);
  return 0;
}
