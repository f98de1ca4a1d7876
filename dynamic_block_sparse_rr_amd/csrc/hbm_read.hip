// Practical HBM read ceiling of the decode attention's access pattern, as a
// standalone program: reads a K and a V cache of [L][Hkv][128] bf16 (two
// buffers of L*Hkv*256 bytes) (1) as one grid-stride 16-byte load stream and
// (2) as the decode attention walks them: workgroup (KV head, run of blocks),
// 128 keys of 256 bytes per block, 2 KiB apart. Prints one JSON line per
// variant with the read rate in TB/s (HIP events over 20 repetitions).
// Usage: hbm_read [L] [Hkv]
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ void __launch_bounds__(256) stream_read(const u32x4* __restrict__ p, size_t n16, uint32_t* out) {
  const size_t tid = (size_t)blockIdx.x * 256 + threadIdx.x, stride = (size_t)gridDim.x * 256;
  u32x4 acc = {0, 0, 0, 0};
  size_t i = tid;
  for (; i + 3 * stride < n16; i += 4 * stride) acc ^= p[i] ^ p[i + stride] ^ p[i + 2 * stride] ^ p[i + 3 * stride];
  for (; i < n16; i += stride) acc ^= p[i];
  out[tid] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

// workgroup (g, sp) reads blocks [sp*cb, sp*cb + cb) of KV head g from K and V
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

static int check(hipError_t e, const char* what) {
  if (e != hipSuccess) {
    fprintf(stderr, "%s: %s\n", what, hipGetErrorString(e));
    return 1;
  }
  return 0;
}

int main(int argc, char** argv) {
  const int L = argc > 1 ? atoi(argv[1]) : 131072, H = argc > 2 ? atoi(argv[2]) : 8;
  if (L < 128 || L % 128 != 0 || H < 1 || (long long)L * H > (1ll << 26)) {
    fprintf(stderr, "hbm_read: L must be a positive multiple of 128 and L*Hkv <= 2^26\n");
    return 2;
  }
  const size_t bytes = (size_t)L * H * 256;
  const int max_grid = 8192;
  u32x4 *k = nullptr, *v = nullptr;
  uint32_t* out = nullptr;
  if (check(hipMalloc(&k, bytes), "hipMalloc") || check(hipMalloc(&v, bytes), "hipMalloc") ||
      check(hipMalloc(&out, (size_t)max_grid * 256 * 4 * 8), "hipMalloc"))
    return 1;
  if (check(hipMemset(k, 1, bytes), "hipMemset") || check(hipMemset(v, 2, bytes), "hipMemset")) return 1;
  hipEvent_t e0, e1;
  if (check(hipEventCreate(&e0), "event") || check(hipEventCreate(&e1), "event")) return 1;
  const int reps = 20;
  float ms = 0.0f;
  for (int grid : {1024, 2048, 4096}) {
    stream_read<<<grid, 256>>>(k, bytes / 16, out);
    (void)hipEventRecord(e0);
    for (int r = 0; r < reps; ++r) {
      stream_read<<<grid, 256>>>(k, bytes / 16, out);
      stream_read<<<grid, 256>>>(v, bytes / 16, out);
    }
    (void)hipEventRecord(e1);
    if (check(hipEventSynchronize(e1), "kernel")) return 1;
    (void)hipEventElapsedTime(&ms, e0, e1);
    printf("{\"probe\": \"stream_read\", \"grid\": %d, \"bytes\": %zu, \"us\": %.2f, \"TBps\": %.3f}\n", grid,
           2 * bytes, ms * 1e3 / reps, 2.0 * bytes * reps / (ms * 1e-3) / 1e12);
  }
  const int nb = L / 128;
  for (int cb : {4, 8, 16, 32}) {
    if (nb % cb) continue;
    const int nsplit = nb / cb, grid = H * nsplit;
    if (grid > max_grid * 8) continue;  // out holds max_grid * 8 workgroups
    block_walk_read<<<grid, 256>>>(k, v, H, nsplit, cb, out);
    (void)hipEventRecord(e0);
    for (int r = 0; r < reps; ++r) block_walk_read<<<grid, 256>>>(k, v, H, nsplit, cb, out);
    (void)hipEventRecord(e1);
    if (check(hipEventSynchronize(e1), "kernel")) return 1;
    (void)hipEventElapsedTime(&ms, e0, e1);
    printf("{\"probe\": \"block_walk_read\", \"blocks_per_workgroup\": %d, \"grid\": %d, \"bytes\": %zu, "
           "\"us\": %.2f, \"TBps\": %.3f}\n",
           cb, grid, 2 * bytes, ms * 1e3 / reps, 2.0 * bytes * reps / (ms * 1e-3) / 1e12);
  }
  (void)hipFree(k);
  (void)hipFree(v);
  (void)hipFree(out);
  return 0;
}
