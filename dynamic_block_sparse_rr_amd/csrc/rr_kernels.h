// Internal launch interface between the host runtime (rr_host.cpp) and the
// gfx950 kernels (search.hip, attn.hip, recall.hip, decode.hip). Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace rr {

// Geometry shared by the launches of one problem.
struct Geometry {
  int L, Hq, Hkv, d, S, B;
  int nb, ns, r, G;  // nb = ceil(L / B), ns = ceil(L / S): the last block and stride may be short
  int causal;
  int bf16;  // 1: bfloat16 tensors, 0: float32
  float tau;
};

// Stage 1 launches.
// chunk_major: kbar as [Hkv][d*esz/16][ns] 16-byte chunks (the search's layout), else [ns][Hkv][d]
hipError_t launch_pool_keys(const Geometry& g, const void* k, void* kbar, bool chunk_major, hipStream_t st);
// kbar in the chunk-major layout
hipError_t launch_search(const Geometry& g, const void* q, const void* kbar, float* mass,
                         hipStream_t st);
// tau_heads: optional device thresholds [Hq] in place of g.tau.
hipError_t launch_select(const Geometry& g, const float* mass, int zero_fill, int32_t* row_count,
                         int32_t* col_idx, const float* tau_heads, hipStream_t st);

// Variant: every head of a KV head gets the union of the group's selections.
hipError_t launch_union_lists(const Geometry& g, const int32_t* row_count, const int32_t* col_idx,
                              int32_t* out_count, int32_t* out_idx, hipStream_t st);

// Stage 2 launches. queues: kAttnQueues device counters of the bf16
// attention's work queues (one per XCD); launch_transpose_v zeroes them, so
// the two run in this order on one stream, one pair per call at a time.
constexpr int kAttnQueues = 8;
hipError_t launch_transpose_v(const Geometry& g, const void* v, void* vt, int32_t* queues, hipStream_t st);
hipError_t launch_attention(const Geometry& g, const void* q, const void* k, const void* v,
                            const void* vt, int32_t* queues, const int32_t* row_count,
                            const int32_t* col_idx, void* out, hipStream_t st);

// Selection quality: full-attention softmax mass inside the selected blocks.
hipError_t launch_recall(const Geometry& g, const void* q, const void* k, const int32_t* row_count,
                         const int32_t* col_idx, float* recall, hipStream_t st);

// Decode step (one new query per head against the cache).
constexpr int kDecodeSplit = 16;  // list entries per split-K workgroup of the decode attention
bool decode_grouped(const Geometry& g);  // bf16 with G <= 8: one workgroup serves a KV head's G query heads
int decode_splits(const Geometry& g);     // split-K partials per head
int decode_chunks(const Geometry& g);  // 256-stride chunks of the decode scores
// per 256-stride chunk (max, exp-sum) [Hq][nchunk][2] and block sums bsum [Hq][nb] relative to the chunk max
hipError_t launch_decode_scores(const Geometry& g, const void* q, const void* kbar, float* bsum, float* zpart,
                                hipStream_t st);
// block masses [Hq][nb] from the chunk partials, lists, and selection flags sel [Hq][nbp] (nbp >= nb)
hipError_t launch_decode_select(const Geometry& g, const float* bsum, const float* zpart, float* mass,
                                int32_t* row_count, int32_t* col_idx, uint8_t* sel, int nbp, hipStream_t st);
hipError_t launch_lists_to_flags(const Geometry& g, const int32_t* row_count, const int32_t* col_idx, uint8_t* sel,
                                 int nbp, hipStream_t st);
hipError_t launch_decode_attn(const Geometry& g, const void* q, const void* k, const void* v,
                              const int32_t* row_count, const int32_t* col_idx, const uint8_t* sel, int nbp,
                              float* part, void* out, hipStream_t st);

// Kernel-side limits checked by the host before any launch.
constexpr int kMaxSelectBlocks = 8192;  // LDS sort capacity of the select kernel (nb): 12 B per key

}  // namespace rr
