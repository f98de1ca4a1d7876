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

constexpr int kMaxSeqPerLaunch = 32;

// The search of a packed batch of sequences (up to kMaxSeqPerLaunch) in one
// launch per kernel: per sequence its first token, length, block and stride
// counts, the offsets of its pooled keys (elements, chunk-major layout), its
// block masses (floats) and its block lists (entries), and prefix counts of
// the work of each launch (pool: threads, search: workgroups, select: rows;
// entry n is the total). g describes the sequences but for L, nb and ns.
struct SearchBatch {
  int n;
  int pool_off[kMaxSeqPerLaunch + 1];
  int blk_off[kMaxSeqPerLaunch + 1];
  int row_off[kMaxSeqPerLaunch + 1];
  int tok_off[kMaxSeqPerLaunch];
  int L[kMaxSeqPerLaunch];
  int nb[kMaxSeqPerLaunch];
  int ns[kMaxSeqPerLaunch];
  long long kbar_off[kMaxSeqPerLaunch];
  long long mass_off[kMaxSeqPerLaunch];
  long long rc_off[kMaxSeqPerLaunch];
  long long ci_off[kMaxSeqPerLaunch];
};
void search_batch_counts(const Geometry& g, int nb, int ns, int* pool_threads, int* search_blocks, int* rows);
hipError_t launch_pool_keys_batched(const Geometry& g, const SearchBatch& sb, const void* k, void* kbar,
                                    hipStream_t st);
hipError_t launch_search_batched(const Geometry& g, const SearchBatch& sb, const void* q, const void* kbar,
                                 float* mass, hipStream_t st);
hipError_t launch_select_batched(const Geometry& g, const SearchBatch& sb, const float* mass, int32_t* row_count,
                                 int32_t* col_idx, hipStream_t st);

// Variant: every head of a KV head gets the union of the group's selections.
hipError_t launch_union_lists(const Geometry& g, const int32_t* row_count, const int32_t* col_idx,
                              int32_t* out_count, int32_t* out_idx, hipStream_t st);

// A packed batch of sequences covered by one launch of the head-pair
// attention and one of its V re-layout: per sequence its first token, length,
// block count, the entry offsets of its block lists, the byte offset of its V
// re-layout, the first of its work items (multiples of 16; item_off[n] is the
// total) and the first of its V tiles (tile_off[n] is the total).
struct SeqBatch {
  int n;
  int item_off[kMaxSeqPerLaunch + 1];
  int tile_off[kMaxSeqPerLaunch + 1];
  int tok_off[kMaxSeqPerLaunch];
  int L[kMaxSeqPerLaunch];
  int nb[kMaxSeqPerLaunch];
  long long rc_off[kMaxSeqPerLaunch];
  long long ci_off[kMaxSeqPerLaunch];
  long long vt_off[kMaxSeqPerLaunch];
};

// Stage 2 launches. queues: kAttnQueues device counters of the bf16
// attention's work queues (one per XCD); launch_transpose_v zeroes them, so
// the two run in this order on one stream, one pair per call at a time.
constexpr int kAttnQueues = 8;
bool attn_pair_shape(const Geometry& g);  // bf16 with B = 128: the head-pair kernel
int attn_items(const Geometry& g);        // work items of one sequence's head-pair launch
hipError_t attn_cu_count(hipStream_t st, int* ncu);  // CUs of the stream's device (looked up once per device)
// A sequence of a packed batch whose head-pair launch holds at least this
// many work items per CU gets a launch of its own (it fills the GPU alone and
// can balance its XCDs through the work queues); the shorter ones share
// batched launches, where one launch fills the GPU for all of them.
constexpr int kVarlenSoloItemsPerCU = 8;
hipError_t launch_transpose_v(const Geometry& g, const void* v, void* vt, int32_t* queues, hipStream_t st);
hipError_t launch_attention(const Geometry& g, const void* q, const void* k, const void* v,
                            const void* vt, int32_t* queues, const int32_t* row_count,
                            const int32_t* col_idx, void* out, hipStream_t st);
// The batched head-pair forms: g describes the sequences but for L and nb
// (taken from sb); q, k, v, out are the packed tensors, row_count / col_idx
// the packed lists, vt the base of the sequences' re-layouts.
hipError_t launch_transpose_v_batched(const Geometry& g, const SeqBatch& sb, const void* v, void* vt,
                                      int32_t* queues, hipStream_t st);
hipError_t launch_attention_batched(const Geometry& g, const SeqBatch& sb, const void* q, const void* k,
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

// The device buffer of rr_decode_noalloc (static_ws.hip): kStaticWorkspaceBytes
// per GPU, its address on the device that runs `st` (looked up once per device).
constexpr size_t kStaticWorkspaceBytes = 32u << 20;
hipError_t static_workspace(hipStream_t st, void** ptr);

// Kernel-side limits checked by the host before any launch.
constexpr int kMaxSelectBlocks = 8192;  // block rows the select kernel stages in LDS: 4 rows x nb floats per workgroup

}  // namespace rr
