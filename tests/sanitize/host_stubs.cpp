// CPU stand-ins for the kernel launches of the C-ABI library, so that its
// host runtime (argument checks, workspace layout, the varlen and decode
// sequencing in rr_host.cpp) can be built with g++ under AddressSanitizer and
// UndefinedBehaviorSanitizer and driven without a GPU (tests/sanitize/
// host_driver.cpp). Every launch records its call and checks that each
// buffer the host carved out of the caller's workspace lies inside it.
#include <stdio.h>
#include <stdlib.h>

#include "rr_kernels.h"
#include "stub_state.h"

StubState g_stub;

static void in_ws(const void* p, size_t bytes, const char* what) {
  const char* b = static_cast<const char*>(g_stub.ws);
  const char* q = static_cast<const char*>(p);
  if (!b || q < b || q + bytes > b + g_stub.ws_bytes) {
    fprintf(stderr, "workspace range violated: %s (%zu bytes at offset %td of %zu)\n", what, bytes, q - b,
            g_stub.ws_bytes);
    abort();
  }
}

static size_t esz(const rr::Geometry& g) { return g.bf16 ? 2 : 4; }

namespace rr {

hipError_t launch_pool_keys(const Geometry& g, const void*, void* kbar, bool, hipStream_t) {
  ++g_stub.calls;
  if (g_stub.ws) {
    const char* b = static_cast<const char*>(g_stub.ws);
    const char* q = static_cast<const char*>(kbar);
    if (q >= b && q < b + g_stub.ws_bytes) in_ws(kbar, (size_t)g.ns * g.Hkv * g.d * esz(g), "pooled keys");
  }
  return g_stub.fail_launch ? hipErrorLaunchFailure : hipSuccess;
}

hipError_t launch_search(const Geometry& g, const void*, const void* kbar, float* mass, hipStream_t) {
  ++g_stub.calls;
  in_ws(kbar, (size_t)g.ns * g.Hkv * g.d * esz(g), "pooled keys (search)");
  if (!g_stub.user_mass) in_ws(mass, (size_t)g.Hq * g.nb * g.nb * sizeof(float), "block masses");
  return hipSuccess;
}

hipError_t launch_select(const Geometry& g, const float* mass, int, int32_t*, int32_t*, const float*, hipStream_t) {
  ++g_stub.calls;
  if (!g_stub.user_mass) in_ws(mass, (size_t)g.Hq * g.nb * g.nb * sizeof(float), "block masses (select)");
  return hipSuccess;
}

void search_batch_counts(const Geometry& g, int nb, int ns, int* pool_threads, int* search_blocks, int* rows) {
  const int hpc = g.G < 64 / g.r ? g.G : 64 / g.r;
  *pool_threads = ns * (g.Hkv * g.d * (int)esz(g) / 16);
  *search_blocks = (nb - 1) * g.Hkv * ((g.G + hpc - 1) / hpc);
  *rows = g.Hq * nb;
}

// The batched search launches: every sequence's pooled keys and masses must lie
// inside the workspace, the prefix counts must match the per-sequence counts.
static void check_search_batch(const Geometry& g, const SearchBatch& sb, const void* kbar, const float* mass) {
  if (sb.n < 1 || sb.n > kMaxSeqPerLaunch) abort();
  for (int m = 0; m < sb.n; ++m) {
    int np, nbk, nr;
    search_batch_counts(g, sb.nb[m], sb.ns[m], &np, &nbk, &nr);
    if (sb.pool_off[m + 1] - sb.pool_off[m] != np || sb.blk_off[m + 1] - sb.blk_off[m] != nbk ||
        sb.row_off[m + 1] - sb.row_off[m] != nr)
      abort();
    in_ws(static_cast<const char*>(kbar) + sb.kbar_off[m] * esz(g), (size_t)sb.ns[m] * g.Hkv * g.d * esz(g),
          "pooled keys (batched)");
    in_ws(mass + sb.mass_off[m], (size_t)g.Hq * sb.nb[m] * sb.nb[m] * sizeof(float), "block masses (batched)");
  }
  ++g_stub.batched_searches;
}

hipError_t launch_pool_keys_batched(const Geometry& g, const SearchBatch& sb, const void*, void* kbar, hipStream_t) {
  ++g_stub.calls;
  check_search_batch(g, sb, kbar, static_cast<const float*>(g_stub.ws));
  return hipSuccess;
}

hipError_t launch_search_batched(const Geometry& g, const SearchBatch& sb, const void*, const void* kbar,
                                 float* mass, hipStream_t) {
  ++g_stub.calls;
  check_search_batch(g, sb, kbar, mass);
  return hipSuccess;
}

hipError_t launch_select_batched(const Geometry& g, const SearchBatch& sb, const float* mass, int32_t*, int32_t*,
                                 hipStream_t) {
  ++g_stub.calls;
  check_search_batch(g, sb, g_stub.ws, mass);
  return hipSuccess;
}

hipError_t launch_union_lists(const Geometry&, const int32_t*, const int32_t*, int32_t*, int32_t*, hipStream_t) {
  ++g_stub.calls;
  return hipSuccess;
}

bool attn_pair_shape(const Geometry& g) { return g.bf16 && g.B == 128; }

hipError_t attn_cu_count(hipStream_t, int* ncu) {
  *ncu = 256;
  return hipSuccess;
}

int attn_items(const Geometry& g) {
  const int G = g.Hq / g.Hkv;
  return G % 2 ? g.Hkv * ((g.nb + 1) / 2) * G : g.Hkv * g.nb * (G / 2);
}

hipError_t launch_transpose_v(const Geometry& g, const void*, void* vt, int32_t* queues, hipStream_t) {
  ++g_stub.calls;
  in_ws(vt, (size_t)g.nb * g.B * g.Hkv * g.d * esz(g), "V re-layout");
  in_ws(queues, kAttnQueues * sizeof(int32_t), "work-queue counters");
  return hipSuccess;
}

hipError_t launch_attention(const Geometry& g, const void*, const void*, const void*, const void* vt,
                            int32_t* queues, const int32_t*, const int32_t*, void*, hipStream_t) {
  ++g_stub.calls;
  ++g_stub.single_launches;
  if (g.bf16) {
    in_ws(vt, (size_t)g.nb * g.B * g.Hkv * g.d * esz(g), "V re-layout (attention)");
    in_ws(queues, kAttnQueues * sizeof(int32_t), "work-queue counters (attention)");
  }
  return hipSuccess;
}

static void check_batch(const Geometry& g, const SeqBatch& sb, const void* vt, int32_t* queues, bool tiles) {
  if (!attn_pair_shape(g) || sb.n < 1 || sb.n > kMaxSeqPerLaunch) abort();
  in_ws(queues, kAttnQueues * sizeof(int32_t), "work-queue counters (batched)");
  for (int m = 0; m < sb.n; ++m) {  // ranges ascending and covering each sequence; longest first
    Geometry gs = g;
    gs.L = sb.L[m];
    gs.nb = (sb.L[m] + g.B - 1) / g.B;
    if (sb.nb[m] != gs.nb || sb.item_off[m] % 16 || sb.item_off[m + 1] - sb.item_off[m] < attn_items(gs)) abort();
    if (tiles && sb.tile_off[m + 1] - sb.tile_off[m] != gs.Hkv * gs.nb) abort();
    if (m > 0 && sb.L[m] > sb.L[m - 1]) abort();
    in_ws(static_cast<const char*>(vt) + sb.vt_off[m], (size_t)gs.nb * gs.B * gs.Hkv * gs.d * esz(gs),
          "V re-layout of one sequence (batched)");
  }
}

hipError_t launch_transpose_v_batched(const Geometry& g, const SeqBatch& sb, const void*, void* vt, int32_t* queues,
                                      hipStream_t) {
  ++g_stub.calls;
  check_batch(g, sb, vt, queues, true);
  return hipSuccess;
}

hipError_t launch_attention_batched(const Geometry& g, const SeqBatch& sb, const void*, const void*,
                                    const void* vt, int32_t* queues, const int32_t*, const int32_t*, void*,
                                    hipStream_t) {
  ++g_stub.calls;
  check_batch(g, sb, vt, queues, false);
  g_stub.batched_items += sb.item_off[sb.n];
  ++g_stub.batched_launches;
  return hipSuccess;
}

hipError_t launch_recall(const Geometry&, const void*, const void*, const int32_t*, const int32_t*, float*,
                         hipStream_t) {
  ++g_stub.calls;
  return hipSuccess;
}

// the decode split / chunk counts only size workspace parts here
bool decode_grouped(const Geometry& g) { return g.bf16 && g.G <= 8; }
int decode_splits(const Geometry& g) { return (g.nb + 15) / 16; }
int decode_chunks(const Geometry& g) { return (g.ns + 255) / 256; }

hipError_t launch_decode_scores(const Geometry& g, const void*, const void* kbar, float* bsum, float* zpart,
                                hipStream_t) {
  ++g_stub.calls;
  if (!g_stub.user_kbar) in_ws(kbar, (size_t)g.ns * g.Hkv * g.d * esz(g), "decode pooled keys");
  in_ws(bsum, (size_t)g.Hq * g.nb * sizeof(float), "decode block sums");
  in_ws(zpart, (size_t)g.Hq * decode_chunks(g) * 2 * sizeof(float), "decode chunk partials");
  return hipSuccess;
}

hipError_t launch_decode_select(const Geometry& g, const float* bsum, const float* zpart, float* mass, int32_t*,
                                int32_t*, uint8_t* sel, int nbp, hipStream_t) {
  ++g_stub.calls;
  in_ws(bsum, (size_t)g.Hq * g.nb * sizeof(float), "decode block sums (select)");
  in_ws(zpart, (size_t)g.Hq * decode_chunks(g) * 2 * sizeof(float), "decode chunk partials (select)");
  if (!g_stub.user_mass) in_ws(mass, (size_t)g.Hq * g.nb * sizeof(float), "decode masses");
  in_ws(sel, (size_t)g.Hq * nbp, "decode flags");
  if (nbp < g.nb) abort();
  return hipSuccess;
}

hipError_t launch_lists_to_flags(const Geometry& g, const int32_t*, const int32_t*, uint8_t* sel, int nbp,
                                 hipStream_t) {
  ++g_stub.calls;
  in_ws(sel, (size_t)g.Hq * nbp, "decode flags (lists)");
  return hipSuccess;
}

hipError_t launch_decode_attn(const Geometry& g, const void*, const void*, const void*, const int32_t*,
                              const int32_t*, const uint8_t* sel, int nbp, float* part, void*, hipStream_t) {
  ++g_stub.calls;
  in_ws(sel, (size_t)g.Hq * nbp, "decode flags (attention)");
  in_ws(part, (size_t)g.Hq * decode_splits(g) * (g.d + 2) * sizeof(float), "decode split partials");
  return hipSuccess;
}

// the library's own decode buffer: a host allocation here (never dereferenced)
hipError_t static_workspace(hipStream_t, void** ptr) {
  static void* buf = nullptr;
  if (!buf) buf = aligned_alloc(256, kStaticWorkspaceBytes);
  *ptr = buf;
  g_stub.ws = buf;
  g_stub.ws_bytes = kStaticWorkspaceBytes;
  return hipSuccess;
}

}  // namespace rr
