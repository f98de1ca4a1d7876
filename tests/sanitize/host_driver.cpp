// Drives every C-ABI entry point of the library's host runtime (rr_host.cpp)
// against the launch stand-ins of host_stubs.cpp, for a g++ build with
// AddressSanitizer and UndefinedBehaviorSanitizer (tests/test_sanitizers_cpu.py).
// Device pointers are fake, 256-byte aligned addresses that nothing
// dereferences; workspaces are real host buffers of the size the library asks
// for, so that the stand-ins can check the carved-out buffers against them.
// Exit status 0 when every call returns the expected status.
#include <limits.h>
#include <math.h>
#include <stdio.h>
#include <stdlib.h>

#include "rr_attn.h"
#include "stub_state.h"

static int bad = 0;
#define EXPECT(call, want)                                                                        \
  do {                                                                                            \
    const rr_status got_ = (call);                                                                \
    if (got_ != (want)) {                                                                         \
      fprintf(stderr, "line %d: %s returned %d, expected %d\n", __LINE__, #call, got_, want);     \
      bad = 1;                                                                                    \
    }                                                                                             \
  } while (0)

static void* fake(int n) { return reinterpret_cast<void*>((uintptr_t)(n + 1) << 28); }
static int32_t* ifake(int n) { return static_cast<int32_t*>(fake(n)); }
static float* ffake(int n) { return static_cast<float*>(fake(n)); }

static void* workspace(size_t bytes) {
  void* p = aligned_alloc(256, (bytes + 255) / 256 * 256 + 256);
  g_stub.ws = p;
  g_stub.ws_bytes = bytes;
  return p;
}

static void problem_calls(rr_problem p) {
  const size_t need = rr_workspace_bytes(&p);
  if (need == 0) {
    fprintf(stderr, "rr_workspace_bytes returned 0 for a supported problem (L=%d)\n", p.L);
    bad = 1;
    return;
  }
  void* ws = workspace(need);
  g_stub.user_mass = false;
  EXPECT(rr_pattern_search(&p, fake(1), fake(2), ifake(3), ifake(4), nullptr, ws, need, nullptr), RR_OK);
  g_stub.user_mass = true;
  EXPECT(rr_pattern_search(&p, fake(1), fake(2), ifake(3), ifake(4), ffake(5), ws, need, nullptr), RR_OK);
  EXPECT(rr_pattern_search_heads(&p, fake(1), fake(2), ffake(6), ifake(3), ifake(4), ffake(5), ws, need, nullptr),
         RR_OK);
  g_stub.user_mass = false;
  EXPECT(rr_block_sparse_attn(&p, fake(1), fake(2), fake(7), ifake(3), ifake(4), fake(8), ws, need, nullptr), RR_OK);
  EXPECT(rr_prefill(&p, fake(1), fake(2), fake(7), fake(8), ifake(3), ifake(4), ws, need, nullptr), RR_OK);
  EXPECT(rr_mass_recall(&p, fake(1), fake(2), ifake(3), ifake(4), ffake(9), nullptr), RR_OK);
  EXPECT(rr_share_group_lists(&p, ifake(3), ifake(4), ifake(10), ifake(11), nullptr), RR_OK);
  EXPECT(rr_pool_keys(&p, fake(2), fake(12), nullptr), RR_OK);
  // the workspace one byte short, misaligned, missing
  EXPECT(rr_prefill(&p, fake(1), fake(2), fake(7), fake(8), ifake(3), ifake(4), ws, need - 1, nullptr),
         RR_ERR_WORKSPACE);
  EXPECT(rr_prefill(&p, fake(1), fake(2), fake(7), fake(8), ifake(3), ifake(4), static_cast<char*>(ws) + 8, need,
                    nullptr),
         RR_ERR_WORKSPACE);
  EXPECT(rr_prefill(&p, fake(1), fake(2), fake(7), fake(8), ifake(3), ifake(4), nullptr, need, nullptr),
         RR_ERR_WORKSPACE);
  free(ws);

  // decode on the same shape: pooled keys in the workspace or given, masses exported or not
  const size_t dneed = rr_decode_workspace_bytes(&p);
  void* dws = workspace(dneed);
  for (int kb = 0; kb < 2; ++kb)
    for (int bm = 0; bm < 2; ++bm) {
      g_stub.user_kbar = kb;
      g_stub.user_mass = bm;
      EXPECT(rr_decode(&p, fake(1), fake(2), fake(7), kb ? fake(12) : nullptr, fake(8), ifake(3), ifake(4),
                       bm ? ffake(5) : nullptr, dws, dneed, nullptr),
             RR_OK);
    }
  g_stub.user_kbar = false;
  g_stub.user_mass = false;
  EXPECT(rr_decode_attend(&p, fake(1), fake(2), fake(7), ifake(3), ifake(4), fake(8), dws, dneed, nullptr), RR_OK);
  EXPECT(rr_decode(&p, fake(1), fake(2), fake(7), nullptr, fake(8), ifake(3), ifake(4), nullptr, dws, dneed - 1,
                   nullptr),
         RR_ERR_WORKSPACE);
  free(dws);
  const rr_status want = dneed <= RR_DECODE_NOALLOC_MAX_WS ? RR_OK : RR_ERR_WORKSPACE;
  EXPECT(rr_decode_noalloc(&p, fake(1), fake(2), fake(7), nullptr, fake(8), ifake(3), ifake(4), nullptr, nullptr),
         want);
  g_stub.user_kbar = true;
  EXPECT(rr_decode_noalloc(&p, fake(1), fake(2), fake(7), fake(12), fake(8), ifake(3), ifake(4), nullptr, nullptr),
         RR_OK);
  g_stub.user_kbar = false;
}

int main() {
  const rr_problem shapes[] = {
      {2048, 8, 2, 128, 16, 128, 0.9f, 1, RR_BF16},   // whole blocks, G = 4
      {1000, 6, 2, 128, 16, 128, 0.9f, 1, RR_BF16},   // ragged length, odd G
      {777, 4, 4, 64, 8, 64, 0.85f, 0, RR_FP32},      // fp32, non-causal, short tail
      {1, 2, 1, 64, 4, 64, 1.0f, 1, RR_BF16},         // a single token
      {4096, 3, 3, 64, 2, 64, 0.5f, 1, RR_BF16},      // r = 32
  };
  for (const rr_problem& p : shapes) problem_calls(p);

  // varlen: three sequences packed, one shared workspace, lists packed per sequence
  rr_problem pv = {300 + 1000 + 128, 8, 2, 128, 16, 128, 0.9f, 1, RR_BF16};
  const int32_t lens[3] = {300, 1000, 128};
  const size_t vneed = rr_workspace_bytes_varlen(&pv, 3, lens);
  void* vws = workspace(vneed);
  EXPECT(rr_prefill_varlen(&pv, 3, lens, fake(1), fake(2), fake(7), fake(8), ifake(3), ifake(4), vws, vneed, nullptr),
         RR_OK);
  if (g_stub.batched_launches != 1 || g_stub.batched_searches != 3) {  // three sequences: one launch per kernel
    fprintf(stderr, "varlen: %ld batched attention launches, %ld batched search launches\n", g_stub.batched_launches,
            g_stub.batched_searches);
    bad = 1;
  }
  free(vws);
  {  // 40 sequences: two launch groups (32 + 8)
    int32_t many[40];
    int total = 0;
    for (int b = 0; b < 40; ++b) total += (many[b] = 50 + 37 * b);
    rr_problem pm = {total, 8, 2, 64, 8, 128, 0.9f, 1, RR_BF16};
    const size_t mneed = rr_workspace_bytes_varlen(&pm, 40, many);
    void* mws = workspace(mneed);
    const long before_launches = g_stub.batched_launches;
    EXPECT(rr_prefill_varlen(&pm, 40, many, fake(1), fake(2), fake(7), fake(8), ifake(3), ifake(4), mws, mneed,
                             nullptr),
           RR_OK);
    if (g_stub.batched_launches - before_launches != 2) {
      fprintf(stderr, "40 sequences: %ld batched launches\n", g_stub.batched_launches - before_launches);
      bad = 1;
    }
    free(mws);
    {  // one sequence long enough for a launch of its own (8 items per CU at 256 CUs), two batched
      const int32_t mixed[3] = {70000, 1000, 333};
      rr_problem px = {70000 + 1000 + 333, 8, 2, 128, 16, 128, 0.9f, 1, RR_BF16};
      const size_t xneed = rr_workspace_bytes_varlen(&px, 3, mixed);
      void* xws = workspace(xneed);
      const long b0 = g_stub.batched_launches, s0 = g_stub.single_launches;
      EXPECT(rr_prefill_varlen(&px, 3, mixed, fake(1), fake(2), fake(7), fake(8), ifake(3), ifake(4), xws, xneed,
                               nullptr),
             RR_OK);
      if (g_stub.single_launches - s0 != 1 || g_stub.batched_launches - b0 != 1) {
        fprintf(stderr, "mixed lengths: %ld solo and %ld batched launches\n", g_stub.single_launches - s0,
                g_stub.batched_launches - b0);
        bad = 1;
      }
      free(xws);
    }
    {  // one query head per KV head (bf16, B = 128): batched like the grouped layers
      rr_problem pg = {300 + 1000 + 128, 4, 4, 128, 16, 128, 0.9f, 1, RR_BF16};
      const size_t gneed = rr_workspace_bytes_varlen(&pg, 3, lens);
      void* gws = workspace(gneed);
      const long b0 = g_stub.batched_launches;
      EXPECT(rr_prefill_varlen(&pg, 3, lens, fake(1), fake(2), fake(7), fake(8), ifake(3), ifake(4), gws, gneed,
                               nullptr),
             RR_OK);
      if (g_stub.batched_launches - b0 != 1) {
        fprintf(stderr, "MHA varlen: %ld batched launches\n", g_stub.batched_launches - b0);
        bad = 1;
      }
      free(gws);
    }
    rr_problem pf = {300 + 1000 + 128, 4, 4, 64, 8, 64, 0.9f, 1, RR_FP32};  // per-sequence attention
    const size_t fneed = rr_workspace_bytes_varlen(&pf, 3, lens);
    void* fws = workspace(fneed);
    EXPECT(rr_prefill_varlen(&pf, 3, lens, fake(1), fake(2), fake(7), fake(8), ifake(3), ifake(4), fws, fneed,
                             nullptr),
           RR_OK);
    free(fws);
    vws = workspace(vneed);
  }
  const int32_t bad_lens[3] = {300, -5, 1133};
  EXPECT(rr_prefill_varlen(&pv, 3, bad_lens, fake(1), fake(2), fake(7), fake(8), ifake(3), ifake(4), vws, vneed,
                           nullptr),
         RR_ERR_INVALID_ARG);
  free(vws);

  // invalid and extreme problems: rejected before any launch, with no overflow on the way
  const long before = g_stub.calls;
  const rr_problem rejected[] = {
      {INT_MAX, 32, 8, 128, 16, 128, 0.9f, 1, RR_BF16},  // too many blocks
      {INT_MAX - 1, 1, 1, 64, 2, 64, 0.9f, 1, RR_BF16},
      {2048, INT_MAX, 1, 128, 16, 128, 0.9f, 1, RR_BF16},
      {2048, 8, 3, 128, 16, 128, 0.9f, 1, RR_BF16},      // Hq % Hkv
      {2048, 8, 2, 96, 16, 128, 0.9f, 1, RR_BF16},       // d
      {2048, 8, 2, 128, 48, 128, 0.9f, 1, RR_BF16},      // B % S
      {2048, 8, 2, 128, 16, 128, NAN, 1, RR_BF16},       // tau
      {2048, 8, 2, 128, 16, 128, 1.5f, 1, RR_BF16},
      {2048, 8, 2, 128, 16, 128, 0.9f, 2, RR_BF16},      // causal flag
      {2048, 8, 2, 128, 16, 128, 0.9f, 1, 7},            // dtype
      {-5, 8, 2, 128, 16, 128, 0.9f, 1, RR_BF16},
  };
  char ws_small[512];
  for (const rr_problem& p : rejected) {
    (void)rr_workspace_bytes(&p);
    (void)rr_decode_workspace_bytes(&p);
    const rr_status s =
        rr_prefill(&p, fake(1), fake(2), fake(7), fake(8), ifake(3), ifake(4), ws_small, sizeof ws_small, nullptr);
    if (s != RR_ERR_INVALID_ARG && s != RR_ERR_UNSUPPORTED) {
      fprintf(stderr, "problem L=%d Hq=%d accepted (%d)\n", p.L, p.Hq, s);
      bad = 1;
    }
    EXPECT(rr_decode_noalloc(&p, fake(1), fake(2), fake(7), nullptr, fake(8), ifake(3), ifake(4), nullptr, nullptr),
           s);
  }
  if (g_stub.calls != before) {
    fprintf(stderr, "a rejected problem reached a launch\n");
    bad = 1;
  }
  EXPECT(rr_prefill(nullptr, fake(1), fake(2), fake(7), fake(8), ifake(3), ifake(4), ws_small, 1, nullptr),
         RR_ERR_INVALID_ARG);

  // a failing launch is reported as RR_ERR_HIP
  rr_problem p = shapes[0];
  const size_t need = rr_workspace_bytes(&p);
  void* ws = workspace(need);
  g_stub.fail_launch = true;
  EXPECT(rr_pattern_search(&p, fake(1), fake(2), ifake(3), ifake(4), nullptr, ws, need, nullptr), RR_ERR_HIP);
  g_stub.fail_launch = false;
  free(ws);

  for (int s = -1; s < 6; ++s)
    if (!rr_status_string(static_cast<rr_status>(s))) bad = 1;
  if (rr_version() < 100) bad = 1;
  if (!bad) printf("host driver ok\n");
  return bad;
}
