// Host runtime of the C ABI declared in include/rr_attn.h: argument checks,
// workspace carving and the launch sequence of the two RRAttention stages
// ("RRAttention: Dynamic Block Sparse Attention via Per-Head Round-Robin
// Shifts for Long-Context Inference", abstract and Figure 2 caption: search,
// then sparse attention). Everything is enqueued on the caller's stream; the
// library allocates nothing and keeps no state.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <new>

#include "rr_attn.h"
#include "rr_kernels.h"

static_assert(rr::kStaticWorkspaceBytes == RR_DECODE_NOALLOC_MAX_WS, "header and library disagree");

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }
bool is_pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

rr_status make_geometry(const rr_problem* p, rr::Geometry* g) {
  if (!p) return RR_ERR_INVALID_ARG;
  if (p->L <= 0 || p->Hq <= 0 || p->Hkv <= 0 || p->d <= 0 || p->S <= 0 || p->B <= 0)
    return RR_ERR_INVALID_ARG;
  if (p->Hq % p->Hkv != 0) return RR_ERR_INVALID_ARG;
  if (p->B % p->S != 0) return RR_ERR_INVALID_ARG;  // L need not be a multiple of B or S
  if (!(p->tau > 0.0f && p->tau <= 1.0f)) return RR_ERR_INVALID_ARG;  // NaN fails too
  if (p->causal != 0 && p->causal != 1) return RR_ERR_INVALID_ARG;
  if (p->dtype != RR_BF16 && p->dtype != RR_FP32) return RR_ERR_INVALID_ARG;
  if (p->d != 64 && p->d != 128) return RR_ERR_UNSUPPORTED;
  if (p->B != 64 && p->B != 128) return RR_ERR_UNSUPPORTED;
  const int r = p->B / p->S;
  if (!is_pow2(p->S) || r < 2 || r > 32) return RR_ERR_UNSUPPORTED;
  // the last block may be short (64-bit: L near INT_MAX must not overflow)
  const long long nbl = ((long long)p->L + p->B - 1) / p->B;
  if (nbl > rr::kMaxSelectBlocks) return RR_ERR_UNSUPPORTED;
  const int nb = (int)nbl;
  if ((long long)p->Hq * nb > (1LL << 30)) return RR_ERR_UNSUPPORTED;
  g->L = p->L;
  g->Hq = p->Hq;
  g->Hkv = p->Hkv;
  g->d = p->d;
  g->S = p->S;
  g->B = p->B;
  g->nb = nb;
  g->ns = (int)(((long long)p->L + p->S - 1) / p->S);  // the last stride may be short
  g->r = r;
  g->G = p->Hq / p->Hkv;
  g->causal = p->causal;
  g->bf16 = p->dtype == RR_BF16;
  g->tau = p->tau;
  return RR_OK;
}

struct Workspace {
  size_t kbar, mass, vt, queues, total;  // byte offsets and total size
};

// V re-laid out per key block (bf16 attention kernels)
size_t vt_bytes(const rr::Geometry& g) { return (size_t)g.nb * g.B * g.Hkv * g.d * 2; }

Workspace layout(const rr::Geometry& g) {
  const size_t esz = g.bf16 ? 2 : 4;
  Workspace w;
  size_t off = 0;
  w.kbar = off;
  off += align_up((size_t)g.ns * g.Hkv * g.d * esz);
  w.mass = off;
  off += align_up((size_t)g.Hq * g.nb * g.nb * sizeof(float));
  w.vt = off;  // nb whole tiles: a short last block is padded with zeros
  if (g.bf16) off += align_up(vt_bytes(g));
  w.queues = off;  // the attention's work-queue counters
  if (g.bf16) off += align_up(rr::kAttnQueues * sizeof(int32_t));
  w.total = off;
  return w;
}

rr_status check_ws(const rr::Geometry& g, const void* ws, size_t ws_bytes) {
  if (!ws || !aligned16(ws) || ws_bytes < layout(g).total) return RR_ERR_WORKSPACE;
  return RR_OK;
}

rr_status hip_status(hipError_t e) { return e == hipSuccess ? RR_OK : RR_ERR_HIP; }

rr_status run_search(const rr::Geometry& g, const void* q, const void* k, int32_t* row_count,
                     int32_t* col_idx, float* block_mass, const float* tau_heads, void* ws, hipStream_t st) {
  const Workspace w = layout(g);
  uint8_t* base = static_cast<uint8_t*>(ws);
  void* kbar = base + w.kbar;
  float* mass = block_mass ? block_mass : reinterpret_cast<float*>(base + w.mass);
  hipError_t e = rr::launch_pool_keys(g, k, kbar, true, st);
  if (e == hipSuccess) e = rr::launch_search(g, q, kbar, mass, st);
  if (e == hipSuccess) e = rr::launch_select(g, mass, block_mass != nullptr, row_count, col_idx, tau_heads, st);
  return hip_status(e);
}

rr_status run_attention(const rr::Geometry& g, const void* q, const void* k, const void* v,
                        const int32_t* row_count, const int32_t* col_idx, void* out, void* ws,
                        hipStream_t st) {
  const Workspace w = layout(g);
  void* vt = static_cast<uint8_t*>(ws) + w.vt;
  int32_t* queues = reinterpret_cast<int32_t*>(static_cast<uint8_t*>(ws) + w.queues);
  hipError_t e = hipSuccess;
  if (g.bf16) e = rr::launch_transpose_v(g, v, vt, queues, st);
  if (e == hipSuccess) e = rr::launch_attention(g, q, k, v, vt, queues, row_count, col_idx, out, st);
  return hip_status(e);
}

}  // namespace

extern "C" {

size_t rr_workspace_bytes(const rr_problem* p) {
  rr::Geometry g;
  if (make_geometry(p, &g) != RR_OK) return 0;
  return layout(g).total;
}

rr_status rr_pattern_search(const rr_problem* p, const void* q, const void* k, int32_t* row_count,
                            int32_t* col_idx, float* block_mass, void* ws, size_t ws_bytes,
                            void* stream) {
  rr::Geometry g;
  rr_status s = make_geometry(p, &g);
  if (s != RR_OK) return s;
  if (!q || !k || !row_count || !col_idx) return RR_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(row_count) || !aligned16(col_idx))
    return RR_ERR_INVALID_ARG;
  if (block_mass && !aligned16(block_mass)) return RR_ERR_INVALID_ARG;
  if ((s = check_ws(g, ws, ws_bytes)) != RR_OK) return s;
  return run_search(g, q, k, row_count, col_idx, block_mass, nullptr, ws, static_cast<hipStream_t>(stream));
}

rr_status rr_pattern_search_heads(const rr_problem* p, const void* q, const void* k, const float* tau_per_head,
                                  int32_t* row_count, int32_t* col_idx, float* block_mass, void* ws,
                                  size_t ws_bytes, void* stream) {
  rr::Geometry g;
  rr_status s = make_geometry(p, &g);
  if (s != RR_OK) return s;
  if (!q || !k || !tau_per_head || !row_count || !col_idx) return RR_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(row_count) || !aligned16(col_idx) ||
      (reinterpret_cast<uintptr_t>(tau_per_head) & 3u) != 0)
    return RR_ERR_INVALID_ARG;
  if (block_mass && !aligned16(block_mass)) return RR_ERR_INVALID_ARG;
  if ((s = check_ws(g, ws, ws_bytes)) != RR_OK) return s;
  return run_search(g, q, k, row_count, col_idx, block_mass, tau_per_head, ws, static_cast<hipStream_t>(stream));
}

rr_status rr_block_sparse_attn(const rr_problem* p, const void* q, const void* k, const void* v,
                               const int32_t* row_count, const int32_t* col_idx, void* out, void* ws,
                               size_t ws_bytes, void* stream) {
  rr::Geometry g;
  rr_status s = make_geometry(p, &g);
  if (s != RR_OK) return s;
  if (!q || !k || !v || !row_count || !col_idx || !out) return RR_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(row_count) ||
      !aligned16(col_idx) || !aligned16(out))
    return RR_ERR_INVALID_ARG;
  if ((s = check_ws(g, ws, ws_bytes)) != RR_OK) return s;
  return run_attention(g, q, k, v, row_count, col_idx, out, ws, static_cast<hipStream_t>(stream));
}

rr_status rr_prefill(const rr_problem* p, const void* q, const void* k, const void* v, void* out,
                     int32_t* row_count, int32_t* col_idx, void* ws, size_t ws_bytes, void* stream) {
  rr::Geometry g;
  rr_status s = make_geometry(p, &g);
  if (s != RR_OK) return s;
  if (!q || !k || !v || !out || !row_count || !col_idx) return RR_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) ||
      !aligned16(row_count) || !aligned16(col_idx))
    return RR_ERR_INVALID_ARG;
  if ((s = check_ws(g, ws, ws_bytes)) != RR_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  s = run_search(g, q, k, row_count, col_idx, nullptr, nullptr, ws, st);
  if (s != RR_OK) return s;
  return run_attention(g, q, k, v, row_count, col_idx, out, ws, st);
}

// Packed variable-length batch: the per-sequence problems, validated before
// anything is enqueued, and the workspace the batch needs. Without the
// head-pair kernel each sequence is searched and attended in turn and reuses
// the workspace as a single sequence would (total = the largest single
// layout). With it, the first part holds the pooled keys and masses of every
// sequence at once (a batched search) or of the longest one (a sequence run
// on its own), whichever is larger; every sequence's V re-layout follows
// (vt_base, in sequence order), then the queue counters (queues). A sequence
// run on its own uses the single-sequence layout, which lies inside this one.
struct VarlenWorkspace {
  size_t vt_base, queues, total;
  bool batched;
};

static rr_status varlen_geometries(const rr_problem* p, int32_t n_seq, const int32_t* seq_lens,
                                   VarlenWorkspace* vw) {
  if (!p || n_seq <= 0 || !seq_lens) return RR_ERR_INVALID_ARG;
  long long total = 0;
  size_t single = 0, search = 0, searches = 0, vts = 0;
  bool pair = false;
  for (int32_t b = 0; b < n_seq; ++b) {
    if (seq_lens[b] <= 0) return RR_ERR_INVALID_ARG;
    rr_problem pb = *p;
    pb.L = seq_lens[b];
    rr::Geometry g;
    const rr_status s = make_geometry(&pb, &g);
    if (s != RR_OK) return s;
    const Workspace w = layout(g);
    single = std::max(single, w.total);
    search = std::max(search, w.vt);  // pooled keys and masses of one sequence
    searches += w.vt;                 // ... of every sequence at once (batched search)
    vts += align_up(vt_bytes(g));
    pair = rr::attn_pair_shape(g);
    total += seq_lens[b];
  }
  if (total != p->L) return RR_ERR_INVALID_ARG;
  vw->batched = pair;
  if (pair) search = std::max(search, searches);
  vw->vt_base = search;
  vw->queues = search + vts;
  vw->total = pair ? vw->queues + align_up(rr::kAttnQueues * sizeof(int32_t)) : single;
  return RR_OK;
}

size_t rr_workspace_bytes_varlen(const rr_problem* p, int32_t n_seq, const int32_t* seq_lens) {
  VarlenWorkspace vw;
  return varlen_geometries(p, n_seq, seq_lens, &vw) == RR_OK ? vw.total : 0;
}

rr_status rr_prefill_varlen(const rr_problem* p, int32_t n_seq, const int32_t* seq_lens, const void* q,
                            const void* k, const void* v, void* out, int32_t* row_count, int32_t* col_idx,
                            void* ws, size_t ws_bytes, void* stream) {
  VarlenWorkspace vw;
  rr_status s = varlen_geometries(p, n_seq, seq_lens, &vw);
  if (s != RR_OK) return s;
  const size_t need = vw.total;
  if (!q || !k || !v || !out || !row_count || !col_idx) return RR_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(row_count) ||
      !aligned16(col_idx))
    return RR_ERR_INVALID_ARG;
  if (!ws || !aligned16(ws) || ws_bytes < need) return RR_ERR_WORKSPACE;
  // every sequence's tensors and lists must start 16-byte aligned
  const size_t esz = p->dtype == RR_BF16 ? 2 : 4;
  for (int32_t b = 0; b < n_seq; ++b) {
    const size_t nb = ((size_t)seq_lens[b] + p->B - 1) / p->B;
    if (((size_t)seq_lens[b] * p->Hkv * p->d * esz) % 16 || ((size_t)p->Hq * nb * sizeof(int32_t)) % 16)
      return RR_ERR_UNSUPPORTED;
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  struct Seq {
    int32_t len;
    size_t tok, rc, ci, vt;
  };
  Seq seqs_small[64];
  Seq* seqs = n_seq <= 64 ? seqs_small : new (std::nothrow) Seq[n_seq];
  if (!seqs) return RR_ERR_INVALID_ARG;
  struct FreeSeqs {  // releases seqs on every return below
    Seq *heap, *inline_buf;
    ~FreeSeqs() {
      if (heap != inline_buf) delete[] heap;
    }
  } free_seqs{seqs, seqs_small};
  {
    size_t tok = 0, rc_off = 0, ci_off = 0, vt_off = 0;
    for (int32_t b = 0; b < n_seq; ++b) {
      rr_problem pb = *p;
      pb.L = seq_lens[b];
      rr::Geometry g;
      make_geometry(&pb, &g);
      seqs[b] = Seq{seq_lens[b], tok, rc_off, ci_off, vt_off};
      tok += seq_lens[b];
      rc_off += (size_t)g.Hq * g.nb;
      ci_off += (size_t)g.Hq * g.nb * g.nb;
      vt_off += align_up(vt_bytes(g));
    }
  }
  auto geometry = [&](const Seq& sq) {
    rr_problem pb = *p;
    pb.L = sq.len;
    rr::Geometry g;
    make_geometry(&pb, &g);
    return g;
  };
  // the sequences' searches share the workspace's pooled-key and mass regions,
  // a single-sequence attention its V re-layout region: everything runs in
  // stream order, so no two of them use one region at once
  auto search = [&](const Seq& sq) {
    return run_search(geometry(sq), static_cast<const uint8_t*>(q) + sq.tok * p->Hq * p->d * esz,
                      static_cast<const uint8_t*>(k) + sq.tok * p->Hkv * p->d * esz, row_count + sq.rc,
                      col_idx + sq.ci, nullptr, nullptr, ws, st);
  };
  auto attend = [&](const Seq& sq) {
    return run_attention(geometry(sq), static_cast<const uint8_t*>(q) + sq.tok * p->Hq * p->d * esz,
                         static_cast<const uint8_t*>(k) + sq.tok * p->Hkv * p->d * esz,
                         static_cast<const uint8_t*>(v) + sq.tok * p->Hkv * p->d * esz, row_count + sq.rc,
                         col_idx + sq.ci, static_cast<uint8_t*>(out) + sq.tok * p->Hq * p->d * esz, ws, st);
  };
  if (!vw.batched) {  // the other kernels: each sequence searched and attended in turn
    for (int32_t b = 0; b < n_seq; ++b) {
      if ((s = search(seqs[b])) != RR_OK || (s = attend(seqs[b])) != RR_OK) return s;
    }
    return RR_OK;
  }
  // Head-pair attention, longest sequences first: a sequence with at least
  // kVarlenSoloItemsPerCU work items per CU is searched and attended in
  // launches of its own (a single-sequence launch fills the GPU and can
  // balance its XCDs through the work queues); the others are searched
  // together and attended together, one launch per kernel per group of
  // kMaxSeqPerLaunch, each sequence's work on a range of its own.
  std::stable_sort(seqs, seqs + n_seq, [](const Seq& a, const Seq& b) { return a.len > b.len; });
  int ncu = 0;
  hipError_t e = rr::attn_cu_count(st, &ncu);
  if (e != hipSuccess) return hip_status(e);
  int32_t nsolo = 0;
  while (nsolo < n_seq &&
         (long long)rr::attn_items(geometry(seqs[nsolo])) >= (long long)rr::kVarlenSoloItemsPerCU * ncu) {
    if ((s = search(seqs[nsolo])) != RR_OK || (s = attend(seqs[nsolo])) != RR_OK) return s;
    ++nsolo;
  }
  const rr::Geometry g0 = geometry(seqs[0]);
  uint8_t* vt = static_cast<uint8_t*>(ws) + vw.vt_base;
  int32_t* queues = reinterpret_cast<int32_t*>(static_cast<uint8_t*>(ws) + vw.queues);
  // the other sequences' searches: pooled keys, scores and selection of up to
  // kMaxSeqPerLaunch sequences per launch, each sequence's pooled keys and
  // masses in a region of their own at the start of the workspace
  for (int32_t b0 = nsolo; b0 < n_seq && e == hipSuccess; b0 += rr::kMaxSeqPerLaunch) {
    rr::SearchBatch sbt;
    sbt.n = std::min<int32_t>(rr::kMaxSeqPerLaunch, n_seq - b0);
    int pool = 0, blk = 0, rows = 0;
    size_t off = 0;
    for (int m = 0; m < sbt.n; ++m) {
      const Seq& sq = seqs[b0 + m];
      const rr::Geometry g = geometry(sq);
      const Workspace w = layout(g);
      int np, nbk, nr;
      rr::search_batch_counts(g, g.nb, g.ns, &np, &nbk, &nr);
      sbt.pool_off[m] = pool;
      sbt.blk_off[m] = blk;
      sbt.row_off[m] = rows;
      sbt.tok_off[m] = (int)sq.tok;
      sbt.L[m] = sq.len;
      sbt.nb[m] = g.nb;
      sbt.ns[m] = g.ns;
      sbt.kbar_off[m] = (long long)(off / esz);
      sbt.mass_off[m] = (long long)((off + w.mass) / sizeof(float));
      sbt.rc_off[m] = (long long)sq.rc;
      sbt.ci_off[m] = (long long)sq.ci;
      pool += np;
      blk += nbk;
      rows += nr;
      off += w.vt;  // this sequence's pooled keys and masses
    }
    sbt.pool_off[sbt.n] = pool;
    sbt.blk_off[sbt.n] = blk;
    sbt.row_off[sbt.n] = rows;
    float* mass = reinterpret_cast<float*>(ws);
    e = rr::launch_pool_keys_batched(g0, sbt, k, ws, st);
    if (e == hipSuccess) e = rr::launch_search_batched(g0, sbt, q, ws, mass, st);
    if (e == hipSuccess) e = rr::launch_select_batched(g0, sbt, mass, row_count, col_idx, st);
  }
  for (int32_t b0 = nsolo; b0 < n_seq && e == hipSuccess; b0 += rr::kMaxSeqPerLaunch) {
    rr::SeqBatch sb;
    sb.n = std::min<int32_t>(rr::kMaxSeqPerLaunch, n_seq - b0);
    int items = 0, tiles = 0;
    for (int m = 0; m < sb.n; ++m) {
      const Seq& sq = seqs[b0 + m];
      const rr::Geometry g = geometry(sq);
      sb.item_off[m] = items;
      sb.tile_off[m] = tiles;
      sb.tok_off[m] = (int)sq.tok;
      sb.L[m] = sq.len;
      sb.nb[m] = g.nb;
      sb.rc_off[m] = (long long)sq.rc;
      sb.ci_off[m] = (long long)sq.ci;
      sb.vt_off[m] = (long long)sq.vt;
      items += (rr::attn_items(g) + 15) / 16 * 16;
      tiles += g.Hkv * g.nb;
    }
    sb.item_off[sb.n] = items;
    sb.tile_off[sb.n] = tiles;
    e = rr::launch_transpose_v_batched(g0, sb, v, vt, queues, st);
    if (e == hipSuccess) e = rr::launch_attention_batched(g0, sb, q, k, vt, queues, row_count, col_idx, out, st);
  }
  return hip_status(e);
}

rr_status rr_mass_recall(const rr_problem* p, const void* q, const void* k, const int32_t* row_count,
                         const int32_t* col_idx, float* recall, void* stream) {
  rr::Geometry g;
  rr_status s = make_geometry(p, &g);
  if (s != RR_OK) return s;
  if (!q || !k || !row_count || !col_idx || !recall) return RR_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(row_count) || !aligned16(col_idx) || !aligned16(recall))
    return RR_ERR_INVALID_ARG;
  return hip_status(rr::launch_recall(g, q, k, row_count, col_idx, recall, static_cast<hipStream_t>(stream)));
}

rr_status rr_share_group_lists(const rr_problem* p, const int32_t* row_count, const int32_t* col_idx,
                               int32_t* shared_row_count, int32_t* shared_col_idx, void* stream) {
  rr::Geometry g;
  rr_status s = make_geometry(p, &g);
  if (s != RR_OK) return s;
  if (!row_count || !col_idx || !shared_row_count || !shared_col_idx) return RR_ERR_INVALID_ARG;
  if (!aligned16(row_count) || !aligned16(col_idx) || !aligned16(shared_row_count) || !aligned16(shared_col_idx))
    return RR_ERR_INVALID_ARG;
  // the outputs are written while other rows of the inputs are still read
  const uintptr_t in0 = reinterpret_cast<uintptr_t>(col_idx), out0 = reinterpret_cast<uintptr_t>(shared_col_idx);
  const uintptr_t ci_bytes = (uintptr_t)g.Hq * g.nb * g.nb * sizeof(int32_t);
  const uintptr_t rc_bytes = (uintptr_t)g.Hq * g.nb * sizeof(int32_t);
  const uintptr_t r0 = reinterpret_cast<uintptr_t>(row_count), s0 = reinterpret_cast<uintptr_t>(shared_row_count);
  auto overlap = [](uintptr_t a, uintptr_t na, uintptr_t b, uintptr_t nb_) { return a < b + nb_ && b < a + na; };
  if (overlap(in0, ci_bytes, out0, ci_bytes) || overlap(r0, rc_bytes, s0, rc_bytes) ||
      overlap(in0, ci_bytes, s0, rc_bytes) || overlap(r0, rc_bytes, out0, ci_bytes))
    return RR_ERR_INVALID_ARG;
  return hip_status(rr::launch_union_lists(g, row_count, col_idx, shared_row_count, shared_col_idx,
                                           static_cast<hipStream_t>(stream)));
}

// Decode workspace: pooled keys | block sums [Hq][nb] | score-chunk partials | masses [Hq][nb] |
// selection flags [Hq][nbp] | split partials.
struct DecodeWorkspace {
  size_t kbar, bsum, zpart, mass, sel, part, total;
  int nbp;
};

DecodeWorkspace decode_layout(const rr::Geometry& g) {
  const size_t esz = g.bf16 ? 2 : 4;
  DecodeWorkspace w;
  size_t off = 0;
  w.kbar = off;
  off += align_up((size_t)g.ns * g.Hkv * g.d * esz);
  w.bsum = off;
  off += align_up((size_t)g.Hq * g.nb * sizeof(float));
  w.zpart = off;
  off += align_up((size_t)g.Hq * rr::decode_chunks(g) * 2 * sizeof(float));
  w.mass = off;
  off += align_up((size_t)g.Hq * g.nb * sizeof(float));
  w.sel = off;
  w.nbp = (g.nb + 15) / 16 * 16;
  off += align_up((size_t)g.Hq * w.nbp);
  w.part = off;
  off += align_up((size_t)g.Hq * rr::decode_splits(g) * (g.d + 2) * sizeof(float));
  w.total = off;
  return w;
}

size_t rr_decode_workspace_bytes(const rr_problem* p) {
  rr::Geometry g;
  if (make_geometry(p, &g) != RR_OK) return 0;
  return decode_layout(g).total;
}

rr_status rr_pool_keys(const rr_problem* p, const void* k, void* kbar, void* stream) {
  rr::Geometry g;
  rr_status s = make_geometry(p, &g);
  if (s != RR_OK) return s;
  if (!k || !kbar || !aligned16(k) || !aligned16(kbar)) return RR_ERR_INVALID_ARG;
  return hip_status(rr::launch_pool_keys(g, k, kbar, false, static_cast<hipStream_t>(stream)));
}

static rr_status decode_step(const rr_problem* p, const void* q, const void* k, const void* v, const void* kbar,
                             void* out, int32_t* row_count, int32_t* col_idx, float* block_mass, void* ws,
                             size_t ws_bytes, bool static_ws, void* stream) {
  rr::Geometry g;
  rr_status s = make_geometry(p, &g);
  if (s != RR_OK) return s;
  if (!q || !k || !v || !out || !row_count || !col_idx) return RR_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(row_count) ||
      !aligned16(col_idx))
    return RR_ERR_INVALID_ARG;
  if (block_mass && !aligned16(block_mass)) return RR_ERR_INVALID_ARG;
  if (kbar && !aligned16(kbar)) return RR_ERR_INVALID_ARG;
  const DecodeWorkspace w = decode_layout(g);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (static_ws) {  // the library's own buffer on the stream's device
    if (w.total > rr::kStaticWorkspaceBytes) return RR_ERR_WORKSPACE;
    if (rr::static_workspace(st, &ws) != hipSuccess) return RR_ERR_HIP;
    ws_bytes = rr::kStaticWorkspaceBytes;
  }
  if (!ws || !aligned16(ws) || ws_bytes < w.total) return RR_ERR_WORKSPACE;
  uint8_t* base = static_cast<uint8_t*>(ws);
  float* mass = block_mass ? block_mass : reinterpret_cast<float*>(base + w.mass);
  hipError_t e = hipSuccess;
  if (!kbar) {  // pool the cache's keys here
    e = rr::launch_pool_keys(g, k, base + w.kbar, false, st);
    kbar = base + w.kbar;
  }
  if (e == hipSuccess)
    e = rr::launch_decode_scores(g, q, kbar, reinterpret_cast<float*>(base + w.bsum),
                                 reinterpret_cast<float*>(base + w.zpart), st);
  uint8_t* sel = base + w.sel;
  if (e == hipSuccess)
    e = rr::launch_decode_select(g, reinterpret_cast<const float*>(base + w.bsum),
                                 reinterpret_cast<const float*>(base + w.zpart), mass, row_count, col_idx, sel, w.nbp,
                                 st);
  if (e == hipSuccess)
    e = rr::launch_decode_attn(g, q, k, v, row_count, col_idx, sel, w.nbp, reinterpret_cast<float*>(base + w.part),
                               out, st);
  return hip_status(e);
}

rr_status rr_decode(const rr_problem* p, const void* q, const void* k, const void* v, const void* kbar, void* out,
                    int32_t* row_count, int32_t* col_idx, float* block_mass, void* ws, size_t ws_bytes,
                    void* stream) {
  return decode_step(p, q, k, v, kbar, out, row_count, col_idx, block_mass, ws, ws_bytes, false, stream);
}

rr_status rr_decode_noalloc(const rr_problem* p, const void* q, const void* k, const void* v, const void* kbar,
                            void* out, int32_t* row_count, int32_t* col_idx, float* block_mass, void* stream) {
  return decode_step(p, q, k, v, kbar, out, row_count, col_idx, block_mass, nullptr, 0, true, stream);
}

rr_status rr_decode_attend(const rr_problem* p, const void* q, const void* k, const void* v, const int32_t* row_count,
                           const int32_t* col_idx, void* out, void* ws, size_t ws_bytes, void* stream) {
  rr::Geometry g;
  rr_status s = make_geometry(p, &g);
  if (s != RR_OK) return s;
  if (!q || !k || !v || !out || !row_count || !col_idx) return RR_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(row_count) ||
      !aligned16(col_idx))
    return RR_ERR_INVALID_ARG;
  const DecodeWorkspace w = decode_layout(g);
  if (!ws || !aligned16(ws) || ws_bytes < w.total) return RR_ERR_WORKSPACE;
  uint8_t* base = static_cast<uint8_t*>(ws);
  hipStream_t st = static_cast<hipStream_t>(stream);
  uint8_t* sel = base + w.sel;
  hipError_t e = rr::launch_lists_to_flags(g, row_count, col_idx, sel, w.nbp, st);
  if (e == hipSuccess)
    e = rr::launch_decode_attn(g, q, k, v, row_count, col_idx, sel, w.nbp, reinterpret_cast<float*>(base + w.part),
                               out, st);
  return hip_status(e);
}

const char* rr_status_string(rr_status s) {
  switch (s) {
    case RR_OK: return "ok";
    case RR_ERR_INVALID_ARG: return "invalid argument";
    case RR_ERR_UNSUPPORTED: return "unsupported problem";
    case RR_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case RR_ERR_HIP: return "HIP runtime or launch error";
  }
  return "unknown status";
}

int32_t rr_version(void) { return 100; }

}  // extern "C"
