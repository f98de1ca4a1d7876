/*
 * rr_attn.h -- C ABI of the MI355X (gfx950) RRAttention prefill library.
 *
 * The operation is the prefill hot path of "RRAttention: Dynamic Block Sparse
 * Attention via Per-Head Round-Robin Shifts for Long-Context Inference"
 * (abstract and TL;DR; the three stages of its Figure 2 caption):
 *   1. pattern search -- head h samples the query at in-stride offset h mod S
 *      of every stride of S tokens, scores it against stride-aggregated keys
 *      (an O(L^2/S^2) estimate), turns each sampled query's scores into a
 *      softmax, sums it into key blocks of B tokens and averages over the
 *      query block's samples, then keeps each query-block row's heaviest key
 *      blocks until their cumulative mass reaches tau (adaptive Top-tau); the
 *      last query block is statically kept whole;
 *   2. block-sparse attention -- exact softmax attention of every query over
 *      the keys of its row's selected blocks (key <= query when causal).
 *
 * Conventions shared by every entry point
 *   - Batch 1, one layer. Q and O are [L][Hq][d], K and V are [L][Hkv][d],
 *     row-major and contiguous, in the dtype named by the problem (bfloat16
 *     or float32). Query head h uses KV head h / (Hq / Hkv) (grouped-query
 *     attention with consecutive grouping).
 *   - nb = ceil(L / B) query (and key) blocks; when B does not divide L the
 *     last block is short (L - (nb - 1) B tokens), and likewise the last
 *     stride of S tokens (its pooled key is the mean of the keys it has).
 *     Block lists: row_count is int32
 *     [Hq][nb], col_idx is int32 [Hq][nb][nb]; row (h, i) selects key blocks
 *     col_idx[h][i][0 .. row_count[h][i]) in strictly ascending order; the
 *     remaining entries are unspecified.
 *   - All tensor arguments are DEVICE pointers, 16-byte aligned. The caller
 *     owns every buffer; the library allocates and frees nothing and keeps no
 *     state between calls (it is re-entrant). `stream` is a hipStream_t
 *     (NULL = the default stream); all work is enqueued asynchronously on it
 *     and nothing is synchronised: the caller synchronises before reading
 *     outputs on the host.
 *   - Errors: arguments are validated on the host before anything is
 *     enqueued; an invalid or unsupported problem returns RR_ERR_INVALID_ARG
 *     or RR_ERR_UNSUPPORTED and launches nothing. A HIP launch failure
 *     returns RR_ERR_HIP (outputs are then undefined). Nothing throws across
 *     the ABI.
 *
 * Supported problems: dtype bf16 or fp32; d in {64, 128}; B in {64, 128};
 * S a power of two with r = B / S in {2, 4, 8, 16, 32}; any L >= 1 with
 * ceil(L / B) <= 8192; Hq a multiple of Hkv; 0 < tau <= 1 (tau = 1 keeps every
 * candidate block); causal 0 or 1.
 */
#ifndef RR_ATTN_H
#define RR_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  RR_OK = 0,
  RR_ERR_INVALID_ARG = 1, /* null/misaligned pointer, bad size, tau out of (0, 1], ... */
  RR_ERR_UNSUPPORTED = 2, /* a valid problem outside the supported set above */
  RR_ERR_WORKSPACE = 3,   /* ws is NULL or ws_bytes < rr_workspace_bytes(p) */
  RR_ERR_HIP = 4          /* a HIP runtime or launch error */
} rr_status;

typedef enum { RR_BF16 = 0, RR_FP32 = 1 } rr_dtype;

typedef struct {
  int32_t L;      /* tokens */
  int32_t Hq;     /* query heads */
  int32_t Hkv;    /* key/value heads, divides Hq */
  int32_t d;      /* head dimension */
  int32_t S;      /* stride of the round-robin sampling and key aggregation */
  int32_t B;      /* block size of the sparse pattern (query and key blocks) */
  float tau;      /* Top-tau mass threshold, 0 < tau <= 1 */
  int32_t causal; /* 1: key <= query (at stride, block and token level); 0: none */
  int32_t dtype;  /* rr_dtype of Q, K, V and O */
} rr_problem;

/* Bytes of device workspace the calls below need for problem p (0 if p is
 * invalid or unsupported). One workspace serves every entry point. */
size_t rr_workspace_bytes(const rr_problem* p);

/*
 * Stage 1, the round-robin pattern search (abstract: sampling positions
 * rotated over the heads, keys aggregated per stride, the adaptive Top-tau
 * cut; TL;DR: the last query block is always kept whole).
 *   q, k        device inputs, [L][Hq][d] and [L][Hkv][d] in p->dtype.
 *   row_count   device output int32 [Hq][nb].
 *   col_idx     device output int32 [Hq][nb][nb] (ascending per row).
 *   block_mass  optional device output float [Hq][nb][nb] (NULL to skip):
 *               the block masses m[h][i][j] of the searched rows (zero for
 *               non-candidate blocks and for the unsearched last row).
 *   ws          device workspace of ws_bytes >= rr_workspace_bytes(p).
 * Pooled keys are the stride mean computed in float32 and rounded to the
 * input dtype; scores use scale 1/sqrt(d); sampled stride s sees key strides
 * t <= s when causal. Row i < nb-1 keeps the blocks of its (mass descending,
 * index ascending) order while the mass before a block is < tau * row total.
 */
rr_status rr_pattern_search(const rr_problem* p, const void* q, const void* k,
                            int32_t* row_count, int32_t* col_idx, float* block_mass,
                            void* ws, size_t ws_bytes, void* stream);

/*
 * Stage 2, block-sparse attention over given block lists (abstract: only the
 * selected blocks, about half of them, are computed). The lists may come from
 * rr_pattern_search or any other source; each row must be non-empty,
 * ascending, < nb, and (causal) <= its query block index: rows breaking this
 * give undefined output (the library does not read lists back to the host).
 *   q, k, v     device inputs in p->dtype; out: device output [L][Hq][d] in p->dtype.
 *   ws          device workspace of rr_workspace_bytes(p) bytes (bf16: a
 *               copy of V re-laid out as one channels-by-keys tile per key
 *               block, and the counters of the attention's work queues; fp32
 *               needs none of it); calls that overlap in time need
 *               workspaces of their own.
 * Scale 1/sqrt(d); with p->causal, key y is visible to query x iff y <= x.
 * p->S and p->tau are not used but must be valid.
 * The kernel is chosen from the problem alone: bf16 with B = 128 runs two
 * query heads per workgroup in a ping-pong schedule (with an odd count of
 * query heads per KV head, one included, the last head of every KV head is
 * paired with itself over two adjacent query blocks in the same launch);
 * bf16 with B = 64 runs one query head per workgroup; fp32 runs on the fp32
 * matrix cores.
 */
rr_status rr_block_sparse_attn(const rr_problem* p, const void* q, const void* k, const void* v,
                               const int32_t* row_count, const int32_t* col_idx, void* out,
                               void* ws, size_t ws_bytes, void* stream);

/*
 * Stage 1 with a threshold per query head (a serving extension; the pages use
 * one tau): tau_per_head is a DEVICE float array [Hq]; head h keeps the
 * blocks of its rows up to tau_per_head[h] of the row total. A value that is
 * NaN or outside (0, 1] keeps every candidate block. p->tau must still be
 * valid and is not used. Other arguments as rr_pattern_search.
 */
rr_status rr_pattern_search_heads(const rr_problem* p, const void* q, const void* k, const float* tau_per_head,
                                  int32_t* row_count, int32_t* col_idx, float* block_mass, void* ws,
                                  size_t ws_bytes, void* stream);

/* Both stages back to back on one stream: search, then attention over the
 * lists it produced (row_count / col_idx are outputs, as in stage 1). */
rr_status rr_prefill(const rr_problem* p, const void* q, const void* k, const void* v, void* out,
                     int32_t* row_count, int32_t* col_idx, void* ws, size_t ws_bytes,
                     void* stream);

/*
 * Mass recall of a selection against full attention: how much of the exact
 * full-attention softmax mass the selected blocks hold (Figure 4 and Figure 5
 * captions: full-attention ground truth next to the selected blocks). For
 * query x of head h, r(x) is the share of its softmax over every admissible
 * key (key <= x when causal; scale 1/sqrt(d)) that falls on keys of the
 * row's selected blocks; recall[h][i] is the mean of r(x) over the B queries
 * of query block i.
 *   q, k        device inputs [L][Hq][d] and [L][Hkv][d] in p->dtype.
 *   row_count, col_idx  device block lists as for rr_block_sparse_attn
 *               (ascending; entries that break the order are not counted).
 *   recall      device output float [Hq][nb].
 * Cost: the scores of every candidate block (a dense causal Q K^T), about half
 * the FLOPs of dense attention. p->S and p->tau are not used but must be valid.
 * Needs no workspace.
 */
rr_status rr_mass_recall(const rr_problem* p, const void* q, const void* k, const int32_t* row_count,
                         const int32_t* col_idx, float* recall, void* stream);

/*
 * Shared mask per KV head: a variant of the per-query-head masks above (the
 * pages select per head; this is not on them). For every KV head g and query
 * block i, the union of the blocks selected by the G = Hq / Hkv query heads
 * of g in row i, written in ascending order to row (h, i) of every head h of
 * g, so all heads of a KV head compute the same blocks.
 *   row_count, col_idx                device input lists (format above).
 *   shared_row_count, shared_col_idx  device output lists, same format; they
 *                                     must not overlap the inputs.
 * The outputs can be passed to rr_block_sparse_attn and rr_mass_recall as
 * they are. p->S and p->tau are not used but must be valid. No workspace.
 */
rr_status rr_share_group_lists(const rr_problem* p, const int32_t* row_count, const int32_t* col_idx,
                               int32_t* shared_row_count, int32_t* shared_col_idx, void* stream);

/*
 * A batch of independent sequences of different lengths packed along the
 * token axis, without padding (varlen prefill). p describes every sequence
 * except its length: p->L must equal the sum of the n_seq lengths in
 * seq_lens (a HOST array, each entry >= 1; a length need not be a multiple
 * of B). q, k, v and out are the packed tensors ([sum L_b][H][d]). The lists
 * of sequence b follow those of the sequences before it: row_count at entry
 * offset sum_{b'<b} Hq nb_b', col_idx at sum_{b'<b} Hq nb_b'^2, with
 * nb_b = ceil(L_b / B). Every sequence's slices must stay 16-byte aligned
 * (else RR_ERR_UNSUPPORTED). Where the problem has the head-pair kernel
 * (bf16, B = 128), the sequences run
 * longest first: one with at least 8 attention work items per compute unit
 * (about 16K tokens at the LLaMA-3.1-8B shape on 256 CUs) is searched and
 * attended in launches of its own, as rr_prefill would; the others are
 * searched and attended together, one launch per kernel per 32 sequences.
 * Otherwise each sequence is searched and attended in turn.
 * One workspace of rr_workspace_bytes_varlen bytes serves them all
 * (0 for an invalid batch). All lengths are checked before anything is
 * enqueued.
 */
size_t rr_workspace_bytes_varlen(const rr_problem* p, int32_t n_seq, const int32_t* seq_lens);
rr_status rr_prefill_varlen(const rr_problem* p, int32_t n_seq, const int32_t* seq_lens, const void* q,
                            const void* k, const void* v, void* out, int32_t* row_count, int32_t* col_idx,
                            void* ws, size_t ws_bytes, void* stream);

/*
 * Decode step: one new query per head against the KV cache (the TL;DR names
 * decode-stage sparsification as future work; this applies the prefill's
 * pieces to it). p->L is the cache length, the new token's own key and value
 * included at position L - 1; q is [Hq][d], k and v [L][Hkv][d], out [Hq][d],
 * all in p->dtype. Per query head: scores of q against every pooled cache key
 * (stride means as in rr_pattern_search, scale 1/sqrt(d)), one softmax over
 * the strides, summed into key blocks; the Top-tau prefix of the (mass desc,
 * index asc) order is kept plus the last block (the one holding the query),
 * and q attends to every key of the kept blocks (p->tau NaN or outside
 * (0, 1): every block). p->causal is not used. All pointers are device
 * memory owned by the caller; the calls are asynchronous on `stream`. Errors:
 * RR_ERR_INVALID_ARG for a NULL or unaligned (16-byte) required pointer,
 * RR_ERR_WORKSPACE for ws_bytes below rr_decode_workspace_bytes(p),
 * RR_ERR_UNSUPPORTED for shapes without kernels (as rr_prefill).
 *   kbar        optional device input [ceil(L/S)][Hkv][d] in p->dtype: the
 *               cache's pooled keys (rr_pool_keys), which a server can keep
 *               with its cache; NULL pools them here (one pass over K).
 *   row_count   device output int32 [Hq]; col_idx int32 [Hq][nb] (ascending).
 *   block_mass  optional device output float [Hq][nb] (NULL to skip).
 *   ws          rr_decode_workspace_bytes(p) bytes.
 */
size_t rr_decode_workspace_bytes(const rr_problem* p);
rr_status rr_decode(const rr_problem* p, const void* q, const void* k, const void* v, const void* kbar, void* out,
                    int32_t* row_count, int32_t* col_idx, float* block_mass, void* ws, size_t ws_bytes,
                    void* stream);

/* The attention stage of rr_decode on its own: q attends to every key of the
 * blocks in each head's list (row_count [Hq], col_idx [Hq][nb] int32 device
 * inputs; entries outside [0, nb) and repeats are ignored, the order does
 * not matter),
 * with the same kernels and results as rr_decode for the same lists. For
 * lists kept over several steps or chosen by the caller. ws as for rr_decode;
 * errors as rr_decode. */
rr_status rr_decode_attend(const rr_problem* p, const void* q, const void* k, const void* v, const int32_t* row_count,
                           const int32_t* col_idx, void* out, void* ws, size_t ws_bytes, void* stream);

/*
 * rr_decode for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation. Same
 * arguments, kernels and results as rr_decode, without ws / ws_bytes: the
 * workspace is a buffer the library owns, RR_DECODE_NOALLOC_MAX_WS bytes on
 * every GPU it runs on, held from the library's load until the process ends.
 * The call allocates nothing. A problem whose rr_decode_workspace_bytes(p)
 * exceeds RR_DECODE_NOALLOC_MAX_WS returns RR_ERR_WORKSPACE and launches
 * nothing (for the 8B-shaped layer, 32 query and 8 KV heads of 128 bf16
 * channels: every supported cache length with kbar given; up to about 245K
 * tokens with the keys pooled inside the call). Every call on one GPU
 * shares that GPU's buffer: calls that overlap in time on one GPU (other
 * streams, other threads) race and give undefined results; calls ordered on
 * one stream are safe. No state carries over between calls.
 */
#define RR_DECODE_NOALLOC_MAX_WS ((size_t)32 << 20)
rr_status rr_decode_noalloc(const rr_problem* p, const void* q, const void* k, const void* v, const void* kbar,
                            void* out, int32_t* row_count, int32_t* col_idx, float* block_mass, void* stream);

/* The pooled keys of rr_pattern_search's first step, on their own: kbar
 * [ceil(L/S)][Hkv][d] in p->dtype receives, per stride of S tokens (the last
 * possibly short), the float32 mean of its keys rounded to the dtype. */
rr_status rr_pool_keys(const rr_problem* p, const void* k, void* kbar, void* stream);

/* Static, NUL-terminated description of a status code. */
const char* rr_status_string(rr_status s);

/* Library version as MAJOR * 10000 + MINOR * 100 + PATCH. */
int32_t rr_version(void);

#ifdef __cplusplus
}
#endif

#endif /* RR_ATTN_H */
