/*
 * kvevict.h -- C ABI of the MI355X (gfx950) KV-cache eviction round.
 *
 * One eviction round, run for every (layer, KV head) list of a batch:
 *   1. score every cache entry            kvevict_score_random / kvevict_score_weighted
 *   2. pin the protected prompt prefix    (part of every scorer and selector)
 *   3. select the entries to keep         kvevict_select_topk / kvevict_select_global
 *      (steps 1-3 fused: kvevict_select_random for the random draw and top-K,
 *      kvevict_score_select_global for the weighted score and global top-B)
 *   4. compact the kept bf16 K/V rows     kvevict_compact
 *
 * Sources of the definitions:
 *   [RA]  "Random Attention" blog summary (sungsoo.github.io, 2026-09-05):
 *         Algorithm 1 (random score, prompt = +inf, top-K per KV head, return
 *         the keep set); persistent budget K and recent buffer r = 64; the
 *         shared draw (one keep set for all heads); the engine's per-KV-head
 *         physical eviction with chronological compaction.
 *   [GS]  "GateSight" (signal-papers 2610.14754): problem statement (model-wide
 *         budget B = L*H*round(p*(n-prot)) exclusive of a protected prefix);
 *         Sec. 4.1 (signals of the up-to-six preceding GDN layers; log
 *         effective write log(beta*|v|)); Sec. 4.3 and Appendix G (kept
 *         entries moved to the front of each layer's pages); baselines
 *         paragraph (KVzip's global top-B over (layer, head, token) scores).
 *
 * Readings where the pages leave a step open (each function repeats its own):
 *   - rand: Philox4x64-10 (Salmon, Moraes, Dror, Shaw, SC 2011), key
 *     (seed, 0), counter (i/4, head, layer, request*2^32 + round); the score
 *     of slot i is the top 24 bits of output word i%4 times 2^-24, in [0, 1).
 *   - ranking: score descending; NaN ranks as -inf; -0 equals +0; among equal
 *     scores the lower position wins (global: the lower list*n + i).
 *   - round(): binary64 product, round half to even.
 *
 * Conventions shared by every entry point:
 *   - Pointers marked "device" are device memory owned by the caller; the
 *     library allocates nothing, frees nothing and keeps no state between
 *     calls, apart from kvevict_select_global_noalloc's static per-GPU array
 *     and the address of it that the first call on each device looks up.
 *     Host arrays are read during the call only.
 *   - All work is enqueued on `stream` (NULL = the default stream); nothing is
 *     synchronised; outputs are valid once the stream reaches that point.
 *   - Arguments are validated on the host before anything is enqueued; on an
 *     error status nothing has been enqueued and no output is touched.
 *     KVEVICT_ERR_HIP reports a failed launch (hipGetLastError).
 *   - One launch holds fewer than 2^32 work-items in a grid dimension.  A call
 *     whose grid would not fit returns KVEVICT_ERR_INVALID_ARG with nothing
 *     enqueued: from 2^22 lists where a list takes a 1024-thread workgroup
 *     (the global top-B; per-head top-K and its random form for lists of more
 *     than 15,360 candidates after the prompt), 2^23 for 512 threads (KeyDiff),
 *     2^24 for 256 (in-place compaction, the one-launch rounds, the page draw)
 *     and 2^25 for 128 (per-head top-K of shorter lists), and from 2^29 tokens
 *     for the weighted scores (a 512-thread workgroup per 64 tokens).
 *   - Empty batches (zero lists or groups) are valid and enqueue nothing.
 */
#ifndef KVEVICT_H
#define KVEVICT_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVEVICT_ABI_VERSION 1

typedef enum kvevict_status {
  KVEVICT_OK = 0,
  KVEVICT_ERR_INVALID_ARG = 1, /* a size, count or pointer is out of its documented range */
  KVEVICT_ERR_ALIGNMENT = 2,   /* a K/V base or stride is not 16-byte aligned */
  KVEVICT_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required */
  KVEVICT_ERR_UNSUPPORTED = 4, /* a valid request the library does not implement */
  KVEVICT_ERR_HIP = 5          /* the HIP runtime reported an error */
} kvevict_status;

typedef enum kvevict_layout {
  KVEVICT_LAYOUT_CONTIG = 0, /* one dense [capacity][D] slab per (group, head) list */
  KVEVICT_LAYOUT_PAGED = 1   /* a page pool [pages][page_size][H][D] and a page table */
} kvevict_layout;

/*
 * Describes one K or V store (K and V use the same description).  A group is
 * one (request, layer); a list is one (group, KV head), list = group*H + head.
 * Rows are D bf16 elements (2*D bytes, moved verbatim).
 *
 *   CONTIG: row t of list l at element  l*list_stride + t*D,  t < capacity.
 *   PAGED:  row t of (group g, head h) at element
 *             ((page_table[g*pt_ld + t/page_size]*page_size + t%page_size)*H + h)*D,
 *           t < pt_ld*page_size, page ids in [0, capacity).
 * [GS] Sec. 4.3: one block table per attention layer over a shared pool.
 */
typedef struct kvevict_kv_desc {
  int32_t layout;            /* kvevict_layout */
  int32_t head_dim;          /* D: elements per row, multiple of 8 (16-byte rows) */
  int32_t heads;             /* H: KV heads per group */
  int32_t page_size;         /* PAGED: tokens per page (>= 1); ignored for CONTIG */
  int64_t capacity;          /* CONTIG: rows per list; PAGED: pages in the pool */
  int64_t list_stride;       /* CONTIG: elements between lists, >= capacity*D, multiple of 8 */
  const int32_t* page_table; /* PAGED: device [num_groups][pt_ld] physical page ids */
  int64_t pt_ld;             /* PAGED: page-table entries per group (>= 1) */
} kvevict_kv_desc;

/*
 * Random Attention scores ([RA] Algorithm 1 "rand" and "prompt = +inf"; shared
 * draw paragraph).
 *
 * scores  device fp32, row `list` at scores + list*ld, ld >= n.
 *         Per-head draw: num_requests*L*H rows, list = (req*L + layer)*H + head.
 *         Shared draw (shared_draw != 0): num_requests*L rows, list = req*L + layer,
 *         drawn from the head-0 stream, so it equals head 0's per-head draw.
 * Row entries i < prot are +inf; entries prot <= i < n get the Philox draw of
 * (seed, req, layer, head, round, i) described above; entries >= n untouched.
 * Requires 0 <= prot <= n, num_requests < 2^32, L >= 1, H >= 1, lists < 2^31.
 */
kvevict_status kvevict_score_random(float* scores, int64_t ld, int64_t num_requests, int32_t L,
                                    int32_t H, int32_t n, int32_t prot, uint64_t seed,
                                    uint32_t round, int32_t shared_draw, hipStream_t stream);

/*
 * GateSight-style weighted scores ([GS] Sec. 4.1; log effective write).
 *
 *   s[l][h][t] = sum_{slot < win_count[l]} sum_{j < Hg}
 *                  w[((l*H + h)*w_slots + slot)*Hg + j] * ln(beta[e] * vnorm[e]),
 *   e = (win_begin[l] + slot)*sig_stride_g + t*sig_stride_t + j*sig_stride_j,
 *
 * for prot <= t < n, written to scores[(l*H + h)*ld + t]; +inf for t < prot.
 * Logs and the sum are taken in binary64 and rounded once to fp32.
 * beta, vnorm  device fp32 GDN signals (write gate, write magnitude); the
 *              planar layout [G][n][Hg] (strides n*Hg, Hg, 1) is the fast one.
 * w            device fp32 [L][H][w_slots][Hg] fixed per-GDN-head weights.
 * win_begin, win_count  HOST int32 [L]: the GDN layers read by attention
 *              layer l are [win_begin[l], win_begin[l] + win_count[l]) within
 *              [0, G); win_count[l] <= w_slots <= 64.
 * Requires L <= 64, H >= 1, Hg >= 1, 0 <= prot <= n, ld >= n.
 */
kvevict_status kvevict_score_weighted(float* scores, int64_t ld, const float* beta,
                                      const float* vnorm, int64_t sig_stride_g,
                                      int64_t sig_stride_t, int64_t sig_stride_j, const float* w,
                                      int32_t w_slots, const int32_t* win_begin,
                                      const int32_t* win_count, int32_t L, int32_t H, int32_t G,
                                      int32_t Hg, int32_t n, int32_t prot, hipStream_t stream);

/*
 * KeyDiff scores (GateSight Sec. 5.1, baselines paragraph).  A key scores
 * minus its cosine to its head's mean key (keys not normalised first), so a
 * flat per-head budget in kvevict_select_topk keeps the keys that differ most
 * from the mean.
 *
 * For every list (group g, head h), list = g*H + h, with its n keys in the
 * store `keys` (contiguous or paged, see kvevict_kv_desc; values are not read):
 *     scores[list*ld + i] = -cos(k_i, mean of k_0 .. k_{n-1})   for i >= prot,
 *                           +inf                                for i <  prot,
 * computed as -dot / (sqrt(|k_i|^2) * sqrt(|mean|^2)) in binary64 (IEEE square
 * roots and division) and rounded once to fp32.  Precision: the sums run in
 * another order than a plain loop's, so before that rounding the cosine may
 * differ from a plain loop's binary64 value x by at most about
 * 2^-53 * (D + n * |sum_i |k_i|| / |sum_i k_i|) (a few 1e-13 for N(0,1) keys
 * at n = 1088, D = 128); the score is fp32(-x), or its neighbour one fp32 ulp
 * away when -x lies within that bound of a midpoint between two fp32 values.
 * A key or a mean of norm zero gives cos = 0; a zero score is written as +0.
 * A paged row whose page id falls outside the pool reads as zeros.
 * Requires D = head_dim in {8, 16, 32, ..., 512}, 0 <= prot <= n <= rows of a
 * list, n * D / 8 < 2^31, ld >= n, num_groups*H < 2^23 (one workgroup per list,
 * fewer than 2^32 work-items per launch).  KVEVICT_ERR_UNSUPPORTED for other D.
 */
kvevict_status kvevict_score_keydiff(float* scores, int64_t ld, const kvevict_kv_desc* keys,
                                     const void* k_cache, int64_t num_groups, int32_t n,
                                     int32_t prot, hipStream_t stream);

/*
 * Pin + per-head top-K ([RA] Algorithm 1: prompt = +inf, topk, return keep).
 *
 * For each of num_lists lists (row at scores + list*ld): keeps [0, prot) and
 * the K - prot best of [prot, n) in the ranking above, and writes the K kept
 * indices in increasing order to kept_idx[list*kept_ld + j], j < K.  The
 * result does not depend on the scores stored at [0, prot).
 * Requires 0 <= prot <= K <= n, ld >= n, kept_ld >= K.
 */
kvevict_status kvevict_select_topk(int32_t* kept_idx, int64_t kept_ld, const float* scores,
                                   int64_t ld, int64_t num_lists, int32_t n, int32_t K,
                                   int32_t prot, hipStream_t stream);

/*
 * Random scores and per-list top-K in one launch ([RA] Algorithm 1: a random
 * score per entry, the prompt pinned, top-K per KV head, the keep set
 * returned).  kept_idx equals what kvevict_score_random (same seed, round, L,
 * H and draw mode) followed by kvevict_select_topk (K, prot) produce, but the
 * scores are drawn on chip and never stored.
 * kept_idx  device int32 out [lists][kept_ld], kept_ld >= K; lists and their
 *           numbering as in kvevict_score_random.
 * Requires 0 <= prot <= K <= n, num_requests < 2^32, L >= 1, H >= 1, lists < 2^31.
 */
kvevict_status kvevict_select_random(int32_t* kept_idx, int64_t kept_ld, int64_t num_requests,
                                     int32_t L, int32_t H, int32_t n, int32_t K, int32_t prot,
                                     uint64_t seed, uint32_t round, int32_t shared_draw,
                                     hipStream_t stream);

/*
 * Pin + per-layer top-K_l (GateSight Sec. 4.2 and Appendix G: every KV head of
 * attention layer l keeps the protected prefix plus K_l entries, so a layer's
 * kept cache is a dense prefix of K_l + prot rows per head).
 *
 * Groups are (request, layer) pairs, group = request*L + layer; list
 * (group, head) = group*H + head has its scores at scores + list*ld.  Each
 * list keeps [0, prot) and the layer_budget[group % L] best of [prot, n) in the
 * ranking above, writes the kept indices in increasing order to
 * kept_idx[list*kept_ld + j] and its count prot + layer_budget[layer] to
 * kept_count[list] (device int32 [num_groups*H]); entries beyond the count are
 * untouched.
 * layer_budget  HOST int32 [L] (for example from kvevict_layer_power_budget),
 *               each in [0, n - prot].
 * Requires 1 <= L <= 64, num_groups a multiple of L, 0 <= prot <= n, ld >= n,
 * kept_ld >= prot + max(layer_budget), num_groups*H < 2^31.
 */
kvevict_status kvevict_select_topk_layers(int32_t* kept_idx, int64_t kept_ld, int32_t* kept_count,
                                          const float* scores, int64_t ld, int64_t num_groups,
                                          int32_t L, int32_t H, int32_t n, int32_t prot,
                                          const int32_t* layer_budget, hipStream_t stream);

/*
 * Gate-proportional per-layer budgets (GateSight Sec. 4.2: layer l keeps K_l
 * entries per head in proportion to its gate weight w_l, with the model-wide
 * total of a flat allocation; Appendix G, layer_power_budget: integerised by
 * largest remainder so that the layers' budgets sum to L*round(p*n_body); the
 * protected prefix is kept in addition).  Host only; enqueues nothing.
 *
 * gate    HOST float [L], positive and finite, spanning at most 2^40.
 * n_body  candidates per list (n - prot); p in [0, 1].
 * budget  HOST int32 [L] out: K_l.
 * The shares T*w_l/sum(w) are computed exactly on the float gates; equal
 * remainders go to the lower layer; a layer whose share passes n_body keeps
 * n_body and the others share what is left, in proportion.
 */
kvevict_status kvevict_layer_power_budget(const float* gate, int32_t L, int32_t n_body, double p,
                                          int32_t* budget);

/*
 * Shared list scores of a layer (GateSight Appendix H: the KV heads of a layer
 * share one kept list, ranked by the larger of their per-head scores).
 *
 * For every group g < num_groups and position i < n:
 *     shared[g*shared_ld + i] = scores[(g*H + h)*ld + i]  for the head h whose
 * score ranks best (NaN as -inf, -0 equal to +0; the lowest such head, whose
 * bits are copied).  The shared rows then feed kvevict_select_topk as one list
 * per group and kvevict_compact with idx_lists_per_group = 1.
 * Requires H >= 1, ld >= n, shared_ld >= n, num_groups*H < 2^31.
 */
kvevict_status kvevict_reduce_max_heads(float* shared, int64_t shared_ld, const float* scores,
                                        int64_t ld, int64_t num_groups, int32_t H, int32_t n,
                                        hipStream_t stream);

/*
 * Pin + model-wide top-B ([GS] problem statement: B = L*H*round(p*(n-prot))
 * exclusive of the protected prefix; KVzip-style global top-B).
 *
 * B = num_lists * round_half_even(p * (n - prot)).  Keeps [0, prot) of every
 * list plus the B best non-prompt entries over all lists (ties: lower
 * list*n + i), then writes kept_count[list] and the kept indices of each list
 * in increasing order to kept_idx[list*kept_ld + j], j < kept_count[list];
 * entries beyond the count are untouched.
 * budget_out  optional HOST pointer receiving B.
 * workspace   device scratch.  Two-phase protocol: with workspace == NULL the
 *             call writes the required size to *workspace_bytes and returns
 *             KVEVICT_OK without enqueuing anything; otherwise *workspace_bytes
 *             must hold at least that size.  The workspace is overwritten.
 * Requires 0 <= prot <= n, 0 <= p <= 1, ld >= n, kept_ld >= n, num_lists*n < 2^31.
 */
kvevict_status kvevict_select_global(int32_t* kept_idx, int64_t kept_ld, int32_t* kept_count,
                                     int64_t* budget_out, const float* scores, int64_t ld,
                                     int64_t num_lists, int32_t n, int32_t prot, double p,
                                     void* workspace, size_t* workspace_bytes,
                                     hipStream_t stream);

/*
 * kvevict_select_global without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  It allocates nothing: its workspace is a
 * static device array inside the library, KVEVICT_SELECT_GLOBAL_NOALLOC_BYTES
 * bytes, one copy per GPU, held until the process ends; its address is looked
 * up on the first call on each device (hipGetSymbolAddress, with that device
 * current), so the stream must belong to the current device.
 *
 * Arguments, result and validation as kvevict_select_global.  A call whose
 * workspace (the size kvevict_select_global's query reports) would exceed
 * KVEVICT_SELECT_GLOBAL_NOALLOC_BYTES returns KVEVICT_ERR_WORKSPACE, nothing
 * enqueued.  65,536 items fit, an item being a run of up to 8,192 of a list's
 * candidates [prot, n) (e.g. 1,024 lists of 524,288 candidates).
 * KVEVICT_ERR_HIP if the array's address cannot be found.  Every call on one
 * GPU shares that GPU's array and leaves its contents behind (the next call
 * clears what it needs), so calls that overlap in time on one GPU -- on
 * different streams, or from different threads -- race and must be ordered by
 * the caller.
 */
#define KVEVICT_SELECT_GLOBAL_NOALLOC_BYTES 1086208
kvevict_status kvevict_select_global_noalloc(int32_t* kept_idx, int64_t kept_ld,
                                             int32_t* kept_count, int64_t* budget_out,
                                             const float* scores, int64_t ld, int64_t num_lists,
                                             int32_t n, int32_t prot, double p,
                                             hipStream_t stream);

/*
 * Weighted score and pin + model-wide top-B in one call ([GS] Sec. 4.1 and
 * problem statement; KVzip-style global top-B): the results of
 * kvevict_score_weighted on its arguments followed by kvevict_select_global
 * over its L*H lists (list = l*H + h), bit for bit.  The scorer also adds the
 * scores it writes to the select's first radix level, so the select reads
 * the scores one time fewer and skips one launch.
 * Arguments are those of the two calls: scores and ld are the scores buffer
 * the scorer writes and the select reads; workspace follows
 * kvevict_select_global's two-phase protocol with num_lists = L*H (the same
 * size as there); budget_out (optional, HOST) receives B.
 * Requires what both calls require.  Nothing is written when the arguments
 * are invalid.
 */
kvevict_status kvevict_score_select_global(
    int32_t* kept_idx, int64_t kept_ld, int32_t* kept_count, int64_t* budget_out, float* scores,
    int64_t ld, const float* beta, const float* vnorm, int64_t sig_stride_g,
    int64_t sig_stride_t, int64_t sig_stride_j, const float* w, int32_t w_slots,
    const int32_t* win_begin, const int32_t* win_count, int32_t L, int32_t H, int32_t G,
    int32_t Hg, int32_t n, int32_t prot, double p, void* workspace, size_t* workspace_bytes,
    hipStream_t stream);

/*
 * Chronological compaction ([RA] per-KV-head physical eviction, chronological
 * compaction; [GS] Sec. 4.3 kept entries to the front of the layer's pages).
 *
 * For every group g < num_groups, head h < H and j < count:
 *     K_dst row (g, h, j) = K_src row (g, h, idx[j])   and the same for V,
 * with idx = kept_idx + (g*idx_lists_per_group + (idx_lists_per_group == 1 ? 0 : h))*kept_ld
 * and count = kept_count ? kept_count[that index list] : K.
 * idx_lists_per_group is H (one index list per KV head) or 1 (shared draw:
 * one list applied to every head of the group).  Out of place: no byte of
 * k_dst or v_dst may lie in k_src's or v_src's extent, nor k_dst's in v_dst's,
 * else KVEVICT_ERR_INVALID_ARG (the two sources are only read and may overlap).
 * A store's extent follows its descriptor: CONTIG ((num_groups*H - 1)*list_stride
 * + capacity*D)*2 bytes from its base, PAGED the pool, capacity*page_size*H*D*2
 * bytes.  Destination rows >= count are untouched.
 * src, dst     host descriptors (see kvevict_kv_desc), same D and H.
 * k_src ...    device bf16 stores, 16-byte aligned.
 * errors       optional device uint32 counter; each row whose index or page
 *              id falls outside its store is skipped and adds 1, and each
 *              index list whose count is outside [0, K] adds 1 and is clamped
 *              to that range.  May be NULL.
 * Requires K <= dst rows per list, kept_ld >= K, num_groups*H < 2^31.
 */
kvevict_status kvevict_compact(const kvevict_kv_desc* src, const void* k_src, const void* v_src,
                               const kvevict_kv_desc* dst, void* k_dst, void* v_dst,
                               const int32_t* kept_idx, int64_t kept_ld,
                               const int32_t* kept_count, int32_t K, int64_t num_groups,
                               int32_t idx_lists_per_group, uint32_t* errors,
                               hipStream_t stream);

/*
 * Whole-page copy between page pools (GateSight Sec. 4.3: the cache is a pool
 * of fixed-size blocks behind per-layer block tables; a block moves as a unit).
 *
 * For i < count:  K_dst page dst_ids[i] = K_src page src_ids[i], and the same
 * for V, a page being page_bytes bytes at byte offset id*page_bytes of its
 * pool.  It is the paged gather with every slot of each page kept in order and
 * no per-row index: over the same tables it is the copy ceiling of
 * kvevict_compact on paged stores.
 * k_src, v_src   device pools of src_pages pages;  k_dst, v_dst  of dst_pages.
 * src_ids, dst_ids  device int32 [count]; a pair with an id outside its pool
 *                is skipped and adds 1 to *errors (optional device uint32).
 * Requires page_bytes > 0 and a multiple of 16 (KVEVICT_ERR_ALIGNMENT), 16-byte
 * aligned pools, and no destination byte in either source pool nor in the
 * other destination pool (KVEVICT_ERR_INVALID_ARG).  Destination pages listed
 * twice race.
 */
kvevict_status kvevict_copy_pages(const void* k_src, const void* v_src, int64_t src_pages,
                                  const int32_t* src_ids, void* k_dst, void* v_dst,
                                  int64_t dst_pages, const int32_t* dst_ids, int64_t count,
                                  int64_t page_bytes, uint32_t* errors, hipStream_t stream);

/*
 * kvevict_compact with a workspace: the same result, bit for bit, for callers
 * that can provide device scratch.  With a paged destination whose pages the
 * gather writes whole (16-token pages of H*D = 1024 elements, D = 128 and
 * H = 8 among others) and a pool at most four times the pages written, the
 * gather visits the destination pages in increasing physical order, each of
 * the GPU's eight dies (XCDs) walking one contiguous range of the pool,
 * instead of in page-table order: with the tables scattered over the pool, as
 * freshly allocated pages can be (GateSight Sec. 4.3, block tables over a
 * shared pool), this keeps the writes of the workgroups in flight close
 * together.  The order comes from two small kernels that write each page's
 * work item into its slot of the workspace; a page id outside the pool, or
 * one that two items name, makes the gather fall back to table order (such a
 * call is invalid anyway: its rows are skipped and counted as in
 * kvevict_compact).  Other stores take kvevict_compact's path.
 *
 * workspace  device scratch, 256-byte aligned, apart from the four stores.
 *            Two-phase protocol: with workspace == NULL the call writes the
 *            size it needs (dst->capacity*4 bytes plus 256, rounded up to 256;
 *            0 for a contiguous destination) to *workspace_bytes and returns
 *            KVEVICT_OK; otherwise *workspace_bytes must hold at least that
 *            size (KVEVICT_ERR_WORKSPACE).  Overwritten by each call.
 * Other arguments, requirements and errors as kvevict_compact.
 */
kvevict_status kvevict_compact_ordered(const kvevict_kv_desc* src, const void* k_src,
                                       const void* v_src, const kvevict_kv_desc* dst,
                                       void* k_dst, void* v_dst, const int32_t* kept_idx,
                                       int64_t kept_ld, const int32_t* kept_count, int32_t K,
                                       int64_t num_groups, int32_t idx_lists_per_group,
                                       uint32_t* errors, void* workspace,
                                       size_t* workspace_bytes, hipStream_t stream);

/*
 * In-place chronological compaction with a free-page list (GateSight Sec. 4.3
 * and Appendix G: each layer moves the entries it keeps to the front of its
 * own pages, and the freed tail blocks return to the pool, which releases
 * their memory).
 *
 * For every group g < num_groups, head h < H and j < count, in place:
 *     K row (g, h, j) <- K row (g, h, idx[j])   and the same for V,
 * with idx and count chosen as in kvevict_compact.  Each index list must be
 * strictly increasing (as the selections produce), so idx[j] >= j and rows
 * only move towards the front; rows with idx[j] == j are not touched.  Rows
 * at and beyond count keep whatever they held (stale).
 * n       rows of each list in use before the call (count <= K <= n).
 * PAGED:  the group's pages ceil(count_max / page_size) .. ceil(n / page_size) - 1,
 *         count_max the largest count among the group's index lists, are
 *         appended to freed_pages (device int32, room for num_groups *
 *         ceil(n / page_size) ids) at offsets taken with an atomic add on
 *         *freed_count (device uint32, not reset by the call), in an order
 *         that may differ from call to call.  The page table itself is read
 *         only: the caller shortens its block table to the kept pages.
 *         CONTIG: freed_pages and freed_count are ignored (may be NULL).
 * errors  optional device counter: each row whose index is below its slot or
 *         outside the store, or whose page id is invalid, is skipped and adds 1.
 *         Counts outside [0, K] are clamped.
 * Limits: num_groups * H < 2^31, n * head_dim / 8 <= 2^30 and, paged,
 * num_groups * ceil(n / page_size) < 2^32 (free-list offsets), else
 * KVEVICT_ERR_INVALID_ARG.  The K and V extents (as in kvevict_compact) must
 * be disjoint, else KVEVICT_ERR_INVALID_ARG.  Calls on the same store must not
 * overlap in time.
 */
kvevict_status kvevict_compact_inplace(const kvevict_kv_desc* store, void* k, void* v,
                                       const int32_t* kept_idx, int64_t kept_ld,
                                       const int32_t* kept_count, int32_t K, int32_t n,
                                       int64_t num_groups, int32_t idx_lists_per_group,
                                       int32_t* freed_pages, uint32_t* freed_count,
                                       uint32_t* errors, hipStream_t stream);

/*
 * One-launch Random Attention round with in-place compaction ([RA] Algorithm 1:
 * random scores, the prompt pinned, top-K per KV head, the keep set returned;
 * [RA] engine paragraph: per-KV-head physical eviction with chronological
 * compaction; [GS] Sec. 4.3 and Appendix G: kept entries move to the front of
 * their own pages and the freed tail blocks return to the pool).
 *
 * The result equals kvevict_score_random (same seed, round, L and draw mode)
 * followed by kvevict_select_topk (K, prot) and kvevict_compact_inplace (K, n),
 * but no score or index buffer is read from or written to memory.
 * Groups g = req*L + layer for req < num_requests; heads from the store.
 * kept_idx    optional device int32 out: the keep set of each list, increasing,
 *             row list*kept_ld (list = g*H + h per head, g when shared), kept_ld >= K.
 * shared_draw != 0: one keep set per group, the head-0 draw, applied to every head.
 * freed_pages, freed_count, errors: as in kvevict_compact_inplace (every list
 *             keeps K, so pages ceil(K / page_size) .. ceil(n / page_size) - 1 are freed).
 * Requires 0 <= prot <= K <= n <= rows of a list, num_requests < 2^32, L >= 1;
 * KVEVICT_ERR_UNSUPPORTED when (n - prot) + K > 15360 (keys and indices are held on chip).
 * Limits of kvevict_compact_inplace apply, disjoint K and V extents included.
 * Calls on the same store must not overlap in time.
 */
kvevict_status kvevict_evict_random_inplace(const kvevict_kv_desc* store, void* k, void* v,
                                           int64_t num_requests, int32_t L, int32_t n, int32_t K,
                                           int32_t prot, uint64_t seed, uint32_t round,
                                           int32_t shared_draw, int32_t* kept_idx,
                                           int64_t kept_ld, int32_t* freed_pages,
                                           uint32_t* freed_count, uint32_t* errors,
                                           hipStream_t stream);

/*
 * Page-granular Random Attention eviction applied as page-table edits ([RA]
 * Algorithm 1 over the blocks of a paged cache: a random score per block, the
 * prompt pinned, the top blocks kept; [GS] Sec. 4.3: one block table per
 * attention layer over a shared pool, freed blocks back to the pool).
 *
 * For the paged layout of kvevict_kv_desc (token-major pages of page_size
 * slots holding every KV head), one list per group g = req*L + layer over its
 * P = n / page_size pages:
 *   score of page b   = the shared (head-0) kvevict_score_random draw of slot
 *                       b*page_size of group g (same seed, round);
 *   kept pages        = pages 0 .. ceil(prot/page_size)-1 (they hold the prompt)
 *                       plus the K/page_size - ceil(prot/page_size) other pages
 *                       with the largest scores, ties to the lower page, in
 *                       increasing order;
 *   page_table row g  : entry j < K/page_size becomes the old entry of the
 *                       j-th kept page, entries K/page_size .. P-1 become -1,
 *                       entries >= P are untouched (edited in place);
 *   freed_pages       : the old entries of the evicted pages, in page order,
 *                       appended at an offset taken with an atomic add on
 *                       *freed_count (not reset by the call; groups may land in
 *                       any order).  Room: num_groups * (P - K/page_size).
 * Token slot t of a kept page keeps its offset t % page_size, so no K/V byte
 * moves: reading the store through the new table equals the token gather of the
 * kept pages' slots.
 * page_table  device int32 [num_groups][pt_ld], pt_ld >= P.
 * kept_pages  optional device int32 out [num_groups][kept_ld], kept_ld >= K/page_size.
 * Requires page_size >= 1, n and K multiples of page_size, 0 <= prot <= K <= n,
 * num_requests < 2^32, L >= 1; KVEVICT_ERR_UNSUPPORTED when
 * (P - ceil(prot/page_size)) + 2P + K/page_size > 15360 (the group is held on chip);
 * KVEVICT_ERR_INVALID_ARG when num_groups * (P - K/page_size) >= 2^32.
 * Calls on the same table must not overlap.
 */
kvevict_status kvevict_evict_pages_random(int32_t* page_table, int64_t pt_ld, int32_t page_size,
                                         int64_t num_requests, int32_t L, int32_t n, int32_t K,
                                         int32_t prot, uint64_t seed, uint32_t round,
                                         int32_t* kept_pages, int64_t kept_ld,
                                         int32_t* freed_pages, uint32_t* freed_count,
                                         hipStream_t stream);

/* Human-readable name of a status code (static storage). */
const char* kvevict_status_string(kvevict_status status);

/* KVEVICT_ABI_VERSION of the built library. */
int32_t kvevict_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KVEVICT_H */
