/*
 * kdv.h -- C ABI of libkdv: DDTree tree-verify attention for MLA (absorbed form) on MI355X (gfx950).
 *
 * The operation (from "The Architecture of Diagnosis: How Three Threads of Inference Engineering
 * Converged in a Single Session", section "Phase 1: Custom CUDA Kernels", item 2): in the verify step
 * of DDTree speculative decoding, every node of the draft tree is evaluated in one pass.  Each node
 * attends over the KV cache under a visibility mask that follows the tree: the whole prefix, its
 * ancestors and itself.  The cache is MLA's compressed latent (kv_lora_rank latent + qk_rope rotary
 * elements per token per layer; "From Diagnosis to Deployment: Three Threads of Inference Engineering
 * for Kimi K2.6", section "The Second Thread: Pivoting to 200k Context"), stored with one token per
 * page so that accepted tokens can be committed non-contiguously ("The Architecture of Diagnosis...",
 * section "The Discrepancy That Revealed the Truth").  The latent projection is absorbed into the
 * attention: the key map W_UK is folded into the query and the value map W_UV is applied once to the
 * attention output, so no per-head key or value is ever materialised.
 *
 * For node t, head h (all arithmetic on bf16 inputs, fp32 accumulation):
 *   q_lat      = W_UK[h]^T q_nope[t,h]                                  (R)
 *   s_n        = sm_scale * (q_lat . c_kv[pt[n]] + q_rope[t,h] . k_pe[pt[n]])
 *   visible(n) = n < L  or  (n - L) is on the root-to-t path of the tree
 *   p          = softmax of s over the visible n;  o_lat = sum_n p_n c_kv[pt[n]]
 *   out[t,h]   = W_UV[h] o_lat                                           (Dv)
 *   lse[t,h]   = ln sum_{visible n} exp(s_n)
 *
 * Conventions shared by every entry point:
 *   - Memory is owned by the caller.  Device pointers are plain HIP device addresses; bf16 arrays are
 *     passed as uint16_t bit patterns.  The library never allocates, frees or keeps state between calls.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Every call only enqueues work on it and
 *     returns; device faults surface at the caller's next synchronisation.
 *   - Argument errors are detected on the host before anything is enqueued and returned as a negative
 *     kdv_status; nothing is launched in that case.
 *   - Row-major layouts; "[A][B]" means B is the contiguous dimension.
 */
#ifndef KDV_H
#define KDV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Model dimensions of one MLA attention layer.  Supported shapes:
 *   Kimi/DeepSeek shape: qk_nope 128, qk_rope 64, kv_lora_rank 512, v_head 128;
 *   tiny test shape:     qk_nope 32,  qk_rope 16, kv_lora_rank 64,  v_head 32;
 * with 1 <= num_heads <= 128.  sm_scale multiplies q.k (1/sqrt(qk_nope+qk_rope) for Kimi); it must be finite and
 * > 0 (KDV_ERR_SHAPE otherwise). */
typedef struct kdv_mla_dims {
  int32_t num_heads;
  int32_t qk_nope_dim;
  int32_t qk_rope_dim;
  int32_t kv_lora_rank;
  int32_t v_head_dim;
  float sm_scale;
} kdv_mla_dims;

typedef enum kdv_status {
  KDV_OK = 0,
  KDV_ERR_NULL = -1,      /* a required pointer is NULL                                         */
  KDV_ERR_SHAPE = -2,     /* T outside [1, 64], L < 0, L+T overflow, or unsupported dims          */
  KDV_ERR_TREE = -3,      /* parent array is not a rooted tree in topological order (device side) */
  KDV_ERR_ALIGN = -4,     /* a bf16/fp32 array or the workspace is not 16-byte aligned            */
  KDV_ERR_WORKSPACE = -5, /* workspace smaller than kdv_verify_workspace_bytes()                  */
  KDV_ERR_HIP = -6,       /* a HIP launch or query of this call failed (every entry point clears   */
                          /* HIP's per-thread last error before it launches, so an error left by  */
                          /* earlier work is not reported as this call's; it is not kept either)  */
  KDV_ERR_PAGE = -7       /* a page-table entry outside [0, pool_slots) (device side, KDV_DEBUG)  */
} kdv_status;

#define KDV_MAX_TREE_NODES 64
#define KDV_MAX_BATCH 16           /* requests per kdv_verify_mla_attn_batch call */
#define KDV_MAX_DRAFT_ENTRIES 4096 /* block x K entries of the drafter's top-K table */
#define KDV_WS_HEADER 256          /* bytes at the start of every verify workspace: the KDV_DEBUG status */
#define KDV_NOALLOC_SCRATCH_BYTES (32u << 20) /* device array behind kdv_verify_mla_attn_noalloc (32 MiB) */

/* Best-first construction of the draft tree on the device ("The Architecture of Diagnosis...", section
 * "Phase 1: Custom CUDA Kernels", item 1).
 *
 *   logp       : device float32 [block][K]: for each position d of the draft block, the log-probabilities of
 *                the drafter's K best tokens, in decreasing order (logp[d][0] >= logp[d][1] >= ...; finite
 *                or -inf, no NaN).  Positions are independent: a root path scores the float32 sum of its
 *                tokens' log-probabilities, added from the root down.
 *   tok        : device int32 [block][K], the tokens of logp.
 *   block, K   : 1 <= block <= 63, 1 <= K <= 64, block * K <= KDV_MAX_DRAFT_ENTRIES.
 *   budget     : maximum number of tree nodes, root included: 1 <= budget <= 64.
 *   root_token : device int32: the committed token at the root (e.g. kdv_tree_accept's next_token).
 *   parent     : device int32 [budget], written: the tree in node order; parent[0] = -1, parent[i] < i.
 *   tokens     : device int32 [budget], written: tokens[0] = *root_token; a node at depth d >= 1 carries a
 *                token of position d - 1.  Entries past *n_nodes are -1 in both arrays.
 *   n_nodes    : device int32, written: min(budget, 1 + nodes of the full K-ary tree of depth block).
 * Nodes join best-first: the highest-scoring candidate next, ties to the smaller depth, then the smaller
 * parent index, then the better rank; when a node joins, its next-ranked sibling and its best child become
 * candidates.  The tree is therefore the budget - 1 best nodes, in non-increasing score order, and its
 * parent array is valid input for kdv_build_tree_mask.
 * Host-side return: KDV_OK, KDV_ERR_NULL (a pointer is NULL), KDV_ERR_SHAPE (block, K or budget out of
 * range), KDV_ERR_ALIGN (a pointer not 4-byte aligned), KDV_ERR_HIP.  Nothing is allocated. */
int kdv_build_draft_tree(const float* logp, const int32_t* tok, int32_t block, int32_t K, int32_t budget,
                         const int32_t* root_token, int32_t* parent, int32_t* tokens, int32_t* n_nodes, void* stream);

/* Ancestor bitmask of the draft tree ("visibility mask that reflects the tree structure",
 * "The Architecture of Diagnosis...", section "Phase 1: Custom CUDA Kernels", item 2).
 *
 *   parent : device int32 [T].  parent[0] = -1 (node 0 is the root); parent[i] in [0, i) for i > 0,
 *            i.e. the nodes are in topological order, as a best-first tree builder emits them.
 *   T      : number of tree nodes, 1 <= T <= 64.
 *   mask   : device uint32 [T][W], W = (T + 31) / 32, written.  Bit (j % 32) of word j / 32 of row i is
 *            set iff node j is on the root-to-i path (i itself included); all other bits, including
 *            the padding above T, are zero.  Row i equals row parent[i] with bit i added.
 *   status : device int32, nullable.  The parent array lives on the device, so its validity is
 *            reported there: KDV_OK, or KDV_ERR_TREE if parent[0] != -1 or some parent[i] is outside
 *            [0, i).  An invalid row gets only its own bit; rows below it follow the rule above.
 * Host-side return: KDV_OK, KDV_ERR_NULL (parent or mask NULL), KDV_ERR_SHAPE (T out of range),
 * KDV_ERR_ALIGN (parent, mask or status not 4-byte aligned), KDV_ERR_HIP. */
int kdv_build_tree_mask(const int32_t* parent, int32_t T, uint32_t* mask, int32_t* status, void* stream);

/* Greedy acceptance of the verified draft tree: the longest accepted root path, selected on the device
 * ("The Architecture of Diagnosis...", section "Phase 1: Custom CUDA Kernels", item 3).
 *
 *   parent     : device int32 [T], as for kdv_build_tree_mask.  Node 0 is the root, whose token is
 *                already committed.
 *   tokens     : device int32 [T]; tokens[t] is node t's draft token (tokens[0] is not read).
 *   pred       : device int32 [T]; pred[t] is the target model's greedy prediction (argmax) after the
 *                prefix that ends at node t, e.g. from the verify pass's logits.
 *   T          : 1 <= T <= 64.
 *   path       : device int32 [T], written: the accepted root path as node indices, path[0] = 0, each
 *                next entry the child of the previous one whose draft token equals the previous node's
 *                prediction (the lowest index if several siblings carry it); entries past *n_path are -1.
 *   n_path     : device int32, written: number of nodes on the path (>= 1; accepted drafts = n_path - 1).
 *   next_token : device int32, written: pred[path[n_path - 1]], the target's own token after the accepted
 *                prefix.  The step commits tokens[path[1..n_path-1]] followed by next_token.
 *   status     : device int32, nullable: KDV_OK, or KDV_ERR_TREE for a malformed parent array (the mask's
 *                rules), in which case the path is the root alone.
 * Host-side return: KDV_OK, KDV_ERR_NULL (a required pointer is NULL), KDV_ERR_SHAPE (T out of range),
 * KDV_ERR_ALIGN (a pointer not 4-byte aligned), KDV_ERR_HIP.  Nothing is allocated. */
int kdv_tree_accept(const int32_t* parent, const int32_t* tokens, const int32_t* pred, int32_t T, int32_t* path,
                    int32_t* n_path, int32_t* next_token, int32_t* status, void* stream);

/* Bytes of device workspace kdv_verify_mla_attn needs for these dims, tree size T and prefix length L
 * on the current device (the split-KV plan depends on the device's compute-unit count).  Returns 0 if
 * the arguments are unsupported.  The environment variable KDV_SPLITS, if set, overrides the number of
 * KV splits; it must be the same when sizing and when calling. */
size_t kdv_verify_workspace_bytes(const kdv_mla_dims* d, int32_t T, int32_t L);

/* Tree-verify MLA attention for one layer (formula at the top of this file).
 *
 *   d          : dims (host pointer).
 *   q_nope     : device bf16 [T][H][Dn].
 *   q_rope     : device bf16 [T][H][Dr], already rotated (post-RoPE).
 *   w_uk       : device bf16 [H][Dn][R]; per head the key map k_nope = W_UK[h] c.
 *   w_uv       : device bf16 [H][Dv][R]; per head the value map v = W_UV[h] c.
 *   c_kv       : device bf16 pool [P][R] of latent rows.
 *   k_pe       : device bf16 pool [P][Dr] of rotary key rows (post-RoPE).
 *   pool_slots : P.  Every page_table entry must be in [0, P); this is the caller's contract and is not
 *                checked on the hot path.  With KDV_DEBUG set (to anything but "0") in the environment when
 *                the call is made, a one-workgroup kernel first checks every entry of the call's page table
 *                (pages are one token each: "The Architecture of Diagnosis...", section "The Discrepancy That
 *                Revealed the Truth") and writes KDV_OK or KDV_ERR_PAGE to the int32 at offset 0 of the
 *                workspace; on KDV_ERR_PAGE the verify kernels gather nothing and `out` (and `lse`, if given)
 *                are filled with NaN.  Also for the batched and prefix-only calls (their whole page table).
 *   page_table : device int32 [L+T]; logical position n -> pool slot.  Positions 0..L-1 are the prefix;
 *                position L+i holds tree node i's own latent row (already appended by the caller).
 *   L, T       : prefix length (>= 0) and tree size (1..64).
 *   mask       : device uint32 [T][(T+31)/32] from kdv_build_tree_mask.
 *   out        : device bf16 [T][H][Dv], written.
 *   lse        : device fp32 [T][H], nullable; natural-log sum of exp of the scaled visible scores,
 *                for merging with attention computed elsewhere.
 *   workspace  : device scratch of workspace_bytes >= kdv_verify_workspace_bytes(d, T, L); 16-byte
 *                aligned; no initial contents are needed.  After a call its int32 at offset 0 holds the
 *                KDV_DEBUG page-table status (above) when that check ran; the rest is undefined.  Calls that
 *                share a workspace must be ordered on one stream.
 * The call is three kernel launches on the stream: the query absorption, the split-KV pass, and the split
 * combine with the W_UV up-projection.  When all L + T rows fit in one 64-row KV tile and T <= 32 (and no
 * split count is forced with KDV_SPLITS), it is one kernel that takes the query absorption, the scores, the
 * softmax, the latent output and the W_UV product for each (head, block of 32 output columns).
 * Returns KDV_OK or a negative kdv_status (nothing enqueued on error). */
int kdv_verify_mla_attn(const kdv_mla_dims* d, const uint16_t* q_nope, const uint16_t* q_rope,
                        const uint16_t* w_uk, const uint16_t* w_uv, const uint16_t* c_kv, const uint16_t* k_pe,
                        int64_t pool_slots, const int32_t* page_table, int32_t L, int32_t T, const uint32_t* mask,
                        uint16_t* out, float* lse, void* workspace, size_t workspace_bytes, void* stream);

/* kdv_verify_mla_attn for callers that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc.  It takes no workspace: it uses a fixed array of
 * KDV_NOALLOC_SCRATCH_BYTES that the library holds on each device it runs on (reserved when the library is
 * loaded there, kept until the process ends), and it calls no hipMalloc, hipFree or allocating routine.
 * Arguments, results and errors as kdv_verify_mla_attn, plus KDV_ERR_WORKSPACE (nothing enqueued) when the
 * call needs more than KDV_NOALLOC_SCRATCH_BYTES of workspace (kdv_verify_workspace_bytes(d, T, L) tells; every
 * shape of the default split plan on a 256-CU device fits, a large KDV_SPLITS override may not).  All calls on
 * one device share that device's array and it keeps the last call's contents: calls that overlap in time on
 * one device (different streams, or different host threads) race and must not be issued. */
int kdv_verify_mla_attn_noalloc(const kdv_mla_dims* d, const uint16_t* q_nope, const uint16_t* q_rope,
                                const uint16_t* w_uk, const uint16_t* w_uv, const uint16_t* c_kv, const uint16_t* k_pe,
                                int64_t pool_slots, const int32_t* page_table, int32_t L, int32_t T,
                                const uint32_t* mask, uint16_t* out, float* lse, void* stream);

/* kdv_verify_mla_attn that builds the tree's ancestor mask itself: the mask of kdv_build_tree_mask(parent, T)
 * is written to `mask` (device uint32 [T][(T+31)/32], written; the caller can pass it to kdv_verify_mla_attn
 * for the other layers of the step) and `status` (device int32, nullable) by one extra block of the call's
 * first kernel (on the short-sequence path, by the kernel's first workgroup, every workgroup building the rows
 * it needs in LDS), so the verify step needs no separate mask launch.  Other arguments and results as
 * kdv_verify_mla_attn; KDV_ERR_NULL if parent is NULL, KDV_ERR_ALIGN if parent or status is not 4-byte
 * aligned.  A malformed tree is reported in `status` as for kdv_build_tree_mask, and its rows attend as that
 * mask says. */
int kdv_verify_mla_attn_tree(const kdv_mla_dims* d, const uint16_t* q_nope, const uint16_t* q_rope,
                             const uint16_t* w_uk, const uint16_t* w_uv, const uint16_t* c_kv, const uint16_t* k_pe,
                             int64_t pool_slots, const int32_t* page_table, int32_t L, int32_t T,
                             const int32_t* parent, uint32_t* mask, int32_t* status, uint16_t* out, float* lse,
                             void* workspace, size_t workspace_bytes, void* stream);

/* Same computation as kdv_verify_mla_attn, for measurement: `events` points to 2 * kdv_verify_kernel_count(d, T, L)
 * hipEvent_t created by the caller.  events[2k] and events[2k+1] receive the start and end timestamps of kernel k
 * as the hardware dispatches it (q absorption, split-KV pass, split combine with the W_UV up-projection; or the
 * short-sequence kernel alone), so hipEventElapsedTime gives each kernel's device time.  Errors as
 * kdv_verify_mla_attn, plus KDV_ERR_NULL if events is NULL. */
int kdv_verify_mla_attn_profiled(const kdv_mla_dims* d, const uint16_t* q_nope, const uint16_t* q_rope,
                                 const uint16_t* w_uk, const uint16_t* w_uv, const uint16_t* c_kv,
                                 const uint16_t* k_pe, int64_t pool_slots, const int32_t* page_table, int32_t L,
                                 int32_t T, const uint32_t* mask, uint16_t* out, float* lse, void* workspace,
                                 size_t workspace_bytes, void* stream, void* const* events);

/* Batched verify: C requests in one call, each with its own prefix length, tree, page table and queries, over a
 * shared latent pool and the same layer weights.  The pages measure the service at ten concurrent streams
 * beside one ("The Three Acts of Engineering: Diagnosis, Extension, and Analytical Pivot in a Speculative
 * Decoding Stack", section "References", item [3]) and list batching among the throughput levers ("From
 * Diagnosis to Deployment: Three Threads of Inference Engineering for Kimi K2.6", section "The Diagnostic
 * Infrastructure").  Request c's result is what kdv_verify_mla_attn computes for it alone, up to the rounding
 * of a different division of its KV rows into splits: the requests share the launches, and unless a split
 * count is forced (KDV_SPLITS) the KV tiles of all requests are dealt out in equal runs over the CUs.
 *   C          : 1 <= C <= KDV_MAX_BATCH.
 *   L, T       : host int32 [C]: prefix length (>= 0) and tree size (1..64) of each request.
 *   Requests are packed in order.  With n_c = T[0] + ... + T[c-1]:
 *   q_nope     : device bf16 [sum T][H][Dn]; request c's nodes are rows n_c .. n_c + T[c] - 1 (same for
 *                q_rope [sum T][H][Dr], out [sum T][H][Dv] and lse [sum T][H]).
 *   page_table : device int32 [sum (L+T)]; request c's L[c] + T[c] entries follow those of requests < c, laid
 *                out as for kdv_verify_mla_attn.
 *   mask       : device uint32; request c's [T[c]][(T[c]+31)/32] words (kdv_build_tree_mask of its parent
 *                array) follow those of requests < c.
 *   workspace  : >= kdv_verify_batch_workspace_bytes(d, C, L, T) bytes, 16-byte aligned.
 * Other arguments and errors as kdv_verify_mla_attn. */
int kdv_verify_mla_attn_batch(const kdv_mla_dims* d, int32_t C, const int32_t* L, const int32_t* T,
                              const uint16_t* q_nope, const uint16_t* q_rope, const uint16_t* w_uk,
                              const uint16_t* w_uv, const uint16_t* c_kv, const uint16_t* k_pe, int64_t pool_slots,
                              const int32_t* page_table, const uint32_t* mask, uint16_t* out, float* lse,
                              void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes for kdv_verify_mla_attn_batch (host arrays L, T of C entries); 0 if unsupported. */
size_t kdv_verify_batch_workspace_bytes(const kdv_mla_dims* d, int32_t C, const int32_t* L, const int32_t* T);

/* Prefix part of a split verify step: the pages' production arrangement gives the long prefix to a dense MLA
 * decode kernel and only the small tree tail to the tree kernel ("The Three Acts of Engineering: Diagnosis,
 * Extension, and Analytical Pivot in a Speculative Decoding Stack", section "References", item [1]).
 * Every query row (t, h) attends to all L prefix positions and to nothing else: no tree rows, no mask.
 * Arguments as kdv_verify_mla_attn, except:
 *   page_table : device int32 [L] (prefix positions only).
 *   L          : >= 1.
 *   lse        : nullable as before, but the merge below needs it.
 *   workspace  : kdv_prefix_workspace_bytes(d, T, L) bytes, which never exceeds kdv_verify_workspace_bytes(d, T, L).
 * The tail part is kdv_verify_mla_attn with L = 0 and a page table of the T tree rows; the two results
 * combine with kdv_merge_attn_states into the result of one kdv_verify_mla_attn over the whole cache.
 * Returns KDV_OK or a negative kdv_status (KDV_ERR_SHAPE for L < 1; nothing enqueued on error). */
int kdv_prefix_mla_attn(const kdv_mla_dims* d, const uint16_t* q_nope, const uint16_t* q_rope, const uint16_t* w_uk,
                        const uint16_t* w_uv, const uint16_t* c_kv, const uint16_t* k_pe, int64_t pool_slots,
                        const int32_t* page_table, int32_t L, int32_t T, uint16_t* out, float* lse, void* workspace,
                        size_t workspace_bytes, void* stream);

/* Workspace bytes for kdv_prefix_mla_attn (L >= 1); 0 if unsupported.  At most kdv_verify_workspace_bytes(d, T, L). */
size_t kdv_prefix_workspace_bytes(const kdv_mla_dims* d, int32_t T, int32_t L);

/* Merge of two attention results over disjoint sets of KV positions into the result over their union (the
 * merge that joins the prefix and tree-tail parts above; the same operator merges the KV splits inside
 * kdv_verify_mla_attn).  For each row r, with M = max(lse_a[r], lse_b[r]) and w_x = exp(lse_x[r] - M):
 *   out[r] = (w_a out_a[r] + w_b out_b[r]) / (w_a + w_b),   lse[r] = M + ln(w_a + w_b).
 * A part with lse = -inf (it saw no position) has weight 0; if both do, out[r] = 0 and lse[r] = -inf.
 *   out_a, out_b : device bf16 [rows][dv], 16-byte aligned (e.g. two kdv_*_mla_attn outputs, rows = T*H).
 *   lse_a, lse_b : device fp32 [rows] (natural log, as the attention entry points write it).
 *   rows, dv     : rows >= 1; 8 <= dv <= 4096, dv % 8 == 0.
 *   out          : device bf16 [rows][dv], written; lse: device fp32 [rows], nullable, written.  Neither may
 *                  overlap an input.
 * Arithmetic in fp32 from the bf16 inputs, out rounded to bf16 (nearest even).
 * Host-side return: KDV_OK, KDV_ERR_NULL, KDV_ERR_SHAPE, KDV_ERR_ALIGN, KDV_ERR_HIP.  Nothing is allocated. */
int kdv_merge_attn_states(const uint16_t* out_a, const float* lse_a, const uint16_t* out_b, const float* lse_b,
                          int64_t rows, int32_t dv, uint16_t* out, float* lse, void* stream);

/* Number of KV splits kdv_verify_mla_attn will use for these arguments on the current device
 * (diagnostic; 0 if unsupported). */
int32_t kdv_verify_num_splits(const kdv_mla_dims* d, int32_t T, int32_t L);

/* Number of kernels one kdv_verify_mla_attn call launches for these arguments: 3 (absorption, split-KV,
 * combine), or 1 (the short-sequence kernel) when L + T <= 64 and T <= 32 and KDV_SPLITS is unset; 0 if
 * unsupported.  The prefix-only call and batches of two or more requests always launch 3. */
int32_t kdv_verify_kernel_count(const kdv_mla_dims* d, int32_t T, int32_t L);

/* DIAGNOSTIC ONLY, not part of the attention path: a measurement aid for the benchmark.  Launches `blocks`
 * workgroups of 256 threads in which every wave issues `iters` rounds of four independent 32x32x16 bf16 MFMA
 * chains (4 * iters * 32768 flop per wave), the issue-rate ceiling the verify kernels are compared with.
 * sink: device float [blocks * 256], written (zeros).  Time it with events on `stream`.  Returns KDV_OK,
 * KDV_ERR_NULL, KDV_ERR_SHAPE (iters < 1, blocks outside [1, 2^20]), KDV_ERR_ALIGN, KDV_ERR_HIP. */
int kdv_mfma_probe(int32_t iters, float* sink, int32_t blocks, void* stream);

/* Static English description of a kdv_status value. */
const char* kdv_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* KDV_H */
