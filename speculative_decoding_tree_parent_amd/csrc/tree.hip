// Tree utilities of the DDTree verify step: best-first construction of the draft tree, the ancestor bitmask
// built before verification, and the greedy acceptance of the verified tree.
//
// The ancestor bitmask itself is built by build_ancestor_mask (tree_mask.h).
#include "tree_mask.h"

namespace kdv {

__global__ __launch_bounds__(64) void tree_mask_kernel(const int32_t* __restrict__ parent, int T,
                                                       uint32_t* __restrict__ mask, int32_t* __restrict__ status) {
  build_ancestor_mask(parent, T, mask, status, threadIdx.x);
}

// Best-first construction of the draft tree ("The Architecture of Diagnosis...", section "Phase 1: Custom
// CUDA Kernels", item 1: the tree is built on the device instead of with a host-side priority queue).
// The drafter gives, per position d of the block, its K best tokens tok[d][r] with log-probabilities
// logp[d][r] sorted in decreasing order.  Node 0 is the root (the committed token); a node at depth d >= 1
// takes a token of position d - 1 and scores its parent's score plus that token's log-probability (float32).
// The candidate with the highest score joins next (ties: smaller depth, then parent index, then rank); when a
// node joins, its next sibling (rank + 1) and its first child (rank 0, depth + 1) become candidates.
//
// One wave; lane j holds candidate slot j and, once node j exists, node j's score.  Each step the best
// candidate is found by a wave-wide max of its orderable score bits and, only on an exact tie, a min of
// (depth, parent, rank), which is unique per candidate.  Every step removes one candidate and adds at most two,
// so at most budget <= 64 slots are ever in use; the new sibling takes the winner's slot and the new child the
// lowest free slot.
__device__ __forceinline__ uint32_t orderable(float f) {
  const uint32_t u = __float_as_uint(f + 0.f);  // -0 -> +0: equal scores compare equal
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Wave-wide unsigned max / min with DPP row shifts and row broadcasts (no LDS permutes): lane i first takes
// the extreme of lanes [row start, i] of its 16-lane row (shifts by 1, 2, 4, 8), then rows 1 and 3 fold in
// rows 0 and 2 (broadcast of lane 15), then rows 2 and 3 fold in row 1 (broadcast of lane 31); lane 63 ends
// up with the wave's extreme.  A lane whose source is outside its row keeps its own value.
template <bool MAX>
__device__ __forceinline__ uint32_t wave_reduce_u32(uint32_t v) {
  auto step = [&](uint32_t x, uint32_t y) { return MAX ? (x > y ? x : y) : (x < y ? x : y); };
  v = step(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x111, 0xf, 0xf, false));  // row_shr:1
  v = step(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x112, 0xf, 0xf, false));  // row_shr:2
  v = step(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x114, 0xf, 0xf, false));  // row_shr:4
  v = step(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x118, 0xf, 0xf, false));  // row_shr:8
  v = step(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x142, 0xa, 0xf, false));  // row_bcast:15
  v = step(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x143, 0xc, 0xf, false));  // row_bcast:31
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

__global__ __launch_bounds__(64) void draft_tree_kernel(const float* __restrict__ logp,
                                                        const int32_t* __restrict__ tok, int block, int K,
                                                        int budget, const int32_t* __restrict__ root_token,
                                                        int32_t* __restrict__ parent, int32_t* __restrict__ tokens,
                                                        int32_t* __restrict__ n_nodes) {
  __shared__ float s_logp[KDV_MAX_DRAFT_ENTRIES];
  __shared__ int32_t s_tok[KDV_MAX_DRAFT_ENTRIES];
  const int j = threadIdx.x;
  for (int e = j; e < block * K; e += 64) {
    s_logp[e] = logp[e];
    s_tok[e] = tok[e];
  }
  __syncthreads();
  // candidate in this slot
  bool cand = false;
  float c_score = 0.f;
  int c_depth = 0, c_parent = 0, c_rank = 0;
  // node j (once it exists)
  float n_score = 0.f;
  int n_parent = -1, n_token = 0;
  if (j == 0) {
    n_token = root_token[0];
    if (budget > 1) {  // first candidate: best token of position 0
      cand = true;
      c_score = 0.f + s_logp[0];
      c_depth = 1;
    }
  }
  int n = 1;
  for (; n < budget; ++n) {  // wave-uniform loop, at most budget - 1 <= 63 steps
    // best candidate: highest score, then smaller (depth, parent, rank); candidates have keys >= 1
    const uint32_t skey = cand ? orderable(c_score) : 0u;
    const uint32_t smax = wave_reduce_u32<true>(skey);
    if (smax == 0u) break;  // no candidate left: the whole K-ary tree of depth block is in
    const unsigned long long top = __ballot(cand && skey == smax);
    if (top == 0ull) break;  // (cannot happen: smax is some candidate's key)
    int w = __builtin_ctzll(top);
    if (top & (top - 1)) {  // equal scores: the tie key decides (unique per candidate)
      const uint32_t tkey = (cand && skey == smax) ? (uint32_t)((c_depth << 12) | (c_parent << 6) | c_rank)
                                                   : 0xffffffffu;
      const uint32_t tmin = wave_reduce_u32<false>(tkey);
      w = __builtin_ctzll(__ballot(tkey == tmin));
    }
    const float s = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(c_score), w));
    const int d = __builtin_amdgcn_readlane(c_depth, w), p = __builtin_amdgcn_readlane(c_parent, w);
    const int r = __builtin_amdgcn_readlane(c_rank, w);
    const float ps = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(n_score), p));  // parent's score
    // The three table entries this step needs sit at wave-uniform addresses: every lane reads them together
    // (LDS broadcasts), so the step waits for one LDS round trip instead of three in turn.  An entry that is not
    // needed is read at a valid stand-in address and ignored.
    const bool sib = r + 1 < K, child = d < block;
    const int e = (d - 1) * K + r;
    const int32_t tk = s_tok[e];
    const float l_sib = s_logp[sib ? e + 1 : e];
    const float l_child = s_logp[child ? d * K : 0];
    asm volatile("" ::"v"(tk), "v"(l_sib), "v"(l_child));  // (keeps the three reads together, ahead of the branches)
    // the lowest free slot once the winner's slot has taken its sibling or been freed
    const unsigned long long freem = __ballot(!cand) | (sib ? 0ull : (1ull << w));
    if (j == n) {  // node n joins
      n_score = s;
      n_parent = p;
      n_token = tk;
    }
    if (j == w) {  // the winner's slot takes its next sibling, if any
      cand = sib;
      if (sib) {
        c_score = ps + l_sib;
        c_rank = r + 1;
      }
    }
    if (child) {  // first child of node n, in the lowest free slot
      const int f = __builtin_ctzll(freem);
      if (j == f) {
        cand = true;
        c_score = s + l_child;
        c_depth = d + 1;
        c_parent = n;
        c_rank = 0;
      }
    }
  }
  if (j < budget) {
    parent[j] = j < n ? n_parent : -1;
    tokens[j] = j < n ? n_token : -1;
  }
  if (j == 0) n_nodes[0] = n;
}

// Greedy acceptance ("The Architecture of Diagnosis...", section "Phase 1: Custom CUDA Kernels", item 3: after
// verification the longest prefix of accepted tokens is selected on the device).  Node 0 is the root, whose
// token is already committed; pred[t] is the target's greedy prediction after the prefix that ends at node t.
// A child is accepted when its draft token equals its parent's prediction.  One wave, one node per lane:
// each step every lane checks whether it is an accepted child of the current node, and the lowest such
// lane (ballot, lowest set bit) becomes the current node.  A path has at most T nodes, so at most T - 1
// steps.  Malformed trees (the mask's rules) give KDV_ERR_TREE and the root alone.
__global__ __launch_bounds__(64) void tree_accept_kernel(const int32_t* __restrict__ parent,
                                                         const int32_t* __restrict__ tokens,
                                                         const int32_t* __restrict__ pred, int T,
                                                         int32_t* __restrict__ path, int32_t* __restrict__ n_path,
                                                         int32_t* __restrict__ next_token,
                                                         int32_t* __restrict__ status) {
  const int i = threadIdx.x;
  const bool live = i < T;
  const int p = live ? parent[i] : -2;
  const int tk = live ? tokens[i] : 0;
  const int pr = live ? pred[i] : 0;
  const bool valid = !live || (i == 0 ? p == -1 : (p >= 0 && p < i));
  const bool tree_ok = !__any(!valid);
  int cur = 0, n = 1;
  if (tree_ok) {
    for (int step = 1; step < T; ++step) {  // wave-uniform loop
      const int want = __shfl(pr, cur);
      const unsigned long long hits = __ballot(live && p == cur && tk == want);
      if (hits == 0ull) break;
      cur = __builtin_ctzll(hits);
      if (i == 0) path[n] = cur;
      ++n;
    }
  }
  const int nt = __shfl(pr, cur);
  if (live && i >= n) path[i] = -1;
  if (i == 0) {
    path[0] = 0;
    n_path[0] = n;
    next_token[0] = nt;
    if (status != nullptr) status[0] = tree_ok ? KDV_OK : KDV_ERR_TREE;
  }
}

}  // namespace kdv

extern "C" int kdv_build_tree_mask(const int32_t* parent, int32_t T, uint32_t* mask, int32_t* status,
                                   void* stream) {
  if (parent == nullptr || mask == nullptr) return KDV_ERR_NULL;
  if (T < 1 || T > KDV_MAX_TREE_NODES) return KDV_ERR_SHAPE;
  if ((reinterpret_cast<uintptr_t>(parent) & 3) || (reinterpret_cast<uintptr_t>(mask) & 3) ||
      (reinterpret_cast<uintptr_t>(status) & 3))
    return KDV_ERR_ALIGN;
  (void)hipGetLastError();  // (an error left by earlier work is not this call's)
  hipLaunchKernelGGL(kdv::tree_mask_kernel, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream), parent, T,
                     mask, status);
  return hipGetLastError() == hipSuccess ? KDV_OK : KDV_ERR_HIP;
}

extern "C" int kdv_tree_accept(const int32_t* parent, const int32_t* tokens, const int32_t* pred, int32_t T,
                               int32_t* path, int32_t* n_path, int32_t* next_token, int32_t* status, void* stream) {
  if (parent == nullptr || tokens == nullptr || pred == nullptr || path == nullptr || n_path == nullptr ||
      next_token == nullptr)
    return KDV_ERR_NULL;
  if (T < 1 || T > KDV_MAX_TREE_NODES) return KDV_ERR_SHAPE;
  const void* ptrs[] = {parent, tokens, pred, path, n_path, next_token, status};
  for (const void* q : ptrs)
    if (reinterpret_cast<uintptr_t>(q) & 3) return KDV_ERR_ALIGN;
  (void)hipGetLastError();  // (an error left by earlier work is not this call's)
  hipLaunchKernelGGL(kdv::tree_accept_kernel, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream), parent,
                     tokens, pred, T, path, n_path, next_token, status);
  return hipGetLastError() == hipSuccess ? KDV_OK : KDV_ERR_HIP;
}

extern "C" int kdv_build_draft_tree(const float* logp, const int32_t* tok, int32_t block, int32_t K, int32_t budget,
                                    const int32_t* root_token, int32_t* parent, int32_t* tokens, int32_t* n_nodes,
                                    void* stream) {
  if (logp == nullptr || tok == nullptr || root_token == nullptr || parent == nullptr || tokens == nullptr ||
      n_nodes == nullptr)
    return KDV_ERR_NULL;
  if (block < 1 || block > 63 || K < 1 || K > 64 || block * K > KDV_MAX_DRAFT_ENTRIES || budget < 1 ||
      budget > KDV_MAX_TREE_NODES)
    return KDV_ERR_SHAPE;
  const void* ptrs[] = {logp, tok, root_token, parent, tokens, n_nodes};
  for (const void* q : ptrs)
    if (reinterpret_cast<uintptr_t>(q) & 3) return KDV_ERR_ALIGN;
  (void)hipGetLastError();  // (an error left by earlier work is not this call's)
  hipLaunchKernelGGL(kdv::draft_tree_kernel, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream), logp, tok,
                     block, K, budget, root_token, parent, tokens, n_nodes);
  return hipGetLastError() == hipSuccess ? KDV_OK : KDV_ERR_HIP;
}
