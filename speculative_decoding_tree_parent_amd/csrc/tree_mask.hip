// Tree utilities of the DDTree verify step: the ancestor bitmask, built before verification, and the greedy
// acceptance of the verified tree.
//
// Ancestor bitmask of a DDTree draft tree.
//
// A draft-tree node may attend to the prefix, its ancestors and itself ("The Architecture of
// Diagnosis...", section "Phase 1: Custom CUDA Kernels", item 2: a visibility mask that reflects the
// tree structure).  Nodes are in topological order (parent[i] < i), so every chain of parents is at
// most T - 1 <= 63 steps long.  One wave holds one node per lane and builds all rows at once by
// pointer jumping: after round r a lane holds the bits of the first 2^r nodes of its root path and
// the node 2^r steps up, so six rounds of cross-lane reads (ds_bpermute) cover any path.
#include "common.h"

namespace kdv {

__global__ __launch_bounds__(64) void tree_mask_kernel(const int32_t* __restrict__ parent, int T,
                                                       uint32_t* __restrict__ mask, int32_t* __restrict__ status) {
  const int i = threadIdx.x;
  const bool live = i < T;
  const int p = live ? parent[i] : -1;
  // A row is valid when the root has no parent and every other node's parent precedes it.  The walk
  // from an invalid row stops at that row: its mask holds its own bit only.
  const bool valid = !live || (i == 0 ? p == -1 : (p >= 0 && p < i));
  int up = (live && valid && i != 0) ? p : -1;  // next node on the path, -1 at its end
  uint64_t anc = live ? (1ull << i) : 0ull;
#pragma unroll
  for (int r = 0; r < 6; ++r) {
    const int src = up < 0 ? i : up;
    const uint32_t lo = __shfl((uint32_t)anc, src);
    const uint32_t hi = __shfl((uint32_t)(anc >> 32), src);
    const int up2 = __shfl(up, src);
    if (up >= 0) {
      anc |= ((uint64_t)hi << 32) | lo;
      up = up2;
    }
  }
  if (live) {
    const int W = (T + 31) >> 5;
    mask[i * W] = (uint32_t)anc;
    if (W == 2) mask[i * W + 1] = (uint32_t)(anc >> 32);
  }
  const bool any_bad = __any(!valid);
  if (i == 0 && status != nullptr) status[0] = any_bad ? KDV_ERR_TREE : KDV_OK;
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
  hipLaunchKernelGGL(kdv::tree_accept_kernel, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream), parent,
                     tokens, pred, T, path, n_path, next_token, status);
  return hipGetLastError() == hipSuccess ? KDV_OK : KDV_ERR_HIP;
}
