// Ancestor bitmask of a DDTree draft tree.
//
// A draft-tree node may attend to the prefix, its ancestors and itself ("The Architecture of
// Diagnosis...", section "Phase 1: Custom CUDA Kernels", item 2: a visibility mask that reflects the
// tree structure).  With nodes in topological order (parent[i] < i) the mask of node i is the mask of
// its parent plus its own bit; each lane here walks its node's parent chain, which is at most T long.
#include "common.h"

namespace kdv {

__global__ __launch_bounds__(64) void tree_mask_kernel(const int32_t* __restrict__ parent, int T,
                                                       uint32_t* __restrict__ mask, int32_t* __restrict__ status) {
  __shared__ int any_bad;
  __shared__ int par[KDV_MAX_TREE_NODES];  // the walk reads parents from LDS: one global load per node
  const int i = threadIdx.x;
  if (i == 0) any_bad = 0;
  if (i < T) par[i] = parent[i];
  __syncthreads();
  if (i < T) {
    uint32_t w0 = 0u, w1 = 0u;
    int j = i;
    // Walk i -> parent -> ... -> root.  A valid chain strictly decreases, so T steps always suffice.
    for (int step = 0; step < KDV_MAX_TREE_NODES; ++step) {
      if (j < 32) w0 |= 1u << j; else w1 |= 1u << (j - 32);
      const int p = par[j];
      const bool ok = (j == 0) ? (p == -1) : (p >= 0 && p < j);
      if (!ok) {
        if (j == i) atomicOr(&any_bad, 1);   // report each invalid row once, from its own lane
        break;
      }
      if (j == 0) break;
      j = p;
    }
    const int W = (T + 31) >> 5;
    mask[i * W] = w0;
    if (W == 2) mask[i * W + 1] = w1;
  }
  __syncthreads();
  if (i == 0 && status != nullptr) status[0] = any_bad ? KDV_ERR_TREE : KDV_OK;
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
