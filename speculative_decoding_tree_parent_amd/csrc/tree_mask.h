// Ancestor bitmask of a DDTree draft tree, as a device function for one wave (used by the stand-alone mask
// kernel and by the verify call that builds its own mask).
//
// A draft-tree node may attend to the prefix, its ancestors and itself ("The Architecture of
// Diagnosis...", section "Phase 1: Custom CUDA Kernels", item 2: a visibility mask that reflects the
// tree structure).  Nodes are in topological order (parent[i] < i), so every chain of parents is at
// most T - 1 <= 63 steps long.  One wave holds one node per lane and builds all rows at once by
// pointer jumping: after round r a lane holds the bits of the first 2^r nodes of its root path and
// the node 2^r steps up, so six rounds of cross-lane reads (ds_bpermute) cover any path.
#pragma once
#include "common.h"

namespace kdv {

// Called by all 64 lanes of one wave (lane = node index); T <= 64.
__device__ __forceinline__ void build_ancestor_mask(const int32_t* __restrict__ parent, int T,
                                                    uint32_t* __restrict__ mask, int32_t* __restrict__ status,
                                                    int i) {
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

}  // namespace kdv
