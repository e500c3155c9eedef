// Tree-verify MLA attention in absorbed form, split over the KV sequence (gfx950 / CDNA4).
//
// What is computed follows "The Architecture of Diagnosis...", section "Phase 1: Custom CUDA Kernels",
// item 2 (every draft-tree node attends over the KV cache under the tree's visibility mask, with the
// latent projection absorbed), over the 512 + 64 element MLA latent cache of "From Diagnosis to
// Deployment...", section "The Second Thread: Pivoting to 200k Context", addressed one token per page
// ("The Architecture of Diagnosis...", section "The Discrepancy That Revealed the Truth").
//
// Three kernels, enqueued in order on the caller's stream:
//   q_absorb : q_cat[m] = [W_UK[h]^T q_nope[t,h] ; q_rope[t,h]]          (m = t*H + h; bf16 MFMA)
//   splitkv  : one workgroup per (64 query rows, KV split).  KV tiles of 64 paged rows are gathered into
//              LDS by DMA one tile ahead; scores S^T = K Q^T and O^T += V^T P^T run on 32x32x16 bf16 MFMA
//              with an online softmax; the partial (O, max, sum) of the split goes to the workspace.
//   combine_up : log-sum-exp merge of the splits -> lse and the latent output o[t,h] (bf16, in LDS), then
//              out[t,h] = W_UV[h] o[t,h]                                   (bf16 MFMA)
// A single call whose L + T rows fit in one KV tile (and T <= 32) is one kernel instead, short_verify: per (head,
// block of output columns) the absorption, the scores, an exact one-tile softmax, P V and the W_UV product.
#include <hip/hip_ext.h>
#include <algorithm>
#include <atomic>
#include <type_traits>
#include <mutex>
#include <math.h>
#include <stdlib.h>

#include "common.h"
#include "tree_mask.h"

namespace kdv {

constexpr int KV_TILE = 64;   // KV rows per LDS tile
constexpr int M_TILE = 64;    // query rows (node, head) per split-KV workgroup
constexpr int NTHREADS = 256;
constexpr int NUM_XCD = 8;    // MI355X: 8 accelerator complex dies, each with its own L2
constexpr int MAX_BATCH = KDV_MAX_BATCH;

// Launch parameters of one request of a (possibly batched) call, computed on the host and passed by value in
// the kernel arguments.  Requests are packed: their nodes, page-table entries and mask words follow one another.
struct ReqArgs {
  int L, T, N;                  // prefix rows, tree nodes, KV rows attended (L + T, or L for a prefix-only pass)
  int node0, pt0, mask0;        // first node (q, out and lse rows), first page-table entry, first mask word
  int m_tiles, Mp;              // 64-row query tiles of the request's T*H rows, and their padded row count
  int tiles_per_split, splits;  // KV split plan
  int xoff;                     // the request's splits start at this XCD (spreads small requests over the dies)
  int lin;                      // > 0: contiguous placement, lin workgroup slots per XCD (see splitkv_kernel)
  long long po, pml;            // element offsets of the request's partials in part_o and part_ml
  long long sk_base;            // stream-K plan: the request's first KV tile in the concatenation of all requests
};
// NB = capacity: 1 for the single-request entry points (a small kernel-argument block), MAX_BATCH for batches.
template <int NB>
struct BatchArgs {
  int n, H;
  int blk_split[NB + 1];  // first split-KV workgroup of each request (multiples of NUM_XCD)
  int blk_comb[NB + 1];   // first combine workgroup of each request (multiples of NUM_XCD)
  ReqArgs r[NB];
  // stream-K plan of a batch (sk_w > 0): KV tiles per run, KV tiles of all requests, workgroups per group (one
  // per query tile), workgroup slots per XCD, groups
  long long sk_w, sk_u;
  int sk_g, sk_lin, sk_groups;
};
// Request owning workgroup b (uniform): the last one whose first workgroup is <= b.
__device__ __forceinline__ int request_of(const int* first, int n, int b) {
  int c = 0;
  while (c + 1 < n && b >= first[c + 1]) ++c;
  return c;
}

template <int R, int DR>
struct Shape {
  static constexpr int DQ = R + DR;      // score contraction length (576 for the Kimi shape)
  static constexpr int KB = DQ / 16;     // 16-deep MFMA k-blocks of the score contraction
  static constexpr int PITCH = DQ + 8;   // LDS row pitch in elements: +16 B keeps 16-row b128 reads conflict-free
  static constexpr int CH = DQ / 8;      // 16-byte chunks per KV row
  static constexpr int DB = R / 64;      // 32-wide output column blocks per wave (a wave owns R/2 columns)
};

// ------------------------------------------------------------------------------------------------ splitkv
// LDS layout of one 64-row KV tile: the latent rows [64][R] then the rotary rows [64][DR], bf16, row-major.
// Within a row the 16-byte chunks are XOR-swizzled (chunk c of row r is stored at c ^ swz(r)) so that
//   - the score MFMA's 16 lanes, which read the same chunk of 16 consecutive rows, hit 16 distinct bank
//     groups, and
//   - the value MFMA's transposed reads, 4 consecutive rows x 4 adjacent chunks per 32 lanes, hit 16.
// The swizzle replaces row padding, so two tiles fit in LDS (2 x 72 KB for the Kimi shape).
// For rows of >= 16 chunks, swz(r) = 4*(r % 4) + (r / 4) % 4: any 16 aligned rows get 16 distinct values (score
// reads), and the 32 lanes of a transposed read -- 4 aligned rows x 4 adjacent chunks -- land on 16 distinct
// 16-byte bank groups.  Narrower rows (test shape) use a simpler row-dependent rotation.
template <int C>  // C = 16-byte chunks per row
__device__ __forceinline__ int swz(int row) {
  if constexpr (C >= 16) return ((row & 3) << 2) | ((row >> 2) & 3);
  else return (row >> (C == 8 ? 1 : C == 4 ? 2 : 3)) & (C - 1);
}

// Query-tile staging swizzle (rows of QC 16-byte chunks): XOR within aligned groups of 8 chunks.
template <int QC>
__device__ __forceinline__ int qswz(int row, int ch) {
  if constexpr (QC % 8 == 0) return (ch & ~7) | ((ch ^ (row >> 1)) & 7);
  else return ch;
}

template <int R, int DR>
struct TileLayout {
  static constexpr int CK = R / 8;                     // chunks per latent row
  static constexpr int CP = DR / 8;                    // chunks per rotary row
  static constexpr int CKV_BYTES = KV_TILE * R * 2;
  static constexpr int BYTES = CKV_BYTES + KV_TILE * DR * 2;
  static constexpr int NDMA = CK + CP;                 // 64-lane x 16-byte DMA instructions per tile
  // byte offset of (row, logical chunk) in the tile
  __device__ static __forceinline__ int ckv(int row, int ch) { return row * (R * 2) + ((ch ^ swz<CK>(row)) << 4); }
  __device__ static __forceinline__ int kpe(int row, int ch) {
    return CKV_BYTES + row * (DR * 2) + ((ch ^ swz<CP>(row)) << 4);
  }
};

// Gather one tile of paged rows straight into LDS with global_load_lds_dwordx4: lane l of an instruction
// writes LDS bytes [16l, 16l+16) of that instruction's 1 KB block (M0 holds the block address).  The loads
// are issued from inline assembly so that the compiler neither tracks them as LDS stores (it would wait for
// the prefetch before every read of the other buffer) nor keeps per-instruction 64-bit addresses live;
// completion is awaited explicitly (wait_vmem_all + barrier) before a tile is read.
// `slot_v` holds, in lane j, the pool slot of tile row j; the work is split over the 4 waves.
// M0 is listed as clobbered; the compiler treats it as reserved and does not preserve it around the asm, which
// is harmless here because nothing else in these kernels reads M0 (no LDS-DMA builtins, GWS or message ops).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16_uniform_base(const void* sbase, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase),
               "s"(lds_addr)
               : "memory", "m0");
}
__device__ __forceinline__ void dma16_lane_addr(const void* vaddr, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(vaddr), "s"(lds_addr)
               : "memory", "m0");
}
// 4 bytes per lane: lane l's word lands at lds_addr + 4 l.
__device__ __forceinline__ void dma4_lane_addr(const void* vaddr, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(vaddr), "s"(lds_addr)
               : "memory", "m0");
}
#pragma clang diagnostic pop
// Wait until at most N vector-memory loads of this wave are outstanding.  Loads complete in issue order, so
// this covers every load issued before the last N (the compiler's own waits do not count the DMA asm).
template <int N>
__device__ __forceinline__ void wait_vmem_below() {
  static_assert(N >= 0 && N < 64, "vmcnt field");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
__device__ __forceinline__ uint32_t lds_address(const void* p) {
  return (uint32_t)(size_t)(const __attribute__((address_space(3))) char*)(p);
}

// The DMA instructions of one tile, as issued by one wave: latent rows first (wave w takes rows w, w+4, ...),
// then rotary rows.  `issue(k)` sends this wave's k-th instruction, so the loads of the next tile can be spread
// between the MFMAs of the current one.  `slot_v` holds, in lane j, the pool slot of tile row j.
template <int R, int DR>
struct TileDma {
  using TL = TileLayout<R, DR>;
  static constexpr int NKC = (TL::CK + 3) / 4, NKP = (TL::CP + 3) / 4, NK = NKC + NKP;
  const char* c_kv;
  const char* k_pe;
  uint32_t lbase;
  int slot_v, wave, lane;
  uint32_t voff[4];  // per-lane offsets of a latent row (64-chunk rows: the swizzle repeats every 4 rows)
  int kp_slot[NKP];  // pool slot of this lane's rotary row in each rotary instruction, taken from slot_v by
                     // target(), so that the cross-lane read's latency passes before the instruction is issued

  __device__ __forceinline__ TileDma(const uint16_t* ckv, const uint16_t* kpe, int wave_, int lane_)
      : c_kv(reinterpret_cast<const char*>(ckv)), k_pe(reinterpret_cast<const char*>(kpe)), lbase(0), slot_v(0),
        wave(wave_), lane(lane_) {
#pragma unroll
    for (int k = 0; k < 4; ++k) voff[k] = (uint32_t)((lane ^ swz<TL::CK>(wave + 4 * k)) << 4);
  }
  __device__ __forceinline__ void target(const char* buf, int slots) {
    lbase = lds_address(buf);
    slot_v = slots;
#pragma unroll
    for (int k = 0; k < NKP; ++k) kp_slot[k] = __shfl(slots, ((wave + 4 * k) * 64 + lane) / TL::CP);
  }
  __device__ __forceinline__ void issue(int k) const {
    if (k < NKC) {
      const int i = wave + 4 * k;
      if constexpr (TL::CK == 64) {
        const int slot = __builtin_amdgcn_readlane(slot_v, i);
        dma16_uniform_base(c_kv + (size_t)slot * (R * 2), voff[k & 3], lbase + i * 1024);
      } else if (TL::CK % 4 == 0 || i < TL::CK) {
        const int flat = i * 64 + lane, row = flat / TL::CK, pos = flat % TL::CK;
        const int slot = __shfl(slot_v, row);
        dma16_lane_addr(c_kv + (size_t)slot * (R * 2) + ((pos ^ swz<TL::CK>(row)) << 4), lbase + i * 1024);
      }
    } else {
      const int j = wave + 4 * (k - NKC);
      if (TL::CP % 4 == 0 || j < TL::CP) {
        const int flat = j * 64 + lane, row = flat / TL::CP, pos = flat % TL::CP;
        dma16_lane_addr(k_pe + (size_t)kp_slot[k - NKC] * (DR * 2) + ((pos ^ swz<TL::CP>(row)) << 4),
                        lbase + TL::CKV_BYTES + j * 1024);
      }
    }
  }
};

__device__ __forceinline__ void wait_vmem_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Softmax state of the two query rows a lane serves in the value product: row c of row block 0 and row c of
// row block 1 (c = lane % 32, a row block = 32 rows).  Every lane with the same c, in every wave, holds the
// same values.
struct RowState {
  float m_ref[2];  // reference max per row block (log2 units; an integer or -inf): P = 2^(s - m_ref) <= 2^8
  float l[2];      // sum_n P relative to m_ref
};

// Value-product split: each wave owns CPW latent columns for all 64 query rows, so every transposed V
// fragment it reads from LDS feeds two MFMAs (row blocks 0 and 1).  (Transposed LDS reads cost about three
// times as much per byte as plain 16-byte reads; this halves them.)  The narrow test shape (R = 64) uses two
// waves of 32 columns.
template <int R>
struct PvSplit {
  static constexpr int CPW = R / 4 >= 32 ? R / 4 : 32;  // latent columns per wave
  static constexpr int WAVES = R / CPW;                  // waves that own columns
  static constexpr int DBW = CPW / 32;                   // 32-column blocks per wave
};

// One tile.  Wave (wi, wj) computes the scores of row block wi against its 32 KV rows (half wj of the tile)
// and proposes a softmax reference for its rows; P (bf16), proposals and row sums of all four waves are
// swapped through LDS; every wave then agrees on each row block's maximum, brings its O to it (exact powers
// of two) and accumulates O^T += V^T P^T for its columns over the whole tile.  The next tile's DMA
// instructions (if `dma_on`) are spread over the score MFMAs.
template <int R, int DR>
__device__ __forceinline__ void tile_compute(const char* tile, const bf16x8 (&q)[(R + DR) / 16],
                                             f32x16 (&o)[2][PvSplit<R>::DBW], RowState& st, int n0, int L, int N,
                                             uint32_t mw0, uint32_t mw1, float scale_log2, uint4 (*pbuf)[2][2][64],
                                             float (*mxch)[2][32], float (*psum)[2][32], int wi, int wj, int wave,
                                             int lane, const TileDma<R, DR>& dma, bool dma_on) {
  using TL = TileLayout<R, DR>;
  constexpr int KB = (R + DR) / 16;
  const int g = lane >> 5, c = lane & 31;
  // ---- scores S^T[n][m] for tile rows n = wj*32 + (r/4)*8 + g*4 + r%4
  // The swizzle only touches the low log2(F) bits of a chunk index, so a row's fragment offsets repeat with
  // period F/2 k-blocks plus a compile-time stride: a few per-lane bases and immediate offsets.
  constexpr int FK = TL::CK < 16 ? TL::CK : 16, PK = FK / 2;
  constexpr int FP = TL::CP < 16 ? TL::CP : 16, PP = FP / 2;
  f32x16 acc0 = zero16(), acc1 = zero16();  // two chains: a single dependent MFMA chain issues ~25% slower
  const int nrow = wj * 32 + c;
  const char* ckp[PK];
  const char* kpp[PP];
#pragma unroll
  for (int i = 0; i < PK; ++i) ckp[i] = tile + nrow * (R * 2) + (((2 * i + g) ^ swz<TL::CK>(nrow)) << 4);
#pragma unroll
  for (int i = 0; i < PP; ++i) kpp[i] = tile + TL::CKV_BYTES + nrow * (DR * 2) + (((2 * i + g) ^ swz<TL::CP>(nrow)) << 4);
  auto kfrag = [&](int kb) -> bf16x8 {
    const int kr = kb - R / 16;
    const char* p = (kb < R / 16) ? ckp[kb % PK] + (kb / PK) * FK * 16 : kpp[kr % PP] + (kr / PP) * FP * 16;
    return *reinterpret_cast<const bf16x8*>(p);
  };
  // Software pipeline: fragment kb+QD is requested before the MFMA of kb.  With one wave per SIMD nothing else
  // hides LDS latency, so the order is pinned with scheduling fences (the compiler would otherwise shorten
  // the pipeline to save registers).  A DMA instruction goes out every DSTEP MFMAs: its issue stalls while the
  // address unit drains the previous ones, and the MFMAs in flight cover that stall.
  constexpr int QD = KB < 6 ? KB : 6;
  constexpr int DSTEP = KB / TileDma<R, DR>::NK > 0 ? KB / TileDma<R, DR>::NK : 1;
  bf16x8 kf[QD];
#pragma unroll
  for (int i = 0; i < QD; ++i) kf[i] = kfrag(i);
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    const bf16x8 a = kf[kb % QD];
    if (kb + QD < KB) kf[kb % QD] = kfrag(kb + QD);
    if (kb % DSTEP == 0 && kb / DSTEP < TileDma<R, DR>::NK && dma_on) dma.issue(kb / DSTEP);
    __builtin_amdgcn_sched_barrier(0);
    if (kb & 1) acc1 = mfma32(a, q[kb], acc1);
    else acc0 = mfma32(a, q[kb], acc0);
    __builtin_amdgcn_sched_barrier(0);
  }
  if (KB < TileDma<R, DR>::NK && dma_on) {  // (narrow test shape: more DMA instructions than k-blocks)
#pragma unroll
    for (int k = KB; k < TileDma<R, DR>::NK; ++k) dma.issue(k);
  }
  float s[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) s[r] = acc0[r] + acc1[r];  // unscaled: the scale (> 0) goes into the exp2's fma
  if (n0 + KV_TILE > L) {  // tile reaches the tree rows (or past N): apply the ancestor mask
    const uint64_t mw = (uint64_t)mw0 | ((uint64_t)mw1 << 32);
    const int T = N - L;
    const int jb = n0 + wj * 32 + g * 4 - L;  // tree index of register 0's row
#pragma unroll
    for (int r = 0; r < 16; ++r) {  // (bitwise, not short-circuit: selects in place, no per-element branches)
      const int jn = jb + (r >> 2) * 8 + (r & 3);
      const bool vis = (jn < 0) | ((jn < T) & (((uint32_t)(mw >> (jn & 63)) & 1u) != 0u));
      s[r] = vis ? s[r] : -INFINITY;
    }
  }
  float tmax = -INFINITY;
#pragma unroll
  for (int r = 0; r < 16; ++r) tmax = fmaxf(tmax, s[r]);
  tmax = pair_max(tmax) * scale_log2;  // max of the scaled scores (scale > 0; -inf stays -inf)
  // ---- proposed reference for row (wi, c): keep the current one unless this half-tile exceeds it by more
  // than 2^8.  P of this half-tile is taken relative to the proposal.
  const float mref = (wi == 0) ? st.m_ref[0] : st.m_ref[1];  // (no dynamic index: st stays in registers)
  const float prop = (tmax > mref + 8.f) ? ceilf(tmax) : mref;
  const float puse = (prop == -INFINITY) ? 0.f : prop;
  bf16x8 pk[2];
  float ps;  // unrounded row sum of this half-tile
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float p0 = fast_exp2(fmaf(s[e], scale_log2, -puse)), p1 = fast_exp2(fmaf(s[8 + e], scale_log2, -puse));
    ps = (e == 0) ? p0 + p1 : ps + (p0 + p1);
    pk[0][e] = (__bf16)p0;
    pk[1][e] = (__bf16)p1;
  }
  ps = pair_sum(ps);
  pbuf[wi][wj][0][lane] = __builtin_bit_cast(uint4, pk[0]);
  pbuf[wi][wj][1][lane] = __builtin_bit_cast(uint4, pk[1]);
  if (g == 0) {
    mxch[wi][wj][c] = prop;
    psum[wi][wj][c] = ps;
  }

  // ---- O^T[d][m] += sum_n V^T[d][n] P^T[n][m]; within a 16-row k-step the contraction index k = g*8+e is
  // KV row (e/4)*8 + g*4 + e%4, matching the score layout.  Fragment idx = k-step ks (KV rows ks*16..+15) x
  // column block db of this wave's columns.
  // Lane's rows are ks*16 + rl (+8): the swizzle depends only on rl and the +8, and the column chunk's
  // swizzled bits only on db, so 8 per-tile pointers plus immediates address all fragments (F = 16 case).
  using PV = PvSplit<R>;
  constexpr int DBW = PV::DBW;
  const bool pv_wave = wave < PV::WAVES;
  const int rl = g * 4 + ((lane & 15) >> 2);
  const int cl = ((lane & 31) >> 4) * 2 + ((lane & 3) >> 1);  // chunk within a 32-column block
  const int sub = (lane & 1) * 8;                              // byte offset inside the chunk
  const int col0 = (pv_wave ? wave : 0) * PV::CPW;             // first latent column of this wave
  const char* pvp[2][DBW < 4 ? DBW : 4];
  if constexpr (TL::CK >= 16) {
    static_assert(PV::CPW % 128 == 0, "column base must be a multiple of 16 chunks");
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int d4 = 0; d4 < (DBW < 4 ? DBW : 4); ++d4)
        pvp[s2][d4] = tile + col0 * 2 + (rl + 8 * s2) * (R * 2) + (((d4 * 4 + cl) ^ swz<TL::CK>(rl + 8 * s2)) << 4) + sub;
  }
  constexpr int NV = 4 * DBW, VD = NV < 6 ? NV : 6;
  auto vfrag = [&](int idx) -> bf16x8 {
    const int ks = idx / DBW, db = idx % DBW;
    const int rb = ks * 16;
    const char *p0, *p1;
    if constexpr (TL::CK >= 16) {
      const int imm = rb * (R * 2) + (db >> 2) * 256;
      p0 = pvp[0][db & 3] + imm;
      p1 = pvp[1][db & 3] + imm;
    } else {
      const int ch = (col0 + db * 32) / 8 + cl;
      p0 = tile + TL::ckv(rb + rl, ch) + sub;
      p1 = tile + TL::ckv(rb + rl + 8, ch) + sub;
    }
    return concat_tr(lds_read_tr16(p0), lds_read_tr16(p1));
  };
  // the first value fragments are requested before the exchange barrier
  bf16x8 vf[VD];
  if (pv_wave) {
#pragma unroll
    for (int i = 0; i < VD; ++i) vf[i] = vfrag(i);
  }
  __syncthreads();

  // ---- every row block: agree on M = max of both halves' proposals, bring O and the P blocks to it, and update
  // the row sum (fixed order, so all waves hold the same bits)
  // all exchange reads are issued together (the own P block is read back too: same bits, no branch)
  bf16x8 pf[2][4];  // [row block][k-step]: k-steps 0, 1 from KV half 0, 2, 3 from half 1
  float pr[2][2], sm[2][2];
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int jh = 0; jh < 2; ++jh) {
      pr[b][jh] = mxch[b][jh][c];
      sm[b][jh] = psum[b][jh][c];
#pragma unroll
      for (int h = 0; h < 2; ++h) pf[b][jh * 2 + h] = __builtin_bit_cast(bf16x8, pbuf[b][jh][h][lane]);
    }
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const float p0 = pr[b][0], p1 = pr[b][1];
    const float s0 = sm[b][0], s1 = sm[b][1];
    const float M = fmaxf(p0, p1);  // >= m_ref: a proposal never lowers the reference
    // A row that has seen nothing yet (M = -inf) has O = 0, l = 0 and P = 0: scaling it by 2^(x - 0) = 0 is exact.
    const float Ms = (M == -INFINITY) ? 0.f : M;
    const float a = fast_exp2(st.m_ref[b] - Ms);  // m_ref = -inf -> 0
    if (__any(M > st.m_ref[b])) {
#pragma unroll
      for (int db = 0; db < DBW; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[b][db][r] *= a;
    }
    const float f0 = fast_exp2(p0 - Ms), f1 = fast_exp2(p1 - Ms);
    if (__any((f0 != 1.f || f1 != 1.f) && M != -INFINITY)) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float f = (k < 2) ? f0 : f1;
#pragma unroll
        for (int e = 0; e < 8; ++e) pf[b][k][e] = (__bf16)((float)pf[b][k][e] * f);
      }
    }
    st.l[b] = st.l[b] * a + (s0 * f0 + s1 * f1);
    st.m_ref[b] = M;
  }
  if (!pv_wave) return;  // wave-uniform; the caller's next barrier is the only one that follows
#pragma unroll
  for (int idx = 0; idx < NV; ++idx) {
    const int ks = idx / DBW, db = idx % DBW;
    const bf16x8 a = vf[idx % VD];
    if (idx + VD < NV) vf[idx % VD] = vfrag(idx + VD);
    __builtin_amdgcn_sched_barrier(0);
    o[0][db] = mfma32(a, pf[0][ks], o[0][db]);
    o[1][db] = mfma32(a, pf[1][ks], o[1][db]);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// The part of a split-KV segment after its prologue: the query tile (staged in LDS at qbuf) into registers, the
// loop over the segment's KV tiles (the first one already gathered into the first KV buffer, the next tile's
// page-table slice in slot_v), and the partial (O / l, max, sum) of the segment into partial slot `split`.  All
// threads of the workgroup call it together.
template <int R, int DR>
__device__ __forceinline__ void seg_body(char* kvbuf, const char* qbuf, uint4 (*pbuf)[2][2][64], float (*mxch)[2][32],
                                         float (*psum)[2][32], TileDma<R, DR>& dma, int slot_v,
                                         const int32_t* __restrict__ page_table, int tile_begin, int tile_end, int L,
                                         int N, uint32_t mw0, uint32_t mw1, float scale_log2, int mt, int split, int Mp,
                                         uint16_t* __restrict__ part_o, float2* __restrict__ part_ml) {
  using TL = TileLayout<R, DR>;
  constexpr int DQ = R + DR, KB = DQ / 16;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wi = wave >> 1, wj = wave & 1;
  const int g = lane >> 5, c = lane & 31;
  bf16x8 q[KB];
  {
    constexpr int QC = DQ / 8;
    const int r = wi * 32 + c;
    const char* qrow = qbuf + r * QC * 16;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) q[kb] = *reinterpret_cast<const bf16x8*>(qrow + qswz<QC>(r, 2 * kb + g) * 16);
  }
  // Register classes: the query fragments (MFMA B operands) live in AGPRs and the O accumulators in VGPRs
  // (MFMA's VGPR form, selected at build time), so the softmax rescale of O needs no AGPR<->VGPR copies.
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) asm volatile("" : "+a"(q[kb]));
  constexpr int DBW = PvSplit<R>::DBW;
  f32x16 o[2][DBW];
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int db = 0; db < DBW; ++db) o[b][db] = zero16();
  RowState st{{-INFINITY, -INFINITY}, {0.f, 0.f}};

  for (int tile = tile_begin; tile < tile_end; ++tile) {
    const int cur = (tile - tile_begin) & 1;
    wait_vmem_all();  // this wave's share of the current tile has landed
    __syncthreads();  // ... and every wave's; the other buffer and the exchange buffers are free
    const bool more = tile + 1 < tile_end;
    dma.target(kvbuf + (cur ^ 1) * TL::BYTES, slot_v);
    if (tile + 2 < tile_end) slot_v = page_table[min((tile + 2) * KV_TILE + lane, N - 1)];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int db = 0; db < DBW; ++db) asm volatile("" : "+v"(o[b][db]));
    tile_compute<R, DR>(kvbuf + cur * TL::BYTES, q, o, st, tile * KV_TILE, L, N, mw0, mw1, scale_log2, pbuf, mxch,
                        psum, wi, wj, wave, lane, dma, more);
  }

  // Partial of this split: O / l rounded to bf16, row-major [split][row][R] so that a row is one contiguous
  // 1 KB line for the combine, plus fp32 (max, sum) per row, [split][row].  The register fragments go to
  // LDS first (the KV buffers are free once every wave has left the loop), then out as whole rows, written
  // through at agent scope (all workgroups store their partials at about the same time, at the end).
  constexpr int OP = R + 8;  // staging pitch (elements): rows 16 B apart in the bank space
  static_assert(M_TILE * OP * 2 <= 2 * TL::BYTES, "O staging must fit in the KV buffers");
  uint16_t* o_s = reinterpret_cast<uint16_t*>(kvbuf);
  __syncthreads();
  if (wave < PvSplit<R>::WAVES) {
    // lane (c, g) holds rows b*32 + c, columns wave*CPW + db*32 + q4*8 + g*4 + 0..3
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const float inv = (st.l[b] > 0.f) ? 1.f / st.l[b] : 0.f;  // a row that saw nothing here has O = 0
      uint16_t* row_s = o_s + (b * 32 + c) * OP + wave * PvSplit<R>::CPW + g * 4;
#pragma unroll
      for (int db = 0; db < DBW; ++db)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          bf16x4 v;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = (__bf16)(o[b][db][q4 * 4 + e] * inv);
          *reinterpret_cast<bf16x4*>(row_s + db * 32 + q4 * 8) = v;
        }
    }
  }
  if (wave == 0 && g == 0) {
#pragma unroll
    for (int b = 0; b < 2; ++b)
      store_agent8(&part_ml[(size_t)split * Mp + mt * M_TILE + b * 32 + c],
                   u32x2{__float_as_uint(st.m_ref[b]), __float_as_uint(st.l[b])});
  }
  __syncthreads();
  uint16_t* dst = part_o + ((size_t)split * Mp + mt * M_TILE) * R;
  constexpr int CPR = R / 8;  // 16-byte chunks per row
  static_assert(M_TILE * CPR % NTHREADS == 0, "partial rows split evenly over the threads");
#pragma unroll 4
  for (int k = 0; k < M_TILE * CPR / NTHREADS; ++k) {
    const int idx = tid + k * NTHREADS, row = idx / CPR, ch = idx % CPR;
    store_agent16(dst + (size_t)row * R + ch * 8, *reinterpret_cast<const u32x4*>(o_s + row * OP + ch * 8));
  }
}

// Workgroup = 4 waves over 64 query rows (m = t*H + h).  Wave (wi, wj) = (w / 2, w % 2): scores of rows wi*32..+31
// against KV rows wj*32..+31 of each tile; values for latent columns w*CPW..+CPW of all 64 rows.
// Two LDS tiles: while one is computed, the next is gathered by DMA (spread over the score MFMAs).
// One segment of the split-KV pass: query tile mt of request rq against its KV tiles [tile_begin, tile_end),
// ending with the partial (O / l, max, sum) of those tiles in partial slot `split` of the request.  All threads
// of the workgroup call it together (it has barriers); it leaves the LDS buffers free for another segment only
// after the caller's next barrier.
template <int R, int DR>
__device__ __forceinline__ void splitkv_segment(const uint16_t* __restrict__ q_cat_all, const uint16_t* __restrict__ c_kv,
                                                const uint16_t* __restrict__ k_pe,
                                                const int32_t* __restrict__ page_table_all,
                                                const uint32_t* __restrict__ mask_all, const ReqArgs& rq, int H,
                                                int mt, int tile_begin, int tile_end, int split, float scale_log2,
                                                uint16_t* __restrict__ part_o_all, float2* __restrict__ part_ml_all,
                                                char* kvbuf, uint4 (*pbuf)[2][2][64], float (*mxch)[2][32],
                                                float (*psum)[2][32]) {
  using TL = TileLayout<R, DR>;
  constexpr int DQ = R + DR;
  const int L = rq.L, T = rq.T, M = rq.T * H, N = rq.N, Mp = rq.Mp;
  const uint16_t* q_cat = q_cat_all + (size_t)rq.node0 * H * DQ;
  const int32_t* page_table = page_table_all + rq.pt0;
  const uint32_t* mask = (N > L) ? mask_all + rq.mask0 : nullptr;
  // (the offsets are materialised here: the compiler would otherwise sink their loads to the epilogue, where
  // they wait; pinning the integers, not the pointers, keeps the stores global rather than flat)
  long long po = rq.po, pml = rq.pml;
  asm volatile("" : "+s"(po), "+s"(pml));
  uint16_t* part_o = part_o_all + po;
  float2* part_ml = part_ml_all + pml;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wi = wave >> 1, c = lane & 31;
  const int m = mt * M_TILE + wi * 32 + c;


  // Prologue.  Each wave first gathers the first tile's page-table slice by DMA into its own 256 bytes of the
  // (still idle) exchange buffer; the mask words load; then the query tile (64 rows of q_cat) is gathered by
  // DMA into the second KV buffer, which is idle until the loop's first iteration.  A counted wait lets the
  // page-table slice land without waiting for the query tile, and the first tile's gather goes out behind it.
  // Each wave then reads its query fragments from LDS.  (Each DMA asm clobbers memory, so no load or LDS
  // access is moved past it.)  Padding rows (m >= M) repeat the last real row; their partials are never read.
  const int me = min(m, M - 1);
  int* pt_s = reinterpret_cast<int*>(&pbuf[0][0][0][0]) + wave * 64;
  dma4_lane_addr(page_table + min(tile_begin * KV_TILE + lane, N - 1), lds_address(pt_s));  // rows past N reuse
  const int t_row = me / H, W = (T + 31) >> 5;                                              // a real row (masked)
  const bool tree_rows = N > L;  // (a prefix-only pass has no tree rows and no mask)
  const uint32_t mw0 = tree_rows ? mask[t_row * W] : 0u;
  const uint32_t mw1 = (tree_rows && W == 2) ? mask[t_row * W + 1] : 0u;
  char* qbuf = kvbuf + TL::BYTES;
  constexpr int QINS = (M_TILE * (DQ / 8) + 63) / 64;  // query-tile DMA instructions (all waves)
  {
    // LDS holds the tile's rows back to back, DQ/8 chunks each; within aligned groups of 8 chunks, chunk ch of
    // row r sits at position ch ^ ((r >> 1) & 7), so the 16 rows a quarter-wave reads at one chunk fall in 16
    // distinct 16-byte bank groups (an involution: the same formula maps a position back to its chunk).
    // Lane l of DMA instruction i fills position i*64 + l.
    constexpr int QC = DQ / 8, QN = (M_TILE * QC + 255) / 256;
    static_assert(M_TILE * QC * 16 <= TL::BYTES, "query tile must fit in one KV buffer");
    const uint32_t qlds = lds_address(qbuf);
#pragma unroll
    for (int k = 0; k < QN; ++k) {
      const int ins = wave + 4 * k, pos = ins * 64 + lane;
      if (ins * 64 < M_TILE * QC) {
        const int r = pos / QC, ch = qswz<QC>(r, pos % QC);
        const int gr = min(mt * M_TILE + r, M - 1);
        dma16_lane_addr(q_cat + (size_t)gr * DQ + ch * 8, qlds + ins * 1024);
      }
    }
  }
  wait_vmem_below<QINS / 4>();  // every wave issued at least QINS / 4 query-tile loads after its page-table load
  const int slot0 = pt_s[lane];
  TileDma<R, DR> dma(c_kv, k_pe, wave, lane);
  dma.target(kvbuf, slot0);
#pragma unroll
  for (int k = 0; k < TileDma<R, DR>::NK; ++k) dma.issue(k);
  int slot_v = 0;
  if (tile_begin + 1 < tile_end) slot_v = page_table[min((tile_begin + 1) * KV_TILE + lane, N - 1)];
  wait_vmem_all();
  __syncthreads();
  seg_body<R, DR>(kvbuf, qbuf, pbuf, mxch, psum, dma, slot_v, page_table, tile_begin, tile_end, L, N, mw0, mw1,
                  scale_log2, mt, split, Mp, part_o, part_ml);
}

// Blocks past the split-KV blocks of a single request run on CUs the split plan leaves idle; they read W_UV into
// the caches ahead of the combine, which gathers W_UV[h] on XCD h mod 8.  Block split_blocks + 8 r + x is XCD x's
// r-th of cnt and reads its share of the heads x, x + 8, ... in whole 64-chunk instructions, by LDS DMA into a
// 1 KB sink per wave that nothing reads, so that all of a wave's loads are in flight together; the wave waits
// for them once, at the end.  hch_log2: log2 of the 16-byte chunks per head (Dv * R / 8, a power of two).
__device__ __forceinline__ void wuv_prefetch(const uint16_t* __restrict__ w_uv, int hch_log2, int H, int x, int r,
                                             int cnt, char* sink) {
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nh = (H - x + NUM_XCD - 1) / NUM_XCD;
  const int tot = nh << hch_log2, per = ((tot + cnt - 1) / cnt + 63) & ~63;
  const int c0 = r * per, c1 = min(tot, c0 + per);
  const uint32_t sl = lds_address(sink) + wave * 1024;
  for (int i = c0 + wave * 64; i < c1; i += NTHREADS) {  // (uniform) chunks i .. i + 63, lane l takes i + l
    const int idx = min(i + lane, c1 - 1);
    const int h = x + NUM_XCD * (idx >> hch_log2);
    dma16_lane_addr(w_uv + (((size_t)h << hch_log2) + (idx & ((1 << hch_log2) - 1))) * 8, sl);
  }
  wait_vmem_all();
}

template <int R, int DR, int NB>
__global__ __launch_bounds__(NTHREADS, 1) void splitkv_kernel(
    const uint16_t* __restrict__ q_cat_all, const uint16_t* __restrict__ c_kv, const uint16_t* __restrict__ k_pe,
    const int32_t* __restrict__ page_table_all, const uint32_t* __restrict__ mask_all, const BatchArgs<NB> ba,
    float scale_log2, uint16_t* __restrict__ part_o_all, float2* __restrict__ part_ml_all,
    const int32_t* __restrict__ dbg, const uint16_t* __restrict__ w_uv_pf, int pf_hch_log2) {
  using TL = TileLayout<R, DR>;
  if (dbg != nullptr && *dbg != KDV_OK) return;  // page table failed its check: no gather (uniform)
  __shared__ __attribute__((aligned(1024))) char kvbuf[2 * TL::BYTES];
  __shared__ uint4 pbuf[2][2][2][64];  // [row block][kv half][16-row k-step][lane]: P^T fragments (bf16)
  __shared__ float mxch[2][2][32];     // [row block][kv half][row]: proposed reference
  __shared__ float psum[2][2][32];     // [row block][kv half][row]: half-tile row sum

  if (NB > 1 && ba.sk_w > 0) {
    // Stream-K plan of a batch: the KV tiles of all requests, concatenated, are dealt out in equal contiguous
    // runs, one per group of sk_g workgroups; member j of a group takes query tile j of every request its run
    // touches (one segment per request), so a group's members read the same KV tiles at the same time, as the
    // query tiles of one split do.  Groups are laid out contiguously over the XCDs (slots lin*x .. lin*x+lin-1
    // on XCD x).  A request's partial slots are the runs that touch it: slot = group - (first such group).
    const int k = (int)(blockIdx.x % NUM_XCD) * ba.sk_lin + (int)(blockIdx.x / NUM_XCD);
    const int gi = k / ba.sk_g, mj = k % ba.sk_g;
    if (gi >= ba.sk_groups) return;  // spare slot (uniform; before any barrier)
    const long long p1 = min((long long)(gi + 1) * ba.sk_w, ba.sk_u);
    for (long long p = (long long)gi * ba.sk_w; p < p1;) {
      int rqi = 0;
      while (rqi + 1 < ba.n && p >= ba.r[rqi + 1].sk_base) ++rqi;  // (uniform scalar search)
      const ReqArgs& rq = ba.r[rqi];
      const long long nt = (rq.N + KV_TILE - 1) / KV_TILE, seg_end = min(p1, rq.sk_base + nt);
      if (mj < rq.m_tiles)  // (uniform)
        splitkv_segment<R, DR>(q_cat_all, c_kv, k_pe, page_table_all, mask_all, rq, ba.H, mj, (int)(p - rq.sk_base),
                               (int)(seg_end - rq.sk_base), (int)(gi - rq.sk_base / ba.sk_w), scale_log2,
                               part_o_all, part_ml_all, kvbuf, pbuf, mxch, psum);
      p = seg_end;
      __syncthreads();  // the next segment's DMAs reuse the LDS the epilogue read
    }
    return;
  }

  // This workgroup's request; its arrays start at the request's offsets.
  const int rqi = NB > 1 ? request_of(ba.blk_split, ba.n, blockIdx.x) : 0;  // (a constant index for one request)
  const ReqArgs& rq = ba.r[rqi];
  const int m_tiles = rq.m_tiles;
  // Workgroups are dealt to the XCDs round-robin (block b -> XCD b % NUM_XCD; a request's first block is a
  // multiple of NUM_XCD).  Every query tile of one KV split is kept on one XCD so that split's rows are fetched
  // into that XCD's L2 once and then shared; the request's splits start at XCD xoff.  With the contiguous
  // placement (lin > 0) XCD x instead takes the (split, query tile) pairs lin*x .. lin*x + lin - 1 in split-major
  // order: a split straddles at most two XCDs, and the grid can use every CU when the query tiles do not
  // divide an XCD's CUs.
  const int bid = blockIdx.x - ba.blk_split[rqi];
  const int xcd = bid % NUM_XCD, j = bid / NUM_XCD;
  const int kl = xcd * rq.lin + j;
  const int split = rq.lin > 0 ? kl / m_tiles : (xcd - rq.xoff + NUM_XCD) % NUM_XCD + NUM_XCD * (j / m_tiles);
  const int mt = rq.lin > 0 ? kl % m_tiles : j % m_tiles;
  // A padding block, or one past the split blocks (only with a single request), which reads W_UV ahead (uniform; before
  // any barrier; the test comes after the placement so that its argument loads go out with the others)
  if (split >= rq.splits || (NB == 1 && (int)blockIdx.x >= ba.blk_split[1])) {
    if (NB == 1 && (int)blockIdx.x >= ba.blk_split[1] && w_uv_pf != nullptr) {
      const int e = blockIdx.x - ba.blk_split[1];
      wuv_prefetch(w_uv_pf, pf_hch_log2, ba.H, e % NUM_XCD, e / NUM_XCD, (gridDim.x - ba.blk_split[1]) / NUM_XCD,
                   kvbuf);
    }
    return;
  }
  const int ntiles = (rq.N + KV_TILE - 1) / KV_TILE;
  const int tile_begin = split * rq.tiles_per_split;
  const int tile_end = min(tile_begin + rq.tiles_per_split, ntiles);
  splitkv_segment<R, DR>(q_cat_all, c_kv, k_pe, page_table_all, mask_all, rq, ba.H, mt, tile_begin, tile_end, split,
                         scale_log2, part_o_all, part_ml_all, kvbuf, pbuf, mxch, psum);
}

// ------------------------------------------------------------------------------------------------ q_absorb
// grid (H, ceil(R/128), ceil(T/32)); each wave produces 32 latent columns of head h for the workgroup's 32 nodes.
// MFMA D[r][t] = sum_k W_UK[h][k][r] q_nope[t,h][k]: the A operand W^T is read from LDS with transposed
// reads (W_UK is stored k-major), the B operand straight from global memory.
// The W_UK block arrives by LDS DMA (an LDS-DMA gather moves about 2.5 times the bytes per CU that loads into
// registers do).  LDS rows are RB/8 = 16 chunks of 16 bytes with chunk c of row k at c ^ 4*(k % 4): a
// transposed read's 32 lanes cover 4 aligned rows x 4 aligned chunks, which then fall in 16 distinct bank
// groups.  DMA instruction i fills rows 4i..4i+3, lane l the row's position l % 16.
// The absorption of one (head h, 128-column block cb, 32-node block from t_base) piece of q_cat, by the four waves
// of a workgroup; w_s: LDS for the W_UK block (DN x 128 bf16).
template <int DN, int R, int DR>
__device__ __forceinline__ void absorb_block(const uint16_t* __restrict__ q_nope, const uint16_t* __restrict__ q_rope,
                                             const uint16_t* __restrict__ w_uk, uint16_t* __restrict__ q_cat, int T,
                                             int H, int h, int cb, int t_base, char* w_s) {
  constexpr int DQ = R + DR;
  constexpr int RB = 128;                    // latent columns per workgroup
  constexpr int WINS = DN * RB * 2 / 1024;   // DMA instructions for the W_UK block
  static_assert(WINS % 4 == 0, "W_UK block must split evenly over the four waves");
  const int r0 = cb * RB;
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, c = lane & 31;

  {
    const char* wh = reinterpret_cast<const char*>(w_uk + (size_t)h * DN * R);
    const uint32_t wl = lds_address(w_s);
#pragma unroll
    for (int k4 = 0; k4 < WINS / 4; ++k4) {
      const int ins = wave + 4 * k4;
      const int k = ins * 4 + (lane >> 4);
      const int col = r0 + (((lane & 15) ^ (4 * (k & 3))) << 3);
      if (col < R) dma16_lane_addr(wh + ((size_t)k * R + col) * 2, wl + ins * 1024);  // (columns past R: never read)
    }
  }
  // query fragments of this workgroup's 32 nodes; rows past T load node T-1 (their results are never stored)
  bf16x8 qb[DN / 16];
  {
    const int tq = min(t_base + c, T - 1);
#pragma unroll
    for (int kb = 0; kb < DN / 16; ++kb) qb[kb] = load_bf16x8(q_nope + ((size_t)tq * H + h) * DN + kb * 16 + g * 8);
  }
  // The rotary part of q_cat is a copy (first column of workgroups, one 16-byte chunk per thread): loaded here
  // with the other loads, stored after the product, so that no store acknowledgement is waited for before it.
  constexpr int RCH = 32 * (DR / 8);  // rotary chunks of 32 nodes
  static_assert(RCH <= NTHREADS, "one rotary chunk per thread");
  const int rt = t_base + tid / (DR / 8), rcol = (tid % (DR / 8)) * 8;
  const bool rcopy = cb == 0 && tid < RCH && rt < T;
  uint4 rv = make_uint4(0u, 0u, 0u, 0u);
  if (rcopy) rv = *reinterpret_cast<const uint4*>(q_rope + ((size_t)rt * H + h) * DR + rcol);
  wait_vmem_all();
  __syncthreads();
  if (rcopy) *reinterpret_cast<uint4*>(q_cat + (size_t)(rt * H + h) * DQ + R + rcol) = rv;
  const int rs = wave * 32;
  if (r0 + rs >= R) return;  // wave-uniform; no barrier follows
  // lane's transposed-read position: rows kb*16 + g*8 + (lane%16)/4 (+4), chunk rs/8 + cl, byte sub
  const int cl = ((lane & 31) >> 4) * 2 + ((lane & 3) >> 1), sub = (lane & 1) * 8;
  auto wread = [&](int krow) -> i16x4 {
    return lds_read_tr16(w_s + krow * (RB * 2) + (((rs / 8 + cl) ^ (4 * (krow & 3))) << 4) + sub);
  };
  {
    f32x16 acc = zero16();
    const int t = t_base + c;
#pragma unroll
    for (int kb = 0; kb < DN / 16; ++kb) {
      const int krow = kb * 16 + g * 8 + ((lane & 15) >> 2);
      const bf16x8 a = concat_tr(wread(krow), wread(krow + 4));
      acc = mfma32(a, qb[kb], acc);
    }
    if (t < T) {
      uint16_t* dst = q_cat + (size_t)(t * H + h) * DQ + r0 + rs + g * 4;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        bf16x4 v;
        v[0] = (__bf16)acc[q4 * 4 + 0];
        v[1] = (__bf16)acc[q4 * 4 + 1];
        v[2] = (__bf16)acc[q4 * 4 + 2];
        v[3] = (__bf16)acc[q4 * 4 + 3];
        *reinterpret_cast<bf16x4*>(dst + q4 * 8) = v;
      }
    }
  }
}

template <int DN, int R, int DR>
__global__ __launch_bounds__(NTHREADS) void q_absorb_kernel(const uint16_t* __restrict__ q_nope,
                                                            const uint16_t* __restrict__ q_rope,
                                                            const uint16_t* __restrict__ w_uk,
                                                            uint16_t* __restrict__ q_cat, int T, int H,
                                                            const int32_t* __restrict__ parent,
                                                            uint32_t* __restrict__ mask,
                                                            int32_t* __restrict__ status,
                                                            const int32_t* __restrict__ dbg) {
  if (dbg != nullptr && *dbg != KDV_OK && blockIdx.x != H) return;  // page table failed its check (uniform)
  if (blockIdx.x == H) {  // a call that builds its own tree mask has one extra column of blocks (uniform exit)
    if (blockIdx.y == 0 && blockIdx.z == 0 && threadIdx.x < 64)
      build_ancestor_mask(parent, T, mask, status, threadIdx.x);
    return;
  }
  __shared__ __attribute__((aligned(1024))) char w_s[DN * 128 * 2];
  // this workgroup: head blockIdx.x, latent columns blockIdx.y * 128 .. +127, nodes blockIdx.z * 32 .. +31
  absorb_block<DN, R, DR>(q_nope, q_rope, w_uk, q_cat, T, H, blockIdx.x, blockIdx.y, blockIdx.z * 32, w_s);
}

// ------------------------------------------------------------------------------------------------ combine + W_UV
// Merging the splits: o[m] = sum_s 2^(m_s - M) O_s[m] / sum_s 2^(m_s - M) l_s and
// lse[m] = ln 2 * (M + log2 sum_s 2^(m_s - M) l_s), M = max_s m_s, with O_s stored as O_s / l_s in bf16
// (so its weight is 2^(m_s - M) l_s); a split in which row m saw nothing has m_s = -inf, l_s = 0, weight 0.
// The merged latent row, rounded to bf16, goes through the value up-projection right away:
// out[t,h][v] = sum_r W_UV[h][v][r] o[t,h][r].
//
// One workgroup of 8 waves per (head, block of RT nodes).  Workgroups are dealt to the XCDs round-robin, and
// the node blocks of one head are kept on one XCD, so W_UV[h] is fetched into that XCD's L2 once.  The waves
// split the fetching so that none waits for the other's loads (a wave's load counter is in order):
//   - waves 0..3 load the partials of the RT rows into registers and merge them (CPT 16-byte chunks of a row
//     per thread, over every SP-th split; see below);
//   - waves 4..7 gather all of W_UV[h] into LDS by DMA (an LDS-DMA gather moves about 2.5 times the
//     bytes per CU that loads into registers do; the issue cost of a DMA instruction is per wave, so four
//     waves share it).  Chunk ch of W row r sits at position ch ^ (r % WSW) of the row, so the MFMA's
//     quarter-wave reads (16 rows, one chunk) hit 16 distinct bank groups.
// Once the merged rows and W_UV are in LDS (one barrier; two when the split groups' sums meet in LDS first),
// wave w < DV/32 computes D[v][t] = sum_r W_UV[h][v][r] o[t][r] for its 32 columns v, both operands read from
// LDS (r-contiguous); columns t >= RT of the product repeat the last row, never stored.
constexpr int COMB_THREADS = 512;
// RT = tree nodes per workgroup: 4; 2 or 1 when a call has few heads and nodes, so that the grid still fills the
// device; 16 for a batch whose 4-node grid would exceed the CUs (fewer W_UV gathers).  A merging thread takes
// CPT chunks (1, or 4 for 16 nodes).  When the rows have fewer chunks than there are merging threads, the
// threads are split into SP groups that take every SP-th split of the same chunks; the groups' running (max,
// sum, numerators) meet in LDS and are combined in a fixed order.
// Merge of the splits of RT rows (one head, nodes t0 .. t0 + nrow - 1) and their W_UV product, by one workgroup of
// THREADS threads.  With 512 threads waves 4..7 gather W_UV while waves 0..3 merge; with 256 the four waves issue
// the W_UV gather first and then merge.  LDS: w_s (DV x R bf16, 1 KB aligned), o_s (RT merged rows), gx (split
// groups' running sums).  Same arithmetic in both forms.
template <int R, int DV, int RT, int THREADS>
__device__ __forceinline__ void combine_block(const uint16_t* __restrict__ part_o, const float2* __restrict__ part_ml,
                                              int S, int Mp, const uint16_t* __restrict__ w_uv,
                                              uint16_t* __restrict__ out, float* __restrict__ lse, int H, int h,
                                              int t0, int nrow, char* w_s, uint16_t* o_s, float* gx) {
  constexpr bool SEP = THREADS == 512;
  static_assert(THREADS == 512 || THREADS == 256, "8 or 4 waves");
  constexpr int CPR = R / 8;                 // 16-byte chunks per latent row
  constexpr int KS = R / 16;                 // MFMA k-steps
  constexpr int OP = R + 8;                  // LDS pitch of a merged row (elements)
  constexpr int NFW = 4;                     // fetching waves (4..7); waves 0..3 merge
  constexpr int RC = RT * CPR;               // chunks of the workgroup's rows
  constexpr int CPT = RC > 256 ? RC / 256 : 1;  // chunks per merging thread (16 nodes: 4)
  constexpr int RCT = RC / CPT;              // merging threads per split group
  constexpr int SP = 256 / RCT >= 4 ? 4 : (256 / RCT >= 2 ? 2 : 1);  // split groups merged side by side
  constexpr int MT = RCT * SP;               // merging threads (in waves 0..3)
  // splits whose loads are in flight together (17: the most the plan gives 15 query tiles on 256 CUs; fewer
  // when a thread merges several chunks, to bound its registers)
  constexpr int CH = CPT == 1 ? 17 : 16 / CPT;
  constexpr int WSW = CPR < 16 ? CPR : 16;   // W_UV staging swizzle width (chunks)
  constexpr int WBYTES = DV * R * 2;         // all of W_UV[h]
  constexpr int WINS = WBYTES / 1024 / NFW;  // DMA instructions per fetching wave
  static_assert(RC % CPT == 0 && CPR % CPT == 0 && MT <= 256 && (CPT == 1 || SP == 1), "merging threads");
  static_assert(DV % 32 == 0 && DV / 32 <= 4, "one merging wave per 32 output columns");
  static_assert(WBYTES % (1024 * NFW) == 0, "W_UV must split evenly over the fetching waves");
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, c = lane & 31;
  constexpr float LN2 = 0.69314718055994530942f;
  if (!SEP || wave >= 8 - NFW) {
    // ---- W_UV[h] -> LDS: lane l of instruction i fills position (i*64 + l) of the swizzled rows
    const char* wsrc = reinterpret_cast<const char*>(w_uv + (size_t)h * DV * R);
    const uint32_t wl = lds_address(w_s);
#pragma unroll
    for (int k = 0; k < WINS; ++k) {
      const int ins = (SEP ? wave - (8 - NFW) : wave) + NFW * k;
      const int pos = ins * 64 + lane, r = pos / CPR, p = pos % CPR;
      dma16_lane_addr(wsrc + (size_t)r * (R * 2) + ((p ^ (r & (WSW - 1))) << 4), wl + ins * 1024);
    }
    if (SEP) wait_vmem_all();
  }
  if ((!SEP || wave < 8 - NFW) && tid < MT) {
    // ---- merge: thread handles chunks k0 .. k0 + CPT - 1 of row i over splits sp, sp + SP, ... (all if SP = 1)
    const int col = SP == 1 ? tid : tid % RCT, sp = SP == 1 ? 0 : tid / RCT;
    const int i = col * CPT / CPR, k0 = col * CPT % CPR;
    const int t = t0 + min(i, nrow - 1);  // rows past the last node repeat it (never stored)
    const int m = t * H + h;
    const bf16x8* src = reinterpret_cast<const bf16x8*>(part_o + (size_t)m * R) + k0;
    const size_t stride = (size_t)Mp * CPR;  // bf16x8 per split
    float mx = -INFINITY, den = 0.f;
    float num[CPT][8];
#pragma unroll
    for (int u = 0; u < CPT; ++u)
#pragma unroll
      for (int e = 0; e < 8; ++e) num[u][e] = 0.f;
    // This group's splits are taken CH at a time.  Within a batch the reference is the batch's largest m_s, so
    // each split costs one fused multiply-add per element; the running sums are rescaled once per further batch.
    for (int s0 = 0; sp + s0 * SP < S; s0 += CH) {  // split of batch slot q: sp + (s0 + q) * SP
      float2 ml[CH];
      bf16x8 v[CH][CPT];
      if constexpr (CPT == 1 && CPR == 64) {
        // A row's 64 chunks fill a wave here, so the wave's lanes share one row and one split group: lane q loads
        // slot q's (max, sum) and every lane reads the CH pairs back from lanes 0 .. CH - 1 (one load instruction
        // per batch instead of CH).
        const int sl = min(sp + (s0 + min(lane, CH - 1)) * SP, S - 1);  // past S: repeat split S - 1 (weight 0)
        const float2 ml_l = part_ml[(size_t)sl * Mp + m];
#pragma unroll
        for (int q = 0; q < CH; ++q) v[q][0] = src[min(sp + (s0 + q) * SP, S - 1) * stride];
#pragma unroll
        for (int q = 0; q < CH; ++q) {
          ml[q].x = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, ml_l.x), q));
          ml[q].y = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, ml_l.y), q));
        }
      } else {
#pragma unroll
        for (int q = 0; q < CH; ++q) {
          const int sq = min(sp + (s0 + q) * SP, S - 1);  // past S: repeat split S - 1 (weight 0 below)
          ml[q] = part_ml[(size_t)sq * Mp + m];
#pragma unroll
          for (int u = 0; u < CPT; ++u) v[q][u] = src[sq * stride + u];
        }
      }
      float gm = -INFINITY;
#pragma unroll
      for (int q = 0; q < CH; ++q) gm = (sp + (s0 + q) * SP < S) ? fmaxf(gm, ml[q].x) : gm;
      const float mn = fmaxf(mx, gm);
      // (no early exit when nothing is visible yet, mn = -inf: the sums are 0 and every weight below is 0, and
      // without a branch here the partials' loads go out with the (max, sum) loads instead of after them)
      if (s0 > 0) {
        const float a = (mn == -INFINITY) ? 1.f : fast_exp2(mx - mn);  // mx = -inf < mn -> 0 (the sums are 0)
        den *= a;
#pragma unroll
        for (int u = 0; u < CPT; ++u)
#pragma unroll
          for (int e = 0; e < 8; ++e) num[u][e] *= a;
      }
#pragma unroll
      for (int q = 0; q < CH; ++q) {
        // weight 0 for a split past S or one in which row m saw nothing
        const float wq =
            (sp + (s0 + q) * SP < S && ml[q].x != -INFINITY) ? fast_exp2(ml[q].x - mn) * ml[q].y : 0.f;
        den += wq;
#pragma unroll
        for (int u = 0; u < CPT; ++u)
#pragma unroll
          for (int e = 0; e < 8; ++e) num[u][e] = fmaf(wq, (float)v[q][u][e], num[u][e]);
      }
      mx = mn;
    }
    if constexpr (SP == 1) {
      const float inv = 1.f / den;
#pragma unroll
      for (int u = 0; u < CPT; ++u) {
        bf16x8 ov;
#pragma unroll
        for (int e = 0; e < 8; ++e) ov[e] = (__bf16)(num[u][e] * inv);
        *reinterpret_cast<bf16x8*>(&o_s[i * OP + (k0 + u) * 8]) = ov;
      }
      if (lse != nullptr && k0 == 0 && i < nrow) lse[m] = (mx + log2f(den)) * LN2;
    } else {
      float* x = gx + (sp * RCT + col) * 10;
      x[0] = mx;
      x[1] = den;
#pragma unroll
      for (int e = 0; e < 8; ++e) x[2 + e] = num[0][e];
    }
  }
  if (!SEP) wait_vmem_all();  // (the W_UV gather of the merging waves)
  if constexpr (SP > 1) {
    __syncthreads();  // every group's running sums are in LDS
    if (tid < RCT) {
      // groups in a fixed order; a group that saw nothing (max -inf, sums 0) gets weight 0
      const int i = tid / CPR, k0 = tid % CPR;
      float M = -INFINITY;
#pragma unroll
      for (int q = 0; q < SP; ++q) M = fmaxf(M, gx[(q * RCT + tid) * 10]);
      float den = 0.f, num[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) num[e] = 0.f;
#pragma unroll
      for (int q = 0; q < SP; ++q) {
        const float* x = gx + (q * RCT + tid) * 10;
        const float a = (x[0] == -INFINITY) ? 0.f : fast_exp2(x[0] - M);
        den = fmaf(a, x[1], den);
#pragma unroll
        for (int e = 0; e < 8; ++e) num[e] = fmaf(a, x[2 + e], num[e]);
      }
      const float inv = 1.f / den;
      bf16x8 ov;
#pragma unroll
      for (int e = 0; e < 8; ++e) ov[e] = (__bf16)(num[e] * inv);
      *reinterpret_cast<bf16x8*>(&o_s[i * OP + k0 * 8]) = ov;
      const int t = t0 + min(i, nrow - 1);
      if (lse != nullptr && k0 == 0 && i < nrow) lse[t * H + h] = (M + log2f(den)) * LN2;
    }
  }
  __syncthreads();  // merged rows and W_UV are in LDS
  if (wave * 32 >= DV) return;  // wave-uniform; no barrier follows

  // all W fragments first (one round of LDS latency), then two independent accumulation chains
  const char* wrow = w_s + (wave * 32 + c) * (R * 2);
  const int wsz = (wave * 32 + c) & (WSW - 1);
  bf16x8 wf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) wf[ks] = *reinterpret_cast<const bf16x8*>(wrow + (((2 * ks + g) ^ wsz) << 4));
  f32x16 acc0 = zero16(), acc1 = zero16();
  const uint16_t* orow = o_s + min(c, RT - 1) * OP + g * 8;
#pragma unroll
  for (int ks = 0; ks < KS; ks += 2) {
    acc0 = mfma32(wf[ks], *reinterpret_cast<const bf16x8*>(orow + ks * 16), acc0);
    acc1 = mfma32(wf[ks + 1], *reinterpret_cast<const bf16x8*>(orow + (ks + 1) * 16), acc1);
  }
  if (c < nrow) {
    uint16_t* dst = out + ((size_t)(t0 + c) * H + h) * DV + wave * 32 + g * 4;
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      bf16x4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = (__bf16)(acc0[q4 * 4 + e] + acc1[q4 * 4 + e]);
      *reinterpret_cast<bf16x4*>(dst + q4 * 8) = v;
    }
  }
}

// NaN results for the rows of one combine block (page table failed the KDV_DEBUG check).
template <int DV, int THREADS>
__device__ __forceinline__ void combine_block_nan(uint16_t* __restrict__ out, float* __restrict__ lse, int H, int h,
                                                  int t0, int nrow) {
  const int tid = threadIdx.x;
  for (int k = tid; k < nrow * DV; k += THREADS) out[((size_t)(t0 + k / DV) * H + h) * DV + k % DV] = 0x7FC0;
  if (lse != nullptr && tid < nrow) lse[(t0 + tid) * H + h] = __builtin_nanf("");
}

template <int R, int DV, int NB, int RT>
__global__ __launch_bounds__(COMB_THREADS) void combine_up_kernel(const uint16_t* __restrict__ part_o_all,
                                                              const float2* __restrict__ part_ml_all,
                                                              const BatchArgs<NB> ba,
                                                              const uint16_t* __restrict__ w_uv,
                                                              uint16_t* __restrict__ out_all,
                                                              float* __restrict__ lse_all,
                                                              const int32_t* __restrict__ dbg) {
  // LDS sizes (combine_block holds the layout and checks the shapes)
  constexpr int CPR = R / 8;                 // 16-byte chunks per latent row
  constexpr int OP = R + 8;                  // LDS pitch of a merged row (elements)
  constexpr int RC = RT * CPR;               // chunks of the workgroup's rows
  constexpr int CPT = RC > 256 ? RC / 256 : 1;  // chunks per merging thread (16 nodes: 4)
  constexpr int RCT = RC / CPT;              // merging threads per split group
  constexpr int SP = 256 / RCT >= 4 ? 4 : (256 / RCT >= 2 ? 2 : 1);  // split groups merged side by side
  constexpr int WBYTES = DV * R * 2;         // all of W_UV[h]
  __shared__ __attribute__((aligned(16))) uint16_t o_s[RT * OP];
  __shared__ __attribute__((aligned(1024))) char w_s[WBYTES];
  __shared__ float gx[(SP > 1 ? SP * RCT : 1) * 10];  // per split group: max, sum, 8 numerators
  const int rqi = NB > 1 ? request_of(ba.blk_comb, ba.n, blockIdx.x) : 0;
  const ReqArgs& rq = ba.r[rqi];
  const int T = rq.T, H = ba.H;
  // (offsets loaded up front rather than next to their first use; pinning integers, not pointers, keeps the
  // memory accesses global rather than flat)
  long long po = rq.po, pml = rq.pml, obase = (long long)rq.node0 * H;
  int S = rq.splits, Mp = rq.Mp;
  asm volatile("" : "+s"(po), "+s"(pml), "+s"(obase), "+s"(S), "+s"(Mp));
  const uint16_t* part_o = part_o_all + po;
  const float2* part_ml = part_ml_all + pml;
  uint16_t* out = out_all + obase * DV;
  float* lse = (lse_all != nullptr) ? lse_all + obase : nullptr;
  const int bid = blockIdx.x - ba.blk_comb[rqi];  // (a request's first block is a multiple of NUM_XCD)
  const int xcd = bid % NUM_XCD, j = bid / NUM_XCD;
  const int TB = (T + RT - 1) / RT;
  const int h = xcd + NUM_XCD * (j / TB), t0 = (j % TB) * RT;
  if (h >= H) return;  // padding block (uniform; before any barrier)
  const int nrow = min(RT, T - t0);
  if (dbg != nullptr && *dbg != KDV_OK) {  // page table failed its check: NaN results, nothing gathered (uniform)
    combine_block_nan<DV, COMB_THREADS>(out, lse, H, h, t0, nrow);
    return;
  }
  combine_block<R, DV, RT, COMB_THREADS>(part_o, part_ml, S, Mp, w_uv, out, lse, H, h, t0, nrow, w_s, o_s, gx);
}

// ------------------------------------------------------------------------------------------------ short sequence
// When a single request's whole KV sequence fits in one tile (N = L + T <= 64 rows) and its tree has at most 32
// nodes, the whole call is one kernel: no q_cat, no partials, no second or third launch.  Workgroup (h, j) works on
// head h and output columns v0 = j*VC .. v0 + VC - 1:
//   absorb  the W_UK[h] rows are staged in LDS (rows of R columns, 16-byte chunks XOR-swizzled as a KV tile's
//           latent rows) and every wave computes q_lat^T[r][t] = sum_k W_UK[h][k][r] q_nope[t,h][k] for R/4 latent
//           columns r of the T <= 32 nodes t (A = W^T by transposed reads, B = q_nope from global);
//   q tile  q_lat (bf16, as q_cat holds it) and q_rope go to LDS as 32 rows of R + DR elements, once W_UK is
//           consumed; meanwhile the N KV rows and the workgroup's W_UV rows are gathered into the space W_UK held;
//   scores  S^T[n][t] = K[n] . Q[t]: wave (key block nb = w % 2, contraction half kh = w / 2), 32 keys x 32 nodes;
//           the two halves meet in LDS;
//   softmax waves 0 and 1 (one key block each; row maxima and sums meet in LDS), each row's own maximum as the
//           reference (one tile: no running rescale); P^T fragments to LDS in the value MFMA's operand order;
//   values  O^T[r][t] = sum_n V^T[r][n] P^T[n][t] over the tile: each wave R/4 latent columns; o = O / l (bf16, as
//           the combine rounds it) goes over the tile's LDS;
//   output  D[v][t] = sum_r W_UV[h][v0 + v][r] o[t][r], the contraction split over the waves and summed in LDS.
// A call that builds its tree mask builds the T rows it needs in every workgroup (one wave, in LDS); workgroup
// (0, 0) also writes the mask and the tree status for the caller.
// Rows n >= N of the tile repeat row N - 1 and are masked; node rows t >= T repeat node T - 1, never stored.
template <int DN, int R, int DR, int DV>
struct ShortLayout {
  using TL = TileLayout<R, DR>;
  static constexpr int DQ = R + DR;
  static constexpr int VC = 32;                          // output columns per workgroup
  static constexpr int QP = DQ + 8;                      // q-tile row pitch (elements)
  static constexpr int OP = R + 8;                       // latent output row pitch (elements)
  static constexpr int KV_OFF = 0, WUV_OFF = TL::BYTES, QT_OFF = WUV_OFF + VC * R * 2;
  static constexpr int WUK_BYTES = DN * R * 2;
  static constexpr int QT_BYTES = 32 * QP * 2;
  static constexpr int BYTES = (QT_OFF + QT_BYTES > WUK_BYTES ? QT_OFF + QT_BYTES : WUK_BYTES);
  static_assert(DV % VC == 0, "output column blocks");
  static_assert(32 * OP * 2 <= TL::BYTES, "the latent output rows fit in the KV tile's LDS");
  static_assert((WUK_BYTES / 1024) % 4 == 0 && (VC * R * 2 / 1024) % 4 == 0, "DMA rows split over four waves");
};

template <int DN, int R, int DR, int DV>
__global__ __launch_bounds__(NTHREADS) void short_verify_kernel(
    const uint16_t* __restrict__ q_nope, const uint16_t* __restrict__ q_rope, const uint16_t* __restrict__ w_uk,
    const uint16_t* __restrict__ w_uv, const uint16_t* __restrict__ c_kv, const uint16_t* __restrict__ k_pe,
    const int32_t* __restrict__ page_table, const int32_t* __restrict__ parent, uint32_t* __restrict__ mask,
    int32_t* __restrict__ tree_status, int L, int T, int H, float scale_log2, uint16_t* __restrict__ out,
    float* __restrict__ lse, const int32_t* __restrict__ dbg) {
  using SL = ShortLayout<DN, R, DR, DV>;
  using TL = TileLayout<R, DR>;
  using PV = PvSplit<R>;
  constexpr int DQ = R + DR, KB = DQ / 16;  // score k-steps
  constexpr bool EVEN = KB % 2 == 0;        // split over the two wave halves (odd KB, narrow test shape: half 0)
  constexpr int KH0 = EVEN ? KB / 2 : KB;   // k-steps per scoring wave
  constexpr int VC = SL::VC, KQ = 4, KS = R / 16, KSQ = KS / KQ;
  constexpr int CK = R / 8, CPR = R / 8, WSW = CPR < 16 ? CPR : 16, OP = SL::OP, QP = SL::QP;
  constexpr int AW = R / 32 < 4 ? R / 32 : 4;  // waves that absorb (R / 32 latent column blocks over them)
  constexpr int RBW = R / 32 / AW;             // 32-column blocks per absorbing wave
  constexpr int NKB = DN / 16;                 // absorption k-steps
  constexpr int WUK_INS = SL::WUK_BYTES / 1024, WUV_INS = VC * R * 2 / 1024;  // DMA instructions (all waves)
  constexpr float LN2 = 0.69314718055994530942f;
  static_assert(KS % KQ == 0 && R % 32 == 0 && DN % 16 == 0, "shapes");
  __shared__ __attribute__((aligned(1024))) char smem[SL::BYTES];
  __shared__ uint4 pfr[4][64];        // P^T fragments of the tile's four 16-row k-steps (bf16), lane order
  __shared__ float red[3][16][64];    // partial sums exchanged between waves [part][register][lane]
  __shared__ float mx[2][32], sm[2][32];  // per key block: row maximum (unscaled), row sum
  __shared__ uint32_t smask[64];      // ancestor rows, when the call builds them
  char* kvbuf = smem + SL::KV_OFF;
  char* w_s = smem + SL::WUV_OFF;
  uint16_t* q_s = reinterpret_cast<uint16_t*>(smem + SL::QT_OFF);

  const int h = blockIdx.x, v0 = blockIdx.y * VC;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, c = lane & 31;
  const int N = L + T, tq = min(c, T - 1);
  if (parent != nullptr && wave == 0) {
    build_ancestor_mask(parent, T, smask, nullptr, lane);
    if (blockIdx.x == 0 && blockIdx.y == 0) build_ancestor_mask(parent, T, mask, tree_status, lane);
  }
  if (dbg != nullptr && *dbg != KDV_OK) {  // page table failed its check: NaN results, nothing gathered (uniform)
    for (int k = tid; k < T * VC; k += NTHREADS) out[((size_t)(k / VC) * H + h) * DV + v0 + k % VC] = 0x7FC0;
    if (lse != nullptr && blockIdx.y == 0 && tid < T) lse[tid * H + h] = __builtin_nanf("");
    return;
  }

  // ---- W_UK[h] into LDS (lane l of instruction i fills position i*64 + l of the swizzled rows), then the
  // ordinary loads: the absorption's q_nope fragments, the q_rope chunks of the q tile, the page-table entries
  {
    const char* src = reinterpret_cast<const char*>(w_uk + (size_t)h * DN * R);
    const uint32_t base = lds_address(smem);
#pragma unroll 4
    for (int k = 0; k < WUK_INS / 4; ++k) {
      const int ins = wave + 4 * k, pos = ins * 64 + lane, row = pos / CK, p = pos % CK;
      dma16_lane_addr(src + (size_t)row * (R * 2) + ((p ^ swz<CK>(row)) << 4), base + ins * 1024);
    }
  }
  bf16x8 qn[NKB];
  {
    const uint16_t* qrow = q_nope + ((size_t)tq * H + h) * DN + g * 8;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) qn[kb] = load_bf16x8(qrow + kb * 16);
  }
  constexpr int RCH = DR / 8;  // 16-byte chunks of a q_rope row
  const int rrow = tid / RCH, rch = tid % RCH;
  uint4 rv = make_uint4(0u, 0u, 0u, 0u);
  if (rrow < 32) rv = *reinterpret_cast<const uint4*>(q_rope + ((size_t)min(rrow, T - 1) * H + h) * DR + rch * 8);
  const int slot = page_table[min(lane, N - 1)];
  wait_vmem_all();
  __syncthreads();  // W_UK is in LDS (and the mask rows, when built here)
  const uint32_t mw = parent != nullptr ? smask[tq] : mask[tq];  // T <= 32: one word per node

  // ---- absorption: wave w < AW, latent column blocks w*RBW .. +RBW-1; D[r][t] in registers
  f32x16 qa[RBW];
#pragma unroll
  for (int b = 0; b < RBW; ++b) qa[b] = zero16();
  if (wave < AW) {
    const int cl = ((lane & 31) >> 4) * 2 + ((lane & 3) >> 1), sub = (lane & 1) * 8;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      const int krow = kb * 16 + g * 8 + ((lane & 15) >> 2);
#pragma unroll
      for (int b = 0; b < RBW; ++b) {
        const int ch = (wave * RBW + b) * 4 + cl;
        const bf16x8 a = concat_tr(lds_read_tr16(smem + TL::ckv(krow, ch) + sub),
                                   lds_read_tr16(smem + TL::ckv(krow + 4, ch) + sub));
        qa[b] = mfma32(a, qn[kb], qa[b]);
      }
    }
  }
  __syncthreads();  // W_UK is consumed: its LDS takes the KV tile, the W_UV rows and the q tile

  // ---- the KV rows and this workgroup's W_UV rows by DMA; the q tile (bf16) into LDS
  TileDma<R, DR> dma(c_kv, k_pe, wave, lane);
  dma.target(kvbuf, slot);
#pragma unroll
  for (int k = 0; k < TileDma<R, DR>::NK; ++k) dma.issue(k);
  {
    const char* wsrc = reinterpret_cast<const char*>(w_uv + ((size_t)h * DV + v0) * R);
    const uint32_t wl = lds_address(w_s);
#pragma unroll
    for (int k = 0; k < WUV_INS / 4; ++k) {
      const int ins = wave + 4 * k, pos = ins * 64 + lane, r = pos / CPR, p = pos % CPR;
      dma16_lane_addr(wsrc + (size_t)r * (R * 2) + ((p ^ (r & (WSW - 1))) << 4), wl + ins * 1024);
    }
  }
  if (wave < AW) {
#pragma unroll
    for (int b = 0; b < RBW; ++b)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        bf16x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = (__bf16)qa[b][q4 * 4 + e];
        *reinterpret_cast<bf16x4*>(q_s + c * QP + (wave * RBW + b) * 32 + q4 * 8 + g * 4) = v;
      }
  }
  if (rrow < 32) *reinterpret_cast<uint4*>(q_s + rrow * QP + R + rch * 8) = rv;
  __syncthreads();  // the q tile is complete

  const int nb = wave & 1, kh = wave >> 1;
  const int kb0 = EVEN ? kh * KH0 : 0;  // this wave's first score k-step
  bf16x8 qf[KH0];
#pragma unroll
  for (int i = 0; i < KH0; ++i) qf[i] = *reinterpret_cast<const bf16x8*>(q_s + c * QP + (kb0 + i) * 16 + g * 8);
  wait_vmem_below<WUV_INS / 4>();  // the KV rows of this wave are in LDS; the W_UV rows may still be in flight
  __syncthreads();

  // ---- scores: S^T[n][t] for tile rows n = nb*32 + (r/4)*8 + g*4 + r%4 (register r), node t = c
  float s[16];
  {
    f32x16 acc0 = zero16(), acc1 = zero16();
    const int nrow = nb * 32 + c;
    // the k-steps of one wave half, with its first k-step a compile-time constant (every offset is then a
    // per-lane base plus an immediate); fragment i + QD is requested before the MFMA of fragment i
    auto half = [&](auto first) {
      constexpr int F = decltype(first)::value;
      auto kfrag = [&](int i) -> bf16x8 {
        const int kb = F + i;
        const int off = (kb < R / 16) ? TL::ckv(nrow, 2 * kb + g) : TL::kpe(nrow, 2 * (kb - R / 16) + g);
        return *reinterpret_cast<const bf16x8*>(kvbuf + off);
      };
      constexpr int QD = KH0 < 6 ? KH0 : 6;
      bf16x8 kf[QD];
#pragma unroll
      for (int i = 0; i < QD; ++i) kf[i] = kfrag(i);
#pragma unroll
      for (int i = 0; i < KH0; ++i) {
        const bf16x8 a = kf[i % QD];
        if (i + QD < KH0) kf[i % QD] = kfrag(i + QD);
        if (i & 1) acc1 = mfma32(a, qf[i], acc1);
        else acc0 = mfma32(a, qf[i], acc0);
      }
    };
    if (kh == 0) half(std::integral_constant<int, 0>{});  // (wave-uniform)
    else if (EVEN) half(std::integral_constant<int, KH0>{});
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = acc0[r] + acc1[r];
  }
  if (kh == 1) {
#pragma unroll
    for (int r = 0; r < 16; ++r) red[nb][r][lane] = s[r];
  }
  __syncthreads();
  if (kh == 0) {
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] += red[nb][r][lane];
    const int jb = nb * 32 + g * 4 - L;  // tree index of register 0's row
    float tmax = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int j = jb + (r >> 2) * 8 + (r & 3);
      const bool vis = (j < 0) | ((j < T) & (((mw >> (j & 31)) & 1u) != 0u));
      s[r] = vis ? s[r] : -INFINITY;
      tmax = fmaxf(tmax, s[r]);
    }
    tmax = pair_max(tmax);
    if (g == 0) mx[nb][c] = tmax;
  }
  __syncthreads();
  // every node sees its own row (tree position L + t), so each row's maximum is finite
  const float M = fmaxf(mx[0][c], mx[1][c]) * scale_log2;  // (scale > 0)
  if (kh == 0) {
    bf16x8 pk[2];
    float ps;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float p0 = fast_exp2(fmaf(s[e], scale_log2, -M)), p1 = fast_exp2(fmaf(s[8 + e], scale_log2, -M));
      ps = (e == 0) ? p0 + p1 : ps + (p0 + p1);
      pk[0][e] = (__bf16)p0;
      pk[1][e] = (__bf16)p1;
    }
    ps = pair_sum(ps);
    pfr[nb * 2 + 0][lane] = __builtin_bit_cast(uint4, pk[0]);
    pfr[nb * 2 + 1][lane] = __builtin_bit_cast(uint4, pk[1]);
    if (g == 0) sm[nb][c] = ps;
  }
  __syncthreads();

  // ---- values: O^T[r][t] for this wave's latent columns col0 .. col0 + CPW - 1
  constexpr int DBW = PV::DBW;
  const float inv = 1.f / (sm[0][c] + sm[1][c]);
  const int col0 = wave * PV::CPW;
  f32x16 o[DBW];
#pragma unroll
  for (int db = 0; db < DBW; ++db) o[db] = zero16();
  if (wave < PV::WAVES) {
    const int rl = g * 4 + ((lane & 15) >> 2);
    const int cl = ((lane & 31) >> 4) * 2 + ((lane & 3) >> 1);
    const int sub = (lane & 1) * 8;
    bf16x8 pf[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) pf[ks] = __builtin_bit_cast(bf16x8, pfr[ks][lane]);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int db = 0; db < DBW; ++db) {
        const int ch = (col0 + db * 32) / 8 + cl;
        const bf16x8 a = concat_tr(lds_read_tr16(kvbuf + TL::ckv(ks * 16 + rl, ch) + sub),
                                   lds_read_tr16(kvbuf + TL::ckv(ks * 16 + rl + 8, ch) + sub));
        o[db] = mfma32(a, pf[ks], o[db]);
      }
  }
  __syncthreads();  // every wave is done with the KV tile: its LDS takes the latent output rows
  uint16_t* o_s = reinterpret_cast<uint16_t*>(kvbuf);
  if (wave < PV::WAVES) {
#pragma unroll
    for (int db = 0; db < DBW; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        bf16x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = (__bf16)(o[db][q4 * 4 + e] * inv);
        *reinterpret_cast<bf16x4*>(o_s + c * OP + col0 + db * 32 + q4 * 8 + g * 4) = v;
      }
  }
  if (lse != nullptr && blockIdx.y == 0 && wave == 0 && g == 0 && c < T)
    lse[c * H + h] = (M + log2f(sm[0][c] + sm[1][c])) * LN2;
  wait_vmem_all();  // this wave's W_UV rows
  __syncthreads();  // the latent output rows and all of W_UV are in LDS

  // ---- output: D[v][t] = sum_r W_UV[h][v0 + v][r] o[t][r], wave = contraction part kq (one 32-column block)
  const int kq = wave;
  const char* wrow = w_s + c * (R * 2);
  const int wsz = c & (WSW - 1);
  const uint16_t* orow = o_s + tq * OP + g * 8;
  f32x16 u0 = zero16(), u1 = zero16();
#pragma unroll
  for (int i = 0; i < KSQ; ++i) {
    const int ks = kq * KSQ + i;
    const bf16x8 a = *reinterpret_cast<const bf16x8*>(wrow + (((2 * ks + g) ^ wsz) << 4));
    const bf16x8 b = *reinterpret_cast<const bf16x8*>(orow + ks * 16);
    if (i & 1) u1 = mfma32(a, b, u1);
    else u0 = mfma32(a, b, u0);
  }
  float u[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) u[r] = u0[r] + u1[r];
  if (kq > 0) {
#pragma unroll
    for (int r = 0; r < 16; ++r) red[kq - 1][r][lane] = u[r];
  }
  __syncthreads();
  if (kq == 0 && c < T) {
#pragma unroll
    for (int q = 1; q < KQ; ++q)  // parts in a fixed order
#pragma unroll
      for (int r = 0; r < 16; ++r) u[r] += red[q - 1][r][lane];
    uint16_t* dst = out + ((size_t)c * H + h) * DV + v0 + g * 4;
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      bf16x4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = (__bf16)u[q4 * 4 + e];
      *reinterpret_cast<bf16x4*>(dst + q4 * 8) = v;
    }
  }
}


// ------------------------------------------------------------------------------------------------ state merge
// Two attention results over disjoint sets of KV positions, (out_a, lse_a) and (out_b, lse_b), combine into
// the result over their union.  With M = max(lse_a, lse_b) and w_x = e^(lse_x - M) (each part's softmax
// denominator relative to a common reference):
//   out = (w_a out_a + w_b out_b) / (w_a + w_b),   lse = M + ln(w_a + w_b).
// This is the split merge of the combine step with two parts; it is exact (up to rounding) whether the parts'
// outputs are latent rows or their W_UV projections, since W_UV is linear.  A part that saw no position has
// lse = -inf and weight 0; if neither did, out = 0 and lse = -inf.  One thread per 8 output elements.
__global__ __launch_bounds__(NTHREADS) void merge_states_kernel(const uint16_t* __restrict__ out_a,
                                                                const float* __restrict__ lse_a,
                                                                const uint16_t* __restrict__ out_b,
                                                                const float* __restrict__ lse_b, int64_t chunks,
                                                                int cpr, uint16_t* __restrict__ out,
                                                                float* __restrict__ lse) {
  const int64_t idx = (int64_t)blockIdx.x * NTHREADS + threadIdx.x;
  if (idx >= chunks) return;
  const int64_t r = idx / cpr;
  const float la = lse_a[r], lb = lse_b[r];
  const float M = fmaxf(la, lb);
  bf16x8 o;
  float lo = -INFINITY;
  if (M == -INFINITY) {
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = (__bf16)0.f;
  } else {
    const float wa = expf(la - M), wb = expf(lb - M);  // a part with lse = -inf gets weight 0
    const float inv = 1.f / (wa + wb);
    const bf16x8 a = *reinterpret_cast<const bf16x8*>(out_a + idx * 8);
    const bf16x8 b = *reinterpret_cast<const bf16x8*>(out_b + idx * 8);
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = (__bf16)((wa * (float)a[e] + wb * (float)b[e]) * inv);
    lo = M + logf(wa + wb);
  }
  *reinterpret_cast<bf16x8*>(out + idx * 8) = o;
  if (lse != nullptr && idx % cpr == 0) lse[r] = lo;
}

// ------------------------------------------------------------------------------------------------ page-table check
// Debug builds of a call (KDV_DEBUG=1 in the environment): one workgroup reads every page-table entry of the call
// and writes KDV_OK, or KDV_ERR_PAGE if some entry is outside [0, pool_slots), to `status`.  The verify kernels
// that follow read it first and gather nothing when it is not KDV_OK.
__global__ __launch_bounds__(1024) void page_check_kernel(const int32_t* __restrict__ page_table, int64_t n,
                                                          int64_t pool_slots, int32_t* __restrict__ status) {
  int bad = 0;
  for (int64_t i = threadIdx.x; i < n; i += 1024) {
    const int32_t v = page_table[i];
    bad |= (v < 0) | ((int64_t)v >= pool_slots);
  }
  bad = __syncthreads_or(bad);
  if (threadIdx.x == 0) *status = bad ? KDV_ERR_PAGE : KDV_OK;
}

// ------------------------------------------------------------------------------------------------ MFMA ceiling probe
// Diagnostic: every wave runs `iters` rounds of four independent 32x32x16 bf16 MFMA chains (the issue rate of
// back-to-back independent MFMAs, the ceiling the verify kernels are measured against).  Operands are zero, so
// the sums are zero; each thread writes its sum to `sink` so that nothing is optimised away.
__global__ __launch_bounds__(NTHREADS) void mfma_probe_kernel(int iters, float* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(0.f * lane);
    b[e] = (__bf16)0.f;
  }
  f32x16 c0 = zero16(), c1 = zero16(), c2 = zero16(), c3 = zero16();
  for (int it = 0; it < iters; ++it) {
    c0 = mfma32(a, b, c0);
    c1 = mfma32(a, b, c1);
    c2 = mfma32(a, b, c2);
    c3 = mfma32(a, b, c3);
  }
  float t = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) t += c0[r] + c1[r] + c2[r] + c3[r];
  sink[(size_t)blockIdx.x * NTHREADS + threadIdx.x] = t;
}

// ------------------------------------------------------------------------------------------------ host side
struct Plan {
  int H, nodes;           // heads, nodes of all requests
  int split_blocks, comb_blocks;
  int comb_rt;            // tree nodes per combine workgroup (4; 2 or 1 for a small single request, 16 for a batch)
  bool short_seq;         // one request whose L + T rows fit in one KV tile, T <= 32: short_verify_kernel alone
  BatchArgs<MAX_BATCH> ba;
  size_t off_qcat, off_po, off_pml, total;   // workspace regions (after a KDV_WS_HEADER-byte header)
};

enum ShapeId { SHAPE_NONE = 0, SHAPE_KIMI = 1, SHAPE_TINY = 2 };

static ShapeId shape_of(const kdv_mla_dims* d) {
  if (d->num_heads < 1 || d->num_heads > 128) return SHAPE_NONE;
  if (!(d->sm_scale > 0.f) || !(d->sm_scale < INFINITY)) return SHAPE_NONE;  // (NaN fails both)
  if (d->qk_nope_dim == 128 && d->qk_rope_dim == 64 && d->kv_lora_rank == 512 && d->v_head_dim == 128)
    return SHAPE_KIMI;
  if (d->qk_nope_dim == 32 && d->qk_rope_dim == 16 && d->kv_lora_rank == 64 && d->v_head_dim == 32)
    return SHAPE_TINY;
  return SHAPE_NONE;
}

static size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Compute units of the current device, queried once per device (a plan is made on every call).
static int device_cu_count() {
  constexpr int MAX_DEV = 64;
  static std::atomic<int> cached[MAX_DEV];  // 0: not queried yet
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return -1;
  if (dev < MAX_DEV && (cus = cached[dev].load(std::memory_order_relaxed)) > 0) return cus;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) return -1;
  if (dev < MAX_DEV) cached[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

// Plan of a call over C packed requests (C = 1 for the single-request entry points).  Each request's KV
// sequence (L prefix rows, then its T tree rows unless `with_tree` is false) is split so that (query tiles x
// splits) fills the request's share of the device once: one workgroup per CU with all query tiles of a split
// on one XCD, i.e. NUM_XCD * floor(CUs per XCD / query tiles) splits, the CUs shared among the requests in
// proportion to their tile work.  Every split gets the same whole number of 64-row tiles except possibly the
// last.  The environment variable KDV_SPLITS, if set, fixes every request's split count instead.
// The tiles per split are always sized for the L + T rows of the full verify, also for a prefix-only pass,
// so that a prefix-only pass never has more splits (nor needs more workspace) than the full call.
static int make_plan(const kdv_mla_dims* d, int C, const int32_t* Ls, const int32_t* Ts, Plan* p,
                     bool with_tree = true) {
  if (d == nullptr || Ls == nullptr || Ts == nullptr) return KDV_ERR_NULL;
  if (shape_of(d) == SHAPE_NONE || C < 1 || C > MAX_BATCH) return KDV_ERR_SHAPE;
  const int H = d->num_heads;
  int64_t nodes = 0, pt = 0, mwords = 0, work = 0;
  int m_tiles[MAX_BATCH], ntiles[MAX_BATCH];
  for (int c = 0; c < C; ++c) {
    const int L = Ls[c], T = Ts[c];
    if (T < 1 || T > KDV_MAX_TREE_NODES || L < (with_tree ? 0 : 1) || (int64_t)L + T > 0x7fffff00LL)
      return KDV_ERR_SHAPE;
    const int N = L + (with_tree ? T : 0);
    m_tiles[c] = (T * H + M_TILE - 1) / M_TILE;
    ntiles[c] = (N + KV_TILE - 1) / KV_TILE;
    work += (int64_t)m_tiles[c] * ntiles[c];
    ReqArgs& r = p->ba.r[c];
    r.L = L;
    r.T = T;
    r.N = N;
    r.node0 = (int)nodes;
    r.pt0 = (int)pt;
    r.mask0 = (int)mwords;
    r.m_tiles = m_tiles[c];
    r.Mp = m_tiles[c] * M_TILE;
    nodes += T;
    pt += (int64_t)L + T;
    mwords += (int64_t)T * ((T + 31) / 32);
    if (pt > 0x7fffff00LL) return KDV_ERR_SHAPE;
  }
  int env_splits = 0;
  if (const char* env = getenv("KDV_SPLITS")) env_splits = atoi(env);
  const int cus = env_splits > 0 ? 0 : device_cu_count();
  if (env_splits <= 0 && cus <= 0) return KDV_ERR_HIP;
  const int R = d->kv_lora_rank, DQ = R + d->qk_rope_dim;
  // Combine: 4 nodes per workgroup, fewer when a single request's (head, node-block) grid would otherwise leave
  // CUs idle (8 heads x 32 nodes: 64 workgroups of 4 nodes, 256 of one node).
  // A batch takes 16 nodes per workgroup when 4 would need more workgroups than CUs: every workgroup gathers
  // all of W_UV[h] (128 KB), so ten 15-node requests at 4 nodes cost 2560 gathers, at 16 nodes 640.
  const int cus_rt = cus > 0 ? cus : 256;
  p->comb_rt = 4;
  if (C == 1) {
    for (int rt = 1; rt < 4; rt *= 2)
      if ((int64_t)NUM_XCD * ((H + NUM_XCD - 1) / NUM_XCD) * ((Ts[0] + rt - 1) / rt) <= cus_rt) {
        p->comb_rt = rt;
        break;
      }
  } else {
    int64_t wgs4 = 0;
    for (int c = 0; c < C; ++c) wgs4 += (int64_t)NUM_XCD * ((H + NUM_XCD - 1) / NUM_XCD) * ((Ts[c] + 3) / 4);
    if (wgs4 > cus_rt) p->comb_rt = 16;
  }
  p->H = H;
  p->nodes = (int)nodes;
  p->ba.n = C;
  p->ba.H = H;
  p->ba.blk_split[0] = p->ba.blk_comb[0] = 0;
  // A batch (several requests, no fixed split count) takes the stream-K plan: groups of G workgroups (G = the
  // most query tiles of any request), laid out contiguously over the XCDs; the KV tiles of all requests,
  // concatenated, are dealt out in equal contiguous runs, one per group.  A request's partial slots are the
  // runs that touch its KV tiles, the same for each of its query tiles.
  int64_t G = 1, kv_all = 0;
  for (int c = 0; c < C; ++c) {
    G = std::max<int64_t>(G, m_tiles[c]);
    kv_all += ntiles[c];
  }
  const int lin_sk = cus / NUM_XCD;
  const bool streamk = C > 1 && env_splits <= 0 && with_tree && (int64_t)NUM_XCD * lin_sk >= G;
  p->ba.sk_w = p->ba.sk_u = 0;
  p->ba.sk_g = p->ba.sk_lin = p->ba.sk_groups = 0;
  if (streamk) {
    const int64_t groups = std::min<int64_t>((int64_t)NUM_XCD * lin_sk / G, kv_all);
    p->ba.sk_w = (kv_all + groups - 1) / groups;
    p->ba.sk_u = kv_all;
    p->ba.sk_g = (int)G;
    p->ba.sk_lin = lin_sk;
    p->ba.sk_groups = (int)((kv_all + p->ba.sk_w - 1) / p->ba.sk_w);
  }
  int64_t po = 0, pml = 0, blk_s = 0, blk_c = 0, xoff = 0, sk_base = 0;
  for (int c = 0; c < C; ++c) {
    ReqArgs& r = p->ba.r[c];
    r.sk_base = sk_base;
    if (streamk) {
      r.tiles_per_split = ntiles[c];
      r.lin = 0;
      r.xoff = 0;
      r.splits = (int)((sk_base + ntiles[c] - 1) / p->ba.sk_w - sk_base / p->ba.sk_w + 1);
      sk_base += ntiles[c];
      r.po = po;
      r.pml = pml;
      po += (int64_t)r.splits * r.Mp * R;
      pml += (int64_t)r.splits * r.Mp;
      blk_c += (int64_t)NUM_XCD * ((H + NUM_XCD - 1) / NUM_XCD) * ((r.T + p->comb_rt - 1) / p->comb_rt);
      if (blk_c > 0x7fffffff) return KDV_ERR_SHAPE;
      blk_s = (int64_t)NUM_XCD * lin_sk;
      p->ba.blk_split[c + 1] = (int)blk_s;
      p->ba.blk_comb[c + 1] = (int)blk_c;
      continue;
    }
    int want = env_splits;
    if (want <= 0) {
      const int share = (C == 1) ? cus : (int)std::max<int64_t>(NUM_XCD, (int64_t)cus * m_tiles[c] * ntiles[c] / work);
      const int per_xcd = share / NUM_XCD;
      want = (r.m_tiles <= per_xcd) ? NUM_XCD * (per_xcd / r.m_tiles) : share / r.m_tiles;
      if (want < 1) want = 1;
    }
    const int nt_plan = (r.L + r.T + KV_TILE - 1) / KV_TILE;  // tiles of the full verify (see above)
    if (want > nt_plan) want = nt_plan;
    r.tiles_per_split = (nt_plan + want - 1) / want;
    r.lin = 0;
    if (C == 1 && env_splits <= 0) {
      // contiguous placement when it gives every workgroup fewer tiles (e.g. 15 query tiles: 17 splits on
      // 255 CUs instead of 16 on 240)
      const int lin = cus / NUM_XCD, s_lin = std::min(NUM_XCD * lin / r.m_tiles, nt_plan);
      if (s_lin >= 1) {
        const int tps = (nt_plan + s_lin - 1) / s_lin;
        if (tps < r.tiles_per_split) {
          r.tiles_per_split = tps;
          r.lin = lin;
        }
      }
    }
    r.splits = (ntiles[c] + r.tiles_per_split - 1) / r.tiles_per_split;
    r.xoff = (int)(xoff % NUM_XCD);
    xoff += r.splits;
    r.po = po;
    r.pml = pml;
    po += (int64_t)r.splits * r.Mp * R;
    pml += (int64_t)r.splits * r.Mp;
    blk_s += r.lin > 0 ? (int64_t)NUM_XCD * r.lin : (int64_t)NUM_XCD * r.m_tiles * ((r.splits + NUM_XCD - 1) / NUM_XCD);
    blk_c += (int64_t)NUM_XCD * ((H + NUM_XCD - 1) / NUM_XCD) * ((r.T + p->comb_rt - 1) / p->comb_rt);
    if (blk_s > 0x7fffffff || blk_c > 0x7fffffff) return KDV_ERR_SHAPE;
    p->ba.blk_split[c + 1] = (int)blk_s;
    p->ba.blk_comb[c + 1] = (int)blk_c;
  }
  p->split_blocks = (int)blk_s;
  p->comb_blocks = (int)blk_c;
  // A single verify whose whole sequence fits in one tile takes the short-sequence kernel instead of the split-KV
  // pass and the combine (unless a split count is forced: that always takes the split path).
  p->short_seq = C == 1 && with_tree && env_splits <= 0 && Ls[0] + Ts[0] <= KV_TILE && Ts[0] <= 32;
  size_t off = KDV_WS_HEADER;  // header: the debug page-table status (int32 at offset 0)
  p->off_qcat = off;
  off += align256((size_t)nodes * H * DQ * 2);
  p->off_po = off;
  off += align256((size_t)po * 2);
  p->off_pml = off;
  off += align256((size_t)pml * 8);
  p->total = off;
  return KDV_OK;
}

// Launch one kernel; with `ev` (start, stop) the events take the kernel's own start and end timestamps.
template <typename... KArgs, typename... Args>
static void launch_n(void (*k)(KArgs...), dim3 grid, int threads, hipStream_t st, hipEvent_t const* ev, Args... args) {
  if (ev)
    hipExtLaunchKernelGGL(k, grid, dim3(threads), 0, st, ev[0], ev[1], 0, args...);
  else
    hipLaunchKernelGGL(k, grid, dim3(threads), 0, st, args...);
}
template <typename... KArgs, typename... Args>
static void launch(void (*k)(KArgs...), dim3 grid, hipStream_t st, hipEvent_t const* ev, Args... args) {
  launch_n(k, grid, NTHREADS, st, ev, args...);
}

template <int DN, int R, int DR, int DV>
static void launch_all(const Plan& pl, float sm_scale, const uint16_t* q_nope, const uint16_t* q_rope,
                       const uint16_t* w_uk, const uint16_t* w_uv, const uint16_t* c_kv, const uint16_t* k_pe,
                       const int32_t* page_table, const uint32_t* mask, uint16_t* out, float* lse, char* ws,
                       hipStream_t st, hipEvent_t const* ev, const int32_t* parent, int32_t* status,
                       const int32_t* dbg) {
  uint16_t* q_cat = reinterpret_cast<uint16_t*>(ws + pl.off_qcat);
  uint16_t* part_o = reinterpret_cast<uint16_t*>(ws + pl.off_po);
  float2* part_ml = reinterpret_cast<float2*>(ws + pl.off_pml);
  const float scale_log2 = sm_scale * 1.44269504088896340736f;
  if (pl.short_seq) {  // the whole call in one kernel (it builds the tree mask itself when given `parent`)
    const ReqArgs& r = pl.ba.r[0];
    launch(short_verify_kernel<DN, R, DR, DV>, dim3(pl.H, DV / ShortLayout<DN, R, DR, DV>::VC), st,
           ev ? ev + 0 : nullptr, q_nope, q_rope, w_uk, w_uv, c_kv, k_pe, page_table, parent,
           const_cast<uint32_t*>(mask), status, r.L, r.T, pl.H, scale_log2, out, lse, dbg);
    return;
  }
  // The query absorption is per node: the packed nodes of all requests in one grid.  With `parent` (one
  // request) an extra block builds the tree mask the split-KV kernel then reads.
  const dim3 qa_grid(pl.H + (parent != nullptr ? 1 : 0), (R + 127) / 128, (pl.nodes + 31) / 32);
  launch(q_absorb_kernel<DN, R, DR>, qa_grid, st, ev ? ev + 0 : nullptr, q_nope, q_rope, w_uk, q_cat, pl.nodes, pl.H,
         parent, const_cast<uint32_t*>(mask), status, dbg);
  if (pl.ba.n == 1) {
    BatchArgs<1> one;
    one.n = 1;
    one.H = pl.ba.H;
    one.sk_w = 0;
    one.sk_u = 0;
    one.blk_split[0] = one.blk_comb[0] = 0;
    one.blk_split[1] = pl.ba.blk_split[1];
    one.blk_comb[1] = pl.ba.blk_comb[1];
    one.r[0] = pl.ba.r[0];
    // CUs the split plan leaves idle (in whole XCD rounds) read W_UV ahead of the combine
    const int cus = device_cu_count();
    static_assert(((DV * R / 8) & (DV * R / 8 - 1)) == 0, "W_UV chunks per head: a power of two");
    const int pf_blocks = cus > pl.split_blocks ? (cus - pl.split_blocks) / NUM_XCD * NUM_XCD : 0;
    launch(splitkv_kernel<R, DR, 1>, dim3(pl.split_blocks + pf_blocks), st, ev ? ev + 2 : nullptr,
           (const uint16_t*)q_cat, c_kv, k_pe, page_table, mask, one, scale_log2, part_o, part_ml, dbg,
           pf_blocks > 0 ? w_uv : (const uint16_t*)nullptr, __builtin_ctz(DV * R / 8));
    auto comb = pl.comb_rt == 1 ? combine_up_kernel<R, DV, 1, 1>
                : pl.comb_rt == 2 ? combine_up_kernel<R, DV, 1, 2> : combine_up_kernel<R, DV, 1, 4>;
    launch_n(comb, dim3(pl.comb_blocks), COMB_THREADS, st, ev ? ev + 4 : nullptr, (const uint16_t*)part_o,
             (const float2*)part_ml, one, w_uv, out, lse, dbg);
  } else {
    launch(splitkv_kernel<R, DR, MAX_BATCH>, dim3(pl.split_blocks), st, ev ? ev + 2 : nullptr,
           (const uint16_t*)q_cat, c_kv, k_pe, page_table, mask, pl.ba, scale_log2, part_o, part_ml, dbg,
           (const uint16_t*)nullptr, 0);
    launch_n(pl.comb_rt == 16 ? combine_up_kernel<R, DV, MAX_BATCH, 16> : combine_up_kernel<R, DV, MAX_BATCH, 4>,
             dim3(pl.comb_blocks), COMB_THREADS, st, ev ? ev + 4 : nullptr,
             (const uint16_t*)part_o, (const float2*)part_ml, pl.ba, w_uv, out, lse, dbg);
  }
}

static bool misaligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) != 0; }

// KDV_DEBUG set to a value other than "0" in the environment at the time of a call turns on the page-table check.
static bool debug_checks() {
  const char* v = getenv("KDV_DEBUG");
  return v != nullptr && v[0] != '\0' && !(v[0] == '0' && v[1] == '\0');
}

}  // namespace kdv

extern "C" size_t kdv_verify_workspace_bytes(const kdv_mla_dims* d, int32_t T, int32_t L) {
  kdv::Plan p;
  if (kdv::make_plan(d, 1, &L, &T, &p) != KDV_OK) return 0;
  return p.total;
}

extern "C" size_t kdv_verify_batch_workspace_bytes(const kdv_mla_dims* d, int32_t C, const int32_t* L,
                                                   const int32_t* T) {
  kdv::Plan p;
  if (kdv::make_plan(d, C, L, T, &p) != KDV_OK) return 0;
  return p.total;
}

extern "C" size_t kdv_prefix_workspace_bytes(const kdv_mla_dims* d, int32_t T, int32_t L) {
  kdv::Plan p;
  if (kdv::make_plan(d, 1, &L, &T, &p, /*with_tree=*/false) != KDV_OK) return 0;
  return p.total;
}

extern "C" int32_t kdv_verify_kernel_count(const kdv_mla_dims* d, int32_t T, int32_t L) {
  kdv::Plan p;
  if (kdv::make_plan(d, 1, &L, &T, &p) != KDV_OK) return 0;
  return p.short_seq ? 1 : 3;
}

extern "C" int32_t kdv_verify_num_splits(const kdv_mla_dims* d, int32_t T, int32_t L) {
  kdv::Plan p;
  if (kdv::make_plan(d, 1, &L, &T, &p) != KDV_OK) return 0;
  return p.ba.r[0].splits;
}

static int verify_impl(const kdv_mla_dims* d, int32_t C, const int32_t* Ls, const int32_t* Ts,
                       const uint16_t* q_nope, const uint16_t* q_rope, const uint16_t* w_uk, const uint16_t* w_uv,
                       const uint16_t* c_kv, const uint16_t* k_pe, int64_t pool_slots, const int32_t* page_table,
                       const uint32_t* mask, uint16_t* out, float* lse, void* workspace, size_t workspace_bytes,
                       void* stream, hipEvent_t const* ev, bool with_tree = true,
                       const int32_t* parent = nullptr, int32_t* status = nullptr) {
  using namespace kdv;
  if (d == nullptr || Ls == nullptr || Ts == nullptr || q_nope == nullptr || q_rope == nullptr ||
      w_uk == nullptr || w_uv == nullptr || c_kv == nullptr || k_pe == nullptr || page_table == nullptr ||
      (with_tree && mask == nullptr) || out == nullptr || workspace == nullptr)
    return KDV_ERR_NULL;
  const ShapeId sid = shape_of(d);
  if (sid == SHAPE_NONE || pool_slots < 1 || C < 1 || C > MAX_BATCH) return KDV_ERR_SHAPE;
  for (int c = 0; c < C; ++c)
    if (Ts[c] < 1 || Ts[c] > KDV_MAX_TREE_NODES || Ls[c] < (with_tree ? 0 : 1)) return KDV_ERR_SHAPE;
  if (misaligned(q_nope, 16) || misaligned(q_rope, 16) || misaligned(w_uk, 16) || misaligned(w_uv, 16) ||
      misaligned(c_kv, 16) || misaligned(k_pe, 16) || misaligned(out, 16) || misaligned(workspace, 16) ||
      misaligned(page_table, 4) || misaligned(mask, 4) || misaligned(lse, 4) || misaligned(parent, 4) ||
      misaligned(status, 4))
    return KDV_ERR_ALIGN;
  Plan pl;
  const int st = make_plan(d, C, Ls, Ts, &pl, with_tree);
  if (st != KDV_OK) return st;
  if (workspace_bytes < pl.total) return KDV_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  (void)hipGetLastError();
  // KDV_DEBUG=1: check every page-table entry of the call against pool_slots first (status in the workspace header)
  const int32_t* dbg = nullptr;
  if (debug_checks()) {
    int64_t entries = 0;
    for (int c = 0; c < C; ++c) entries += (int64_t)Ls[c] + (with_tree ? Ts[c] : 0);
    int32_t* dst = reinterpret_cast<int32_t*>(ws);
    hipLaunchKernelGGL(page_check_kernel, dim3(1), dim3(1024), 0, s, page_table, entries, pool_slots, dst);
    dbg = dst;
  }
  if (sid == SHAPE_KIMI)
    launch_all<128, 512, 64, 128>(pl, d->sm_scale, q_nope, q_rope, w_uk, w_uv, c_kv, k_pe, page_table, mask, out,
                                  lse, ws, s, ev, parent, status, dbg);
  else
    launch_all<32, 64, 16, 32>(pl, d->sm_scale, q_nope, q_rope, w_uk, w_uv, c_kv, k_pe, page_table, mask, out, lse,
                               ws, s, ev, parent, status, dbg);
  return hipGetLastError() == hipSuccess ? KDV_OK : KDV_ERR_HIP;
}

extern "C" int kdv_verify_mla_attn(const kdv_mla_dims* d, const uint16_t* q_nope, const uint16_t* q_rope,
                                   const uint16_t* w_uk, const uint16_t* w_uv, const uint16_t* c_kv,
                                   const uint16_t* k_pe, int64_t pool_slots, const int32_t* page_table, int32_t L,
                                   int32_t T, const uint32_t* mask, uint16_t* out, float* lse, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  return verify_impl(d, 1, &L, &T, q_nope, q_rope, w_uk, w_uv, c_kv, k_pe, pool_slots, page_table, mask, out, lse,
                     workspace, workspace_bytes, stream, nullptr);
}

// ------------------------------------------------------------------------------------------------ no-allocation entry
// The workspace of kdv_verify_mla_attn_noalloc: one array per device, in the library's code object, reserved when
// the library is loaded on that device and held until the process ends.  Host code never passes the array's name to
// a kernel (on the host it is only a stand-in for the symbol); it takes each device's address once, with that device
// current, and uses that.  Nothing in it needs to start at zero: every region a call reads is first written by the
// same call.  Calls on one device share it, so calls that overlap in time on one device race.
namespace kdv {
static __device__ __align__(256) char scratch[KDV_NOALLOC_SCRATCH_BYTES];
constexpr int MAX_DEVICES = 64;
static std::mutex scratch_mu;
static void* scratch_ptr[MAX_DEVICES];

static int scratch_of_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return KDV_ERR_HIP;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return KDV_ERR_HIP;
    scratch_ptr[dev] = p;
  }
  *out = scratch_ptr[dev];
  return KDV_OK;
}
}  // namespace kdv

extern "C" int kdv_verify_mla_attn_noalloc(const kdv_mla_dims* d, const uint16_t* q_nope, const uint16_t* q_rope,
                                           const uint16_t* w_uk, const uint16_t* w_uv, const uint16_t* c_kv,
                                           const uint16_t* k_pe, int64_t pool_slots, const int32_t* page_table,
                                           int32_t L, int32_t T, const uint32_t* mask, uint16_t* out, float* lse,
                                           void* stream) {
  // argument errors and the scratch limit are reported before the device is touched (the plan needs no device
  // when KDV_SPLITS is set)
  if (d == nullptr || q_nope == nullptr || q_rope == nullptr || w_uk == nullptr || w_uv == nullptr ||
      c_kv == nullptr || k_pe == nullptr || page_table == nullptr || mask == nullptr || out == nullptr)
    return KDV_ERR_NULL;
  if (kdv::shape_of(d) == kdv::SHAPE_NONE || pool_slots < 1 || T < 1 || T > KDV_MAX_TREE_NODES || L < 0)
    return KDV_ERR_SHAPE;
  kdv::Plan pl;
  const int st = kdv::make_plan(d, 1, &L, &T, &pl);
  if (st != KDV_OK) return st;
  if (pl.total > KDV_NOALLOC_SCRATCH_BYTES) return KDV_ERR_WORKSPACE;
  void* ws = nullptr;
  const int sst = kdv::scratch_of_current_device(&ws);
  if (sst != KDV_OK) return sst;
  return verify_impl(d, 1, &L, &T, q_nope, q_rope, w_uk, w_uv, c_kv, k_pe, pool_slots, page_table, mask, out, lse,
                     ws, KDV_NOALLOC_SCRATCH_BYTES, stream, nullptr);
}

extern "C" int kdv_verify_mla_attn_profiled(const kdv_mla_dims* d, const uint16_t* q_nope, const uint16_t* q_rope,
                                            const uint16_t* w_uk, const uint16_t* w_uv, const uint16_t* c_kv,
                                            const uint16_t* k_pe, int64_t pool_slots, const int32_t* page_table,
                                            int32_t L, int32_t T, const uint32_t* mask, uint16_t* out, float* lse,
                                            void* workspace, size_t workspace_bytes, void* stream,
                                            void* const* events) {
  if (events == nullptr) return KDV_ERR_NULL;
  return verify_impl(d, 1, &L, &T, q_nope, q_rope, w_uk, w_uv, c_kv, k_pe, pool_slots, page_table, mask, out, lse,
                     workspace, workspace_bytes, stream, reinterpret_cast<hipEvent_t const*>(events));
}

extern "C" int kdv_verify_mla_attn_tree(const kdv_mla_dims* d, const uint16_t* q_nope, const uint16_t* q_rope,
                                        const uint16_t* w_uk, const uint16_t* w_uv, const uint16_t* c_kv,
                                        const uint16_t* k_pe, int64_t pool_slots, const int32_t* page_table,
                                        int32_t L, int32_t T, const int32_t* parent, uint32_t* mask, int32_t* status,
                                        uint16_t* out, float* lse, void* workspace, size_t workspace_bytes,
                                        void* stream) {
  if (parent == nullptr) return KDV_ERR_NULL;
  return verify_impl(d, 1, &L, &T, q_nope, q_rope, w_uk, w_uv, c_kv, k_pe, pool_slots, page_table, mask, out, lse,
                     workspace, workspace_bytes, stream, nullptr, true, parent, status);
}

extern "C" int kdv_verify_mla_attn_batch(const kdv_mla_dims* d, int32_t C, const int32_t* L, const int32_t* T,
                                         const uint16_t* q_nope, const uint16_t* q_rope, const uint16_t* w_uk,
                                         const uint16_t* w_uv, const uint16_t* c_kv, const uint16_t* k_pe,
                                         int64_t pool_slots, const int32_t* page_table, const uint32_t* mask,
                                         uint16_t* out, float* lse, void* workspace, size_t workspace_bytes,
                                         void* stream) {
  return verify_impl(d, C, L, T, q_nope, q_rope, w_uk, w_uv, c_kv, k_pe, pool_slots, page_table, mask, out, lse,
                     workspace, workspace_bytes, stream, nullptr);
}

extern "C" int kdv_prefix_mla_attn(const kdv_mla_dims* d, const uint16_t* q_nope, const uint16_t* q_rope,
                                   const uint16_t* w_uk, const uint16_t* w_uv, const uint16_t* c_kv,
                                   const uint16_t* k_pe, int64_t pool_slots, const int32_t* page_table, int32_t L,
                                   int32_t T, uint16_t* out, float* lse, void* workspace, size_t workspace_bytes,
                                   void* stream) {
  return verify_impl(d, 1, &L, &T, q_nope, q_rope, w_uk, w_uv, c_kv, k_pe, pool_slots, page_table, nullptr, out,
                     lse, workspace, workspace_bytes, stream, nullptr, /*with_tree=*/false);
}

extern "C" int kdv_merge_attn_states(const uint16_t* out_a, const float* lse_a, const uint16_t* out_b,
                                     const float* lse_b, int64_t rows, int32_t dv, uint16_t* out, float* lse,
                                     void* stream) {
  using namespace kdv;
  if (out_a == nullptr || lse_a == nullptr || out_b == nullptr || lse_b == nullptr || out == nullptr)
    return KDV_ERR_NULL;
  if (rows < 1 || dv < 8 || dv % 8 != 0 || dv > 4096 || rows > (int64_t(1) << 34) / dv) return KDV_ERR_SHAPE;
  if (misaligned(out_a, 16) || misaligned(out_b, 16) || misaligned(out, 16) || misaligned(lse_a, 4) ||
      misaligned(lse_b, 4) || misaligned(lse, 4))
    return KDV_ERR_ALIGN;
  const int64_t chunks = rows * (dv / 8);
  const int64_t blocks = (chunks + NTHREADS - 1) / NTHREADS;
  (void)hipGetLastError();
  hipLaunchKernelGGL(merge_states_kernel, dim3((unsigned)blocks), dim3(NTHREADS), 0, static_cast<hipStream_t>(stream),
                     out_a, lse_a, out_b, lse_b, chunks, dv / 8, out, lse);
  return hipGetLastError() == hipSuccess ? KDV_OK : KDV_ERR_HIP;
}

extern "C" int kdv_mfma_probe(int32_t iters, float* sink, int32_t blocks, void* stream) {
  using namespace kdv;
  if (sink == nullptr) return KDV_ERR_NULL;
  if (iters < 1 || blocks < 1 || blocks > (1 << 20)) return KDV_ERR_SHAPE;
  if (misaligned(sink, 4)) return KDV_ERR_ALIGN;
  (void)hipGetLastError();
  hipLaunchKernelGGL(mfma_probe_kernel, dim3(blocks), dim3(NTHREADS), 0, static_cast<hipStream_t>(stream), iters,
                     sink);
  return hipGetLastError() == hipSuccess ? KDV_OK : KDV_ERR_HIP;
}

extern "C" const char* kdv_status_string(int status) {
  switch (status) {
    case KDV_OK: return "ok";
    case KDV_ERR_NULL: return "a required pointer is NULL";
    case KDV_ERR_SHAPE: return "unsupported shape (T outside [1,64], L < 0, or dims not supported)";
    case KDV_ERR_TREE: return "parent array is not a rooted tree in topological order";
    case KDV_ERR_ALIGN: return "an array or the workspace is not suitably aligned (16 B for bf16 data)";
    case KDV_ERR_WORKSPACE: return "workspace smaller than kdv_verify_workspace_bytes()";
    case KDV_ERR_HIP: return "HIP launch or query failed";
    case KDV_ERR_PAGE: return "a page-table entry is outside [0, pool_slots) (KDV_DEBUG check)";
    default: return "unknown kdv status";
  }
}
