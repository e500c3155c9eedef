// Tree-verify MLA attention in absorbed form, split over the KV sequence (gfx950 / CDNA4).
//
// What is computed follows "The Architecture of Diagnosis...", section "Phase 1: Custom CUDA Kernels",
// item 2 (every draft-tree node attends over the KV cache under the tree's visibility mask, with the
// latent projection absorbed), over the 512 + 64 element MLA latent cache of "From Diagnosis to
// Deployment...", section "The Second Thread: Pivoting to 200k Context", addressed one token per page
// ("The Architecture of Diagnosis...", section "The Discrepancy That Revealed the Truth").
//
// Four kernels, enqueued in order on the caller's stream:
//   q_absorb : q_cat[m] = [W_UK[h]^T q_nope[t,h] ; q_rope[t,h]]          (m = t*H + h; bf16 MFMA)
//   splitkv  : one workgroup per (64 query rows, KV split).  KV tiles of 64 paged rows are gathered into
//              LDS; scores S^T = K Q^T and O^T += V^T P^T run on 32x32x16 bf16 MFMA with an online
//              softmax; the partial (O, max, sum) of the split goes to the workspace.
//   combine  : log-sum-exp merge of the splits -> o_lat (bf16) and lse.
//   up_proj  : out[t,h] = W_UV[h] o_lat[t,h]                              (bf16 MFMA)
#include <math.h>
#include <stdlib.h>

#include "common.h"

namespace kdv {

constexpr int KV_TILE = 64;   // KV rows per LDS tile
constexpr int M_TILE = 64;    // query rows (node, head) per split-KV workgroup
constexpr int NTHREADS = 256;

template <int R, int DR>
struct Shape {
  static constexpr int DQ = R + DR;      // score contraction length (576 for the Kimi shape)
  static constexpr int KB = DQ / 16;     // 16-deep MFMA k-blocks of the score contraction
  static constexpr int PITCH = DQ + 8;   // LDS row pitch in elements: +16 B keeps 16-row b128 reads conflict-free
  static constexpr int CH = DQ / 8;      // 16-byte chunks per KV row
  static constexpr int DB = R / 64;      // 32-wide output column blocks per wave (a wave owns R/2 columns)
};

// ------------------------------------------------------------------------------------------------ q_absorb
// grid (H, ceil(R/128)); each wave produces 32 latent columns for all T nodes of head h.
// MFMA D[r][t] = sum_k W_UK[h][k][r] q_nope[t,h][k]: the A operand W^T is read from LDS with transposed
// reads (W_UK is stored k-major), the B operand straight from global memory.
template <int DN, int R, int DR>
__global__ __launch_bounds__(NTHREADS) void q_absorb_kernel(const uint16_t* __restrict__ q_nope,
                                                            const uint16_t* __restrict__ q_rope,
                                                            const uint16_t* __restrict__ w_uk,
                                                            uint16_t* __restrict__ q_cat, int T, int H) {
  constexpr int DQ = R + DR;
  constexpr int RB = 128;         // latent columns per workgroup
  constexpr int WP = RB + 16;     // LDS pitch (elements)
  __shared__ __attribute__((aligned(16))) uint16_t w_s[DN * WP];
  const int h = blockIdx.x, r0 = blockIdx.y * RB;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, c = lane & 31;

  const uint16_t* wh = w_uk + (size_t)h * DN * R;
  for (int ci = tid; ci < DN * (RB / 8); ci += NTHREADS) {
    const int k = ci / (RB / 8), col = (ci % (RB / 8)) * 8;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (r0 + col < R) v = *reinterpret_cast<const uint4*>(wh + (size_t)k * R + r0 + col);
    *reinterpret_cast<uint4*>(&w_s[k * WP + col]) = v;
  }
  if (blockIdx.y == 0) {
    for (int ci = tid; ci < T * (DR / 8); ci += NTHREADS) {
      const int t = ci / (DR / 8), col = (ci % (DR / 8)) * 8;
      *reinterpret_cast<uint4*>(q_cat + (size_t)(t * H + h) * DQ + R + col) =
          *reinterpret_cast<const uint4*>(q_rope + ((size_t)t * H + h) * DR + col);
    }
  }
  __syncthreads();
  const int rs = wave * 32;
  if (r0 + rs >= R) return;  // wave-uniform; no barrier follows
  for (int tb = 0; tb < T; tb += 32) {
    f32x16 acc = zero16();
    const int t = tb + c;
#pragma unroll
    for (int kb = 0; kb < DN / 16; ++kb) {
      const int krow = kb * 16 + g * 8 + ((lane & 15) >> 2);
      const int col = rs + ((lane & 31) >> 4) * 16 + 4 * (lane & 3);
      const bf16x8 a = concat_tr(lds_read_tr16(&w_s[krow * WP + col]), lds_read_tr16(&w_s[(krow + 4) * WP + col]));
      const bf16x8 b = (t < T) ? load_bf16x8(q_nope + ((size_t)t * H + h) * DN + kb * 16 + g * 8) : zero_bf16x8();
      acc = mfma32(a, b, acc);
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

// ------------------------------------------------------------------------------------------------ splitkv
// Workgroup = 4 waves over 64 query rows.  Wave (wi, wj): rows wi*32..+31 of the tile.
//   scores : the wave computes S^T for KV rows wj*32..+31 of each 64-row tile (full 576-deep contraction);
//   softmax: the two waves of a row pair agree on the running max through LDS, then swap their halves of
//            P (bf16) through LDS;
//   values : the wave accumulates O^T for latent columns wj*R/2..+R/2 over all 64 KV rows of the tile.
// Lane l owns query row m = tile_row + wi*32 + (l%32): the softmax state of a row lives in one lane pair
// (l, l^32) and every per-row factor is a per-lane scalar.
template <int R, int DR>
__global__ __launch_bounds__(NTHREADS, 1) void splitkv_kernel(
    const uint16_t* __restrict__ q_cat, const uint16_t* __restrict__ c_kv, const uint16_t* __restrict__ k_pe,
    const int32_t* __restrict__ page_table, const uint32_t* __restrict__ mask, int L, int T, int H, int M, int N,
    int m_tiles, int tiles_per_split, float scale_log2, float* __restrict__ part_o, float2* __restrict__ part_ml,
    int Mp) {
  using S = Shape<R, DR>;
  __shared__ __attribute__((aligned(16))) uint16_t kv[KV_TILE * S::PITCH];
  __shared__ uint4 pbuf[2][2][64][2];  // [row pair][kv half][lane][16-row k-block]: P^T fragments (bf16)
  __shared__ float xch[2][2][32];      // per-row max / sum exchange within a row pair
  __shared__ int slots[KV_TILE];

  const int mt = blockIdx.x % m_tiles;
  const int split = blockIdx.x / m_tiles;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wi = wave >> 1, wj = wave & 1;
  const int g = lane >> 5, c = lane & 31;
  const int m = mt * M_TILE + wi * 32 + c;

  bf16x8 q[S::KB];
  const bool row_ok = m < M;
#pragma unroll
  for (int kb = 0; kb < S::KB; ++kb)
    q[kb] = row_ok ? load_bf16x8(q_cat + (size_t)m * S::DQ + kb * 16 + g * 8) : zero_bf16x8();
  uint32_t mw0 = 0xffffffffu, mw1 = 0xffffffffu;
  if (row_ok) {
    const int t = m / H, W = (T + 31) >> 5;
    mw0 = mask[t * W];
    mw1 = (W == 2) ? mask[t * W + 1] : 0u;
  }

  f32x16 o[S::DB];
#pragma unroll
  for (int db = 0; db < S::DB; ++db) o[db] = zero16();
  float m_run = -INFINITY, l_part = 0.f;

  const int ntiles = (N + KV_TILE - 1) / KV_TILE;
  const int tile_begin = split * tiles_per_split;
  const int tile_end = min(tile_begin + tiles_per_split, ntiles);
  for (int tile = tile_begin; tile < tile_end; ++tile) {
    const int n0 = tile * KV_TILE;
    __syncthreads();  // every wave is done with the previous tile
    if (tid < KV_TILE) slots[tid] = page_table[min(n0 + tid, N - 1)];  // rows past N reuse a real row (masked)
    __syncthreads();
#pragma unroll 6
    for (int ci = tid; ci < KV_TILE * S::CH; ci += NTHREADS) {
      const int row = ci / S::CH, ch = ci % S::CH;
      const size_t slot = (size_t)slots[row];
      const uint16_t* src = (ch < R / 8) ? (c_kv + slot * R + ch * 8) : (k_pe + slot * DR + (ch - R / 8) * 8);
      *reinterpret_cast<uint4*>(&kv[row * S::PITCH + ch * 8]) = *reinterpret_cast<const uint4*>(src);
    }
    __syncthreads();

    // scores for KV rows wj*32 + (r/4)*8 + g*4 + r%4 of the tile, query row m
    f32x16 acc = zero16();
    const uint16_t* krow = &kv[(wj * 32 + c) * S::PITCH + g * 8];
#pragma unroll
    for (int kb = 0; kb < S::KB; ++kb)
      acc = mfma32(*reinterpret_cast<const bf16x8*>(krow + kb * 16), q[kb], acc);

    float p[16];
    float tmax = -INFINITY;
    const bool tail = n0 + KV_TILE > L;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float sv = acc[r] * scale_log2;
      if (tail) {
        const int n = n0 + wj * 32 + (r >> 2) * 8 + g * 4 + (r & 3);
        if (n >= L) {
          const int jn = n - L;
          const uint32_t word = jn < 32 ? mw0 : mw1;
          const bool vis = (n < N) && ((word >> (jn & 31)) & 1u);
          if (!vis) sv = -INFINITY;
        }
      }
      p[r] = sv;
      tmax = fmaxf(tmax, sv);
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    if (g == 0) xch[wi][wj][c] = tmax;
    __syncthreads();
    tmax = fmaxf(tmax, xch[wi][wj ^ 1][c]);
    const float m_new = fmaxf(m_run, tmax);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;  // all-masked so far: keep exp2 finite
    const float alpha = fast_exp2(m_run - m_use);
    float rsum = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      p[r] = fast_exp2(p[r] - m_use);
      rsum += p[r];
    }
    l_part = l_part * alpha + rsum;
    m_run = m_new;
    if (__any(alpha != 1.f)) {
#pragma unroll
      for (int db = 0; db < S::DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
    }
    bf16x8 pk[2];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      pk[0][e] = (__bf16)p[e];
      pk[1][e] = (__bf16)p[8 + e];
    }
    pbuf[wi][wj][lane][0] = __builtin_bit_cast(uint4, pk[0]);
    pbuf[wi][wj][lane][1] = __builtin_bit_cast(uint4, pk[1]);
    __syncthreads();
    bf16x8 po[2];
    po[0] = __builtin_bit_cast(bf16x8, pbuf[wi][wj ^ 1][lane][0]);
    po[1] = __builtin_bit_cast(bf16x8, pbuf[wi][wj ^ 1][lane][1]);

    // O^T[d][m] += sum_n V^T[d][n] P^T[n][m]; contraction order within a 16-row block follows the score
    // layout: k = g*8 + e  <->  KV row (e/4)*8 + g*4 + e%4.
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2) {
        const bf16x8 pb = (h2 == wj) ? pk[kb2] : po[kb2];
        const int row = h2 * 32 + kb2 * 16 + g * 4 + ((lane & 15) >> 2);
#pragma unroll
        for (int db = 0; db < S::DB; ++db) {
          const int col = wj * (R / 2) + db * 32 + ((lane & 31) >> 4) * 16 + 4 * (lane & 3);
          const bf16x8 a = concat_tr(lds_read_tr16(&kv[row * S::PITCH + col]),
                                     lds_read_tr16(&kv[(row + 8) * S::PITCH + col]));
          o[db] = mfma32(a, pb, o[db]);
        }
      }
    }
  }

  const float l_half = l_part + __shfl_xor(l_part, 32);
  __syncthreads();
  if (g == 0) xch[wi][wj][c] = l_half;
  __syncthreads();
  const float l_tot = l_half + xch[wi][wj ^ 1][c];
  const int mrow = mt * M_TILE + wi * 32 + c;
  float* dst = part_o + ((size_t)split * Mp + mrow) * R + wj * (R / 2) + g * 4;
#pragma unroll
  for (int db = 0; db < S::DB; ++db)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4)
      *reinterpret_cast<float4*>(dst + db * 32 + q4 * 8) =
          make_float4(o[db][q4 * 4 + 0], o[db][q4 * 4 + 1], o[db][q4 * 4 + 2], o[db][q4 * 4 + 3]);
  if (wj == 0 && g == 0) part_ml[(size_t)split * Mp + mrow] = make_float2(m_run, l_tot);
}

// ------------------------------------------------------------------------------------------------ combine
// o_lat[m] = sum_s 2^(m_s - M) O_s[m] / sum_s 2^(m_s - M) l_s,  lse[m] = ln 2 * (M + log2 sum_s 2^(m_s-M) l_s).
// A split in which row m saw nothing has m_s = -inf and l_s = 0 and gets weight 0.
template <int R>
__global__ __launch_bounds__(NTHREADS) void combine_kernel(const float* __restrict__ part_o,
                                                           const float2* __restrict__ part_ml, int S, int Mp,
                                                           int M, uint16_t* __restrict__ o_lat,
                                                           float* __restrict__ lse) {
  constexpr int TPR = R / 4;
  constexpr int RPB = NTHREADS / TPR;
  const int m = blockIdx.x * RPB + threadIdx.x / TPR;
  const int d = (threadIdx.x % TPR) * 4;
  if (m >= M) return;
  float mx = -INFINITY;
  for (int s = 0; s < S; ++s) mx = fmaxf(mx, part_ml[(size_t)s * Mp + m].x);
  float den = 0.f;
  float4 num = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s = 0; s < S; ++s) {
    const float2 ml = part_ml[(size_t)s * Mp + m];
    const float w = (ml.x == -INFINITY) ? 0.f : fast_exp2(ml.x - mx);
    den += w * ml.y;
    const float4 v = *reinterpret_cast<const float4*>(part_o + ((size_t)s * Mp + m) * R + d);
    num.x += w * v.x;
    num.y += w * v.y;
    num.z += w * v.z;
    num.w += w * v.w;
  }
  const float inv = 1.f / den;
  bf16x4 ov;
  ov[0] = (__bf16)(num.x * inv);
  ov[1] = (__bf16)(num.y * inv);
  ov[2] = (__bf16)(num.z * inv);
  ov[3] = (__bf16)(num.w * inv);
  *reinterpret_cast<bf16x4*>(o_lat + (size_t)m * R + d) = ov;
  if (lse != nullptr && d == 0) lse[m] = (mx + log2f(den)) * 0.69314718055994530942f;
}

// ------------------------------------------------------------------------------------------------ up_proj
// grid (H, DV/32); the four waves split the R-deep contraction and reduce through LDS.
// MFMA D[v][t] = sum_r W_UV[h][v][r] o_lat[t,h][r]: both operands are r-contiguous in memory.
template <int R, int DV>
__global__ __launch_bounds__(NTHREADS) void up_proj_kernel(const uint16_t* __restrict__ o_lat,
                                                           const uint16_t* __restrict__ w_uv,
                                                           uint16_t* __restrict__ out, int T, int H) {
  constexpr int KBW = R / 16 / 4;  // k-blocks per wave
  __shared__ float red[4][16][64];
  const int h = blockIdx.x, v0 = blockIdx.y * 32;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, c = lane & 31;
  const uint16_t* wrow = w_uv + ((size_t)h * DV + v0 + c) * R + wave * KBW * 16 + g * 8;
  bf16x8 a[KBW];
#pragma unroll
  for (int kk = 0; kk < KBW; ++kk) a[kk] = load_bf16x8(wrow + kk * 16);
  for (int tb = 0; tb < T; tb += 32) {
    const int t = tb + c;
    f32x16 acc = zero16();
    const uint16_t* orow = o_lat + ((size_t)t * H + h) * R + wave * KBW * 16 + g * 8;
#pragma unroll
    for (int kk = 0; kk < KBW; ++kk)
      acc = mfma32(a[kk], (t < T) ? load_bf16x8(orow + kk * 16) : zero_bf16x8(), acc);
#pragma unroll
    for (int r = 0; r < 16; ++r) red[wave][r][lane] = acc[r];
    __syncthreads();
    if (wave == 0 && t < T) {
      uint16_t* dst = out + ((size_t)t * H + h) * DV + v0 + g * 4;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        bf16x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = q4 * 4 + e;
          v[e] = (__bf16)(red[0][r][lane] + red[1][r][lane] + red[2][r][lane] + red[3][r][lane]);
        }
        *reinterpret_cast<bf16x4*>(dst + q4 * 8) = v;
      }
    }
    __syncthreads();
  }
}

// ------------------------------------------------------------------------------------------------ host side
struct Plan {
  int H, M, Mp, m_tiles, N, ntiles, tiles_per_split, splits;
  size_t off_qcat, off_olat, off_po, off_pml, total;
};

enum ShapeId { SHAPE_NONE = 0, SHAPE_KIMI = 1, SHAPE_TINY = 2 };

static ShapeId shape_of(const kdv_mla_dims* d) {
  if (d->num_heads < 1 || d->num_heads > 128) return SHAPE_NONE;
  if (d->qk_nope_dim == 128 && d->qk_rope_dim == 64 && d->kv_lora_rank == 512 && d->v_head_dim == 128)
    return SHAPE_KIMI;
  if (d->qk_nope_dim == 32 && d->qk_rope_dim == 16 && d->kv_lora_rank == 64 && d->v_head_dim == 32)
    return SHAPE_TINY;
  return SHAPE_NONE;
}

static size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

static int device_cu_count() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return -1;
  return cus;
}

// Split the KV sequence so that (query tiles x splits) fills the device once; every split gets the
// same whole number of 64-row tiles except possibly the last.
static int make_plan(const kdv_mla_dims* d, int T, int L, Plan* p) {
  if (d == nullptr) return KDV_ERR_NULL;
  if (shape_of(d) == SHAPE_NONE) return KDV_ERR_SHAPE;
  if (T < 1 || T > KDV_MAX_TREE_NODES || L < 0 || (int64_t)L + T > 0x7fffff00LL) return KDV_ERR_SHAPE;
  p->H = d->num_heads;
  p->M = T * d->num_heads;
  p->m_tiles = (p->M + M_TILE - 1) / M_TILE;
  p->Mp = p->m_tiles * M_TILE;
  p->N = L + T;
  p->ntiles = (p->N + KV_TILE - 1) / KV_TILE;
  int want = 0;
  if (const char* env = getenv("KDV_SPLITS")) want = atoi(env);
  if (want <= 0) {
    const int cus = device_cu_count();
    if (cus <= 0) return KDV_ERR_HIP;
    want = cus / p->m_tiles;
    if (want < 1) want = 1;
  }
  if (want > p->ntiles) want = p->ntiles;
  p->tiles_per_split = (p->ntiles + want - 1) / want;
  p->splits = (p->ntiles + p->tiles_per_split - 1) / p->tiles_per_split;
  const int R = d->kv_lora_rank, DQ = R + d->qk_rope_dim;
  size_t off = 0;
  p->off_qcat = off;
  off += align256((size_t)p->M * DQ * 2);
  p->off_olat = off;
  off += align256((size_t)p->M * R * 2);
  p->off_po = off;
  off += align256((size_t)p->splits * p->Mp * R * 4);
  p->off_pml = off;
  off += align256((size_t)p->splits * p->Mp * 8);
  p->total = off;
  return KDV_OK;
}

template <int DN, int R, int DR, int DV>
static void launch_all(const Plan& pl, float sm_scale, const uint16_t* q_nope, const uint16_t* q_rope,
                       const uint16_t* w_uk, const uint16_t* w_uv, const uint16_t* c_kv, const uint16_t* k_pe,
                       const int32_t* page_table, int L, int T, const uint32_t* mask, uint16_t* out, float* lse,
                       char* ws, hipStream_t st, hipEvent_t const* ev) {
  uint16_t* q_cat = reinterpret_cast<uint16_t*>(ws + pl.off_qcat);
  uint16_t* o_lat = reinterpret_cast<uint16_t*>(ws + pl.off_olat);
  float* part_o = reinterpret_cast<float*>(ws + pl.off_po);
  float2* part_ml = reinterpret_cast<float2*>(ws + pl.off_pml);
  if (ev) (void)hipEventRecord(ev[0], st);
  hipLaunchKernelGGL((q_absorb_kernel<DN, R, DR>), dim3(pl.H, (R + 127) / 128), dim3(NTHREADS), 0, st, q_nope,
                     q_rope, w_uk, q_cat, T, pl.H);
  const float scale_log2 = sm_scale * 1.44269504088896340736f;
  if (ev) (void)hipEventRecord(ev[1], st);
  hipLaunchKernelGGL((splitkv_kernel<R, DR>), dim3(pl.m_tiles * pl.splits), dim3(NTHREADS), 0, st, q_cat, c_kv,
                     k_pe, page_table, mask, L, T, pl.H, pl.M, pl.N, pl.m_tiles, pl.tiles_per_split, scale_log2,
                     part_o, part_ml, pl.Mp);
  constexpr int RPB = NTHREADS / (R / 4);
  if (ev) (void)hipEventRecord(ev[2], st);
  hipLaunchKernelGGL((combine_kernel<R>), dim3((pl.M + RPB - 1) / RPB), dim3(NTHREADS), 0, st, part_o, part_ml,
                     pl.splits, pl.Mp, pl.M, o_lat, lse);
  if (ev) (void)hipEventRecord(ev[3], st);
  hipLaunchKernelGGL((up_proj_kernel<R, DV>), dim3(pl.H, DV / 32), dim3(NTHREADS), 0, st, o_lat, w_uv, out, T,
                     pl.H);
  if (ev) (void)hipEventRecord(ev[4], st);
}

static bool misaligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) != 0; }

}  // namespace kdv

extern "C" size_t kdv_verify_workspace_bytes(const kdv_mla_dims* d, int32_t T, int32_t L) {
  kdv::Plan p;
  if (kdv::make_plan(d, T, L, &p) != KDV_OK) return 0;
  return p.total;
}

extern "C" int32_t kdv_verify_num_splits(const kdv_mla_dims* d, int32_t T, int32_t L) {
  kdv::Plan p;
  if (kdv::make_plan(d, T, L, &p) != KDV_OK) return 0;
  return p.splits;
}

static int verify_impl(const kdv_mla_dims* d, const uint16_t* q_nope, const uint16_t* q_rope,
                       const uint16_t* w_uk, const uint16_t* w_uv, const uint16_t* c_kv, const uint16_t* k_pe,
                       int64_t pool_slots, const int32_t* page_table, int32_t L, int32_t T, const uint32_t* mask,
                       uint16_t* out, float* lse, void* workspace, size_t workspace_bytes, void* stream,
                       hipEvent_t const* ev) {
  using namespace kdv;
  if (d == nullptr || q_nope == nullptr || q_rope == nullptr || w_uk == nullptr || w_uv == nullptr ||
      c_kv == nullptr || k_pe == nullptr || page_table == nullptr || mask == nullptr || out == nullptr ||
      workspace == nullptr)
    return KDV_ERR_NULL;
  const ShapeId sid = shape_of(d);
  if (sid == SHAPE_NONE || pool_slots < 1 || T < 1 || T > KDV_MAX_TREE_NODES || L < 0) return KDV_ERR_SHAPE;
  if (misaligned(q_nope, 16) || misaligned(q_rope, 16) || misaligned(w_uk, 16) || misaligned(w_uv, 16) ||
      misaligned(c_kv, 16) || misaligned(k_pe, 16) || misaligned(out, 16) || misaligned(workspace, 16) ||
      misaligned(page_table, 4) || misaligned(mask, 4) || misaligned(lse, 4))
    return KDV_ERR_ALIGN;
  Plan pl;
  const int st = make_plan(d, T, L, &pl);
  if (st != KDV_OK) return st;
  if (workspace_bytes < pl.total) return KDV_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  (void)hipGetLastError();
  if (sid == SHAPE_KIMI)
    launch_all<128, 512, 64, 128>(pl, d->sm_scale, q_nope, q_rope, w_uk, w_uv, c_kv, k_pe, page_table, L, T, mask,
                                  out, lse, ws, s, ev);
  else
    launch_all<32, 64, 16, 32>(pl, d->sm_scale, q_nope, q_rope, w_uk, w_uv, c_kv, k_pe, page_table, L, T, mask,
                               out, lse, ws, s, ev);
  return hipGetLastError() == hipSuccess ? KDV_OK : KDV_ERR_HIP;
}

extern "C" int kdv_verify_mla_attn(const kdv_mla_dims* d, const uint16_t* q_nope, const uint16_t* q_rope,
                                   const uint16_t* w_uk, const uint16_t* w_uv, const uint16_t* c_kv,
                                   const uint16_t* k_pe, int64_t pool_slots, const int32_t* page_table, int32_t L,
                                   int32_t T, const uint32_t* mask, uint16_t* out, float* lse, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  return verify_impl(d, q_nope, q_rope, w_uk, w_uv, c_kv, k_pe, pool_slots, page_table, L, T, mask, out, lse,
                     workspace, workspace_bytes, stream, nullptr);
}

extern "C" int kdv_verify_mla_attn_profiled(const kdv_mla_dims* d, const uint16_t* q_nope, const uint16_t* q_rope,
                                            const uint16_t* w_uk, const uint16_t* w_uv, const uint16_t* c_kv,
                                            const uint16_t* k_pe, int64_t pool_slots, const int32_t* page_table,
                                            int32_t L, int32_t T, const uint32_t* mask, uint16_t* out, float* lse,
                                            void* workspace, size_t workspace_bytes, void* stream,
                                            void* const* events) {
  if (events == nullptr) return KDV_ERR_NULL;
  return verify_impl(d, q_nope, q_rope, w_uk, w_uv, c_kv, k_pe, pool_slots, page_table, L, T, mask, out, lse,
                     workspace, workspace_bytes, stream, reinterpret_cast<hipEvent_t const*>(events));
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
    default: return "unknown kdv status";
  }
}
