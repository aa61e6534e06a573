// Block-sparse self-attention with summary rows, written for gfx950 (MI355X).
//
// Kernels (all launched by the extern "C" entry points at the bottom):
//   pool_q_kernel     block means of Q (float64 sums -> float32); in reweight
//                     mode also per-block float64 partial sums of the anchor rows
//   anchor_kernel     reweight only: per-head anchor = mean of the anchor rows
//   pool_kv_kernel    block means of K (for scoring), summary key/value rows and
//                     bias (mean or Spark-Reweight)
//   select_mfma_kernel  float64 block scores on the matrix cores (16 query
//                     blocks a workgroup) and a wavefront top-k with
//                     lowest-index ties, ascending output
//   select_mfma_hi_kernel  the same for top-k with only the high 32 bits of
//                     each key in LDS (two workgroups a CU); blocks that
//                     tie there are ranked by recomputed scores
//   select_kernel     the same with float64 VALU scores, past 1,200 blocks
//                     (1,280 for top-k)
//   row_order_kernel  the order in which attention visits a head's query blocks
//   attn_fwd_kernel   fused gather attention: bf16 MFMA 32x32x16, K and V
//                     tiles staged in LDS (V read back transposed), one online
//                     softmax over the extra tokens (if any), the selected
//                     blocks and the summary rows
//   token_select_kernel  extra tokens: scores of every token of the skipped
//                     blocks on the matrix cores, the E best per query block
//
// Sources of the extra tokens: "H3 Sparse Attention" (WAS Node Suite node
// page), section "The inputs that matter".
//
// Sources: "h3-sparse-attn 0.1.0" (PyPI page), opening paragraph and "Use";
// "Spark-H3: Block Sparse Attention Speeds Up MiniMax-H3 in ComfyUI",
// "What Spark-Attn changes".
#include <hip/hip_runtime.h>
#include <math.h>

#include <algorithm>
#include <mutex>
#include <stdint.h>

#include "bsa.h"

// the runtime error behind the last BSA_ERR_HIP on this thread (also set by
// the reblock calls)
static thread_local hipError_t last_hip_error = hipSuccess;
void bsa_note_hip_error(hipError_t e) { last_hip_error = e; }

namespace {

constexpr int BLK = 128;  // tokens per block
constexpr int HD = 128;   // head_dim
constexpr float LOG2E = 1.4426950408889634f;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ float bf2f(uint32_t h) { return __uint_as_float(h << 16); }

// float -> bfloat16 bits, round to nearest even (inputs here are finite)
__device__ __forceinline__ uint16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ uint4 zero_unless(uint4 u, bool keep) {
  u.x = keep ? u.x : 0u;
  u.y = keep ? u.y : 0u;
  u.z = keep ? u.z : 0u;
  u.w = keep ? u.w : 0u;
  return u;
}

__device__ __forceinline__ void unpack8(const uint4& u, double* out) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = (double)bf2f(w[i] & 0xFFFFu);
    out[2 * i + 1] = (double)bf2f(w[i] >> 16);
  }
}

// ------------------------------------------------------------------ pool ---
// One workgroup of 256 threads per (block c, head h, batch b).  Thread t owns
// the 8 features [8*(t%16), +8) of the rows {t/16 + 16*i : i < 8} of the block.
// Column sums are float64: sums of bfloat16 values are exact for these
// magnitudes, so the order of summation does not change the result.
// GATHER: the blocks are those of a row order perm (position p holds row
// perm[p]); every row is read through it.

__device__ __forceinline__ void lds_colsum(double (*red)[HD], const double* acc, int tid,
                                           double* col_out /* valid for tid < 128 */) {
  const int cc = tid & 15, rp = tid >> 4;
#pragma unroll
  for (int e = 0; e < 8; ++e) red[rp][cc * 8 + e] = acc[e];
  __syncthreads();
  if (tid < HD) {
    double s = 0.0;
#pragma unroll
    for (int i = 0; i < 16; ++i) s += red[i][tid];
    *col_out = s;
  }
  __syncthreads();
}

template <bool REWEIGHT, bool GATHER>
__global__ __launch_bounds__(256) void pool_q_kernel(const uint16_t* __restrict__ q,
                                                     const int32_t* __restrict__ perm,
                                                     float* __restrict__ q_pool,
                                                     double* __restrict__ anchor_part, int N,
                                                     int nb, int anchor_rows) {
  __shared__ double red[16][HD];
  const int c = blockIdx.x, tid = threadIdx.x;
  const size_t bh = (size_t)blockIdx.z * gridDim.y + blockIdx.y;
  const int s = c * BLK, n = min(BLK, N - s);
  const uint16_t* xb = q + bh * N * HD;
  const int cc = tid & 15, rp = tid >> 4;
  int src[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int pos = s + min(rp + 16 * i, n - 1);
    src[i] = GATHER ? perm[bh * N + pos] : pos;
  }
  double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0}, acc_a[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = rp + 16 * i;
    if (row < n) {
      double vals[8];
      unpack8(*(const uint4*)(xb + (size_t)src[i] * HD + cc * 8), vals);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += vals[e];
      if (REWEIGHT && s + row < anchor_rows) {
#pragma unroll
        for (int e = 0; e < 8; ++e) acc_a[e] += vals[e];
      }
    }
  }
  double col;
  lds_colsum(red, acc, tid, &col);
  if (tid < HD) q_pool[(bh * nb + c) * HD + tid] = (float)(col / (double)n);
  if (REWEIGHT && s < anchor_rows) {
    lds_colsum(red, acc_a, tid, &col);
    if (tid < HD) anchor_part[(bh * nb + c) * HD + tid] = col;
  }
}

// anchor[b,h,:] = (sum of the per-block partial sums) / rows.  Eight strided
// partial sums per feature (blocks c = g mod 8, in block order), combined in
// a fixed order, so the result is deterministic.
__global__ __launch_bounds__(1024) void anchor_kernel(const double* __restrict__ anchor_part,
                                                      double* __restrict__ anchor, int nb,
                                                      int anchor_rows) {
  __shared__ double part[8][HD];
  const size_t bh = (size_t)blockIdx.y * gridDim.x + blockIdx.x;
  const int d = threadIdx.x & (HD - 1), g = threadIdx.x >> 7;
  const int nblk = (anchor_rows + BLK - 1) / BLK;
  double s = 0.0;
#pragma unroll 4
  for (int c = g; c < nblk; c += 8) s += anchor_part[(bh * nb + c) * HD + d];
  part[g][d] = s;
  __syncthreads();
  if (g == 0) {
    const double t = ((part[0][d] + part[1][d]) + (part[2][d] + part[3][d])) +
                     ((part[4][d] + part[5][d]) + (part[6][d] + part[7][d]));
    anchor[bh * HD + d] = t / (double)anchor_rows;
  }
}

// GATHER also writes the block's K and V rows in the order's positions to
// k_out and v_out (the tiles the attention kernel loads).
template <bool REWEIGHT, bool GATHER>
__global__ __launch_bounds__(256) void pool_kv_kernel(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, const int32_t* __restrict__ perm,
    uint16_t* __restrict__ k_out, uint16_t* __restrict__ v_out, const double* __restrict__ anchor,
    float* __restrict__ k_pool, uint16_t* __restrict__ sum_k, uint16_t* __restrict__ sum_v,
    float* __restrict__ sum_bias, int N, int nb, double scale) {
  __shared__ double red[16][HD];
  __shared__ double rowred[16][3];
  __shared__ double lrow[BLK];  // reweight: anchor logit, then weight, of each row
  const int c = blockIdx.x, tid = threadIdx.x;
  const size_t bh = (size_t)blockIdx.z * gridDim.y + blockIdx.y;
  const int s = c * BLK, n = min(BLK, N - s);
  const uint16_t* kb = k + bh * N * HD;
  const uint16_t* vb = v + bh * N * HD;
  const int cc = tid & 15, rp = tid >> 4;
  int src[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int pos = s + min(rp + 16 * i, n - 1);
    src[i] = GATHER ? perm[bh * N + pos] : pos;
  }

  uint4 kr[8], vr[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = rp + 16 * i;
    // load a valid row (clamped) and zero it afterwards: no pointer select
    kr[i] = zero_unless(*(const uint4*)(kb + (size_t)src[i] * HD + cc * 8), row < n);
    vr[i] = zero_unless(*(const uint4*)(vb + (size_t)src[i] * HD + cc * 8), row < n);
  }
  if (GATHER) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = rp + 16 * i;
      if (row < n) {
        *(uint4*)(k_out + (bh * N + s + row) * HD + cc * 8) = kr[i];
        *(uint4*)(v_out + (bh * N + s + row) * HD + cc * 8) = vr[i];
      }
    }
  }

  double acc[8], vals[8];
  double colk, colv;
  // plain block mean of K (used for block scoring in both modes)
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    unpack8(kr[i], vals);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] += vals[e];
  }
  lds_colsum(red, acc, tid, &colk);
  const double kmean = colk / (double)n;
  if (tid < HD) k_pool[(bh * nb + c) * HD + tid] = (float)kmean;

  double sk_out = 0.0, sv_out = 0.0, bias_out = 0.0;
  if (!REWEIGHT) {
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      unpack8(vr[i], vals);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += vals[e];
    }
    lds_colsum(red, acc, tid, &colv);
    sk_out = kmean;
    sv_out = colv / (double)n;
  } else {
    // anchor logits l_j = scale * a . k_j (float64), one per row
    const double* a = anchor + bh * HD + cc * 8;
    double l[8];
    double lmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      unpack8(kr[i], vals);
      double part = 0.0;
#pragma unroll
      for (int e = 0; e < 8; ++e) part = fma(a[e], vals[e], part);
      // sum the 16 feature groups of this row (16 adjacent lanes), fixed tree
#pragma unroll
      for (int m = 1; m < 16; m <<= 1) part += __shfl_xor(part, m);
      l[i] = scale * part;
      if (rp + 16 * i < n) lmax = fmax(lmax, l[i]);
    }
    if (cc == 0) {
      rowred[rp][0] = lmax;
#pragma unroll
      for (int i = 0; i < 8; ++i) lrow[rp + 16 * i] = l[i];
    }
    __syncthreads();
    double m = rowred[0][0];
#pragma unroll
    for (int i = 1; i < 16; ++i) m = fmax(m, rowred[i][0]);
    // one float64 exponential per row (the 16 lanes of a row share it)
    if (tid < BLK) lrow[tid] = tid < n ? exp(lrow[tid] - m) : 0.0;
    __syncthreads();
    double w[8], zpart = 0.0, lsum = 0.0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const bool ok = rp + 16 * i < n;
      w[i] = lrow[rp + 16 * i];
      zpart += w[i];
      lsum += ok ? l[i] : 0.0;
    }
    if (cc == 0) { rowred[rp][1] = zpart; rowred[rp][2] = lsum; }
    __syncthreads();
    double Z = 0.0, L = 0.0;
#pragma unroll
    for (int i = 0; i < 16; ++i) { Z += rowred[i][1]; L += rowred[i][2]; }
    // weighted key and value sums
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      unpack8(kr[i], vals);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = fma(w[i], vals[e], acc[e]);
    }
    lds_colsum(red, acc, tid, &colk);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      unpack8(vr[i], vals);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = fma(w[i], vals[e], acc[e]);
    }
    lds_colsum(red, acc, tid, &colv);
    sk_out = colk / Z;
    sv_out = colv / Z;
    // log(mean exp l) - mean l ;  mean l = scale * a . kbar
    bias_out = m + log(Z) - log((double)n) - L / (double)n;
  }
  if (tid < HD) {
    sum_k[(bh * nb + c) * HD + tid] = f2bf((float)sk_out);
    sum_v[(bh * nb + c) * HD + tid] = f2bf((float)sv_out);
  }
  if (tid == 0) sum_bias[bh * nb + c] = (float)bias_out;
}

// ---------------------------------------------------------------- select ---
// One workgroup of 4 wavefronts per RB query blocks of one (b, h), on a 1-D
// grid remapped so each XCD works through whole heads.
//  1. Scores, float64 dot products of the pooled vectors (float32 products
//     are exact in float64), RB x nb of them into LDS, in one of two layouts:
//     thread-per-key (thread t owns the key blocks c = t + 256 i, i < NKT,
//     features in order 0..127, key features DCH at a time) or row-split
//     (LPK lanes share a key row; see below).
//  2. Top-k: each wavefront takes one query block at a time.  Scores become
//     order-preserving 64-bit keys held in registers (NCH keys per lane,
//     key of block c in lane c % 64); an MSB-first bitwise search finds the
//     threshold T, stopping early as soon as exactly k keys are >= the
//     candidate (then those k are the answer).  Otherwise T is the k-th
//     largest key; keys equal to T are taken lowest index first.  The chosen
//     indices are written in ascending order with ballot prefix counts.
// Every score is reduced in the same order whatever its key block, so
// identical key blocks tie bit-exactly and the lower index wins.

__device__ __forceinline__ int xcd_remap(int hw, int total) {
  // workgroups are dealt to the 8 XCDs round-robin; give each XCD a contiguous
  // range of (head, query block) so neighbouring query blocks share its L2
  const int per = total / 8, rem = total % 8;
  const int x = hw & 7, j = hw >> 3;
  return (x < rem) ? x * (per + 1) + j : rem * (per + 1) + (x - rem) * per + j;
}

// sum over the 64 lanes of a wavefront; every lane gets the same bits
__device__ __forceinline__ double wave_sum(double x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

__device__ __forceinline__ uint32_t wave_max32(uint32_t x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x = max(x, (uint32_t)__shfl_xor((int)x, off, 64));
  return x;
}

__device__ __forceinline__ uint64_t order_key(double s) {
  if (s == 0.0) s = 0.0;  // -0 ties with +0
  const uint64_t u = (uint64_t)__double_as_longlong(s);
  return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}

// Top-k phase of the select kernels: wavefront w of an NW-wavefront workgroup
// takes query rows rr = w, w + NW, ... of the RB rows whose float64 scores
// against all nb key blocks sit in sc[rr * nb + c].  Scores become
// order-preserving 64-bit keys held in registers (NCH keys per lane, key of
// block c in lane c % 64).  An MSB-first bitwise search finds the threshold
// T, first over the high 32 bits of the keys and, only if keys still tie
// there at the k-th place, over the low 32 bits of those tied keys; it stops
// as soon as exactly k keys are >= the candidate (then those k are the
// answer).  Otherwise T is the k-th largest key and keys equal to T are taken
// lowest index first.  The chosen indices are written in ascending order
// with ballot prefix counts.
template <int NCH, int NW>
__device__ __forceinline__ void select_topk_rows(const double* sc, int RB, int r0, size_t bh,
                                                 int32_t* __restrict__ block_idx, int nb, int ksel, int f0,
                                                 int f1, int thr_mode, double tau, int tid) {
  const int w = tid >> 6, lane = tid & 63;
  const uint64_t lt = (1ull << lane) - 1ull;
  for (int rr = w; rr < RB; rr += NW) {
    const int r = r0 + rr;
    if (r >= nb || ksel == 0) break;
    const double* srow = sc + rr * nb;
    // threshold mode: only scores above mean + tau * std of the row compete
    double thr = 0.0;
    if (thr_mode) {
      double sum = 0.0;
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        const int cc = i * 64 + lane;
        if (cc < nb) sum += srow[cc];
      }
      const double mean = wave_sum(sum) / nb;
      double sq = 0.0;
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        const int cc = i * 64 + lane;
        if (cc < nb) {
          const double dv = srow[cc] - mean;
          sq = fma(dv, dv, sq);
        }
      }
      thr = mean + tau * sqrt(wave_sum(sq) / nb);
    }
    uint64_t key[NCH];
    int navail = 0;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int cc = i * 64 + lane;
      // real keys are > 0 (their high half too) and 0 marks a block that
      // cannot be kept; sink blocks [f0, f1] take the largest key, so they
      // are always kept and the rest of the row is the top-k of the others
      uint64_t kv = 0ull;
      if (cc < nb) {
        if (cc >= f0 && cc <= f1)
          kv = ~0ull;
        else if (!thr_mode || srow[cc] > thr)
          kv = order_key(srow[cc]);
      }
      key[i] = kv;
      navail += __popcll(__ballot(kv != 0ull));
    }
    const int kr = min(ksel, navail);  // blocks this row keeps
    int32_t* orow = block_idx + (bh * nb + r) * (size_t)ksel;
    if (kr > 0) {
      // high halves: count of keys >= (c << 32) is the count of high halves >= c
      uint32_t th = 0;
      bool exact = false;  // exactly kr keys are >= T
      for (int bit = 31; bit >= 0; --bit) {
        const uint32_t cand = th | (1u << bit);
        int cnt = 0;
#pragma unroll
        for (int i = 0; i < NCH; ++i) cnt += __popcll(__ballot((uint32_t)(key[i] >> 32) >= cand));
        if (cnt >= kr) {
          th = cand;
          if (cnt == kr) {
            exact = true;
            break;
          }
        }
      }
      uint64_t T = (uint64_t)th << 32;
      if (!exact) {
        // th is the high half of the k-th largest key; search the low halves
        // of the keys whose high half is th (the others read 0, below every
        // candidate, which always has a bit set)
        int gt_hi = 0;
        uint32_t lo[NCH];
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
          const uint32_t h = (uint32_t)(key[i] >> 32);
          gt_hi += __popcll(__ballot(h > th));
          lo[i] = h == th ? (uint32_t)key[i] : 0u;
        }
        uint32_t tl = 0;
        for (int bit = 31; bit >= 0; --bit) {
          const uint32_t cand = tl | (1u << bit);
          int cnt = gt_hi;
#pragma unroll
          for (int i = 0; i < NCH; ++i) cnt += __popcll(__ballot(lo[i] >= cand));
          if (cnt >= kr) {
            tl = cand;
            if (cnt == kr) {
              exact = true;
              break;
            }
          }
        }
        T |= tl;
      }
      int need_eq = 0;
      if (!exact) {
        int gt = 0;
#pragma unroll
        for (int i = 0; i < NCH; ++i) gt += __popcll(__ballot(key[i] > T));
        need_eq = kr - gt;  // keys equal to T taken lowest index first
      }
      int eq_before = 0, sel_before = 0;
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        bool sel;
        if (exact) {
          sel = key[i] >= T;
        } else {
          const bool is_eq = key[i] == T;
          const uint64_t em = __ballot(is_eq);
          sel = key[i] > T || (is_eq && eq_before + (int)__popcll(em & lt) < need_eq);
          eq_before += (int)__popcll(em);
        }
        const uint64_t sm = __ballot(sel);
        if (sel) orow[sel_before + __popcll(sm & lt)] = i * 64 + lane;
        sel_before += __popcll(sm);
      }
    }
    for (int j = kr + lane; j < ksel; j += 64) orow[j] = -1;  // unused slots
  }
}

template <int NKT, int RB, bool ROWSPLIT>
__global__ __launch_bounds__(256) void select_kernel(const float* __restrict__ q_pool,
                                                     const float* __restrict__ k_pool,
                                                     int32_t* __restrict__ block_idx, int nb,
                                                     int ksel, int f0, int f1, int thr_mode,
                                                     double tau) {
  constexpr int NCH = NKT * 4;    // 64-key chunks per row in the top-k phase
  constexpr int DCH = 32 / RB;    // features per step
  extern __shared__ double sc[];  // [RB][nb]
  const int tid = threadIdx.x;
  // 1-D grid: each XCD (its own L2) works through a contiguous range of
  // (head, row group), so the pooled keys of a head are read from one L2
  const int n_rg = (nb + RB - 1) / RB;
  const int logical = xcd_remap(blockIdx.x, (int)gridDim.x);
  const int r0 = (logical % n_rg) * RB;
  const size_t bh = (size_t)(logical / n_rg);
  const float* qpb = q_pool + bh * nb * HD;
  const float* kpb = k_pool + bh * nb * HD;

  if constexpr (!ROWSPLIT) {
    double acc[NKT][RB];
#pragma unroll
    for (int i = 0; i < NKT; ++i)
#pragma unroll
      for (int rr = 0; rr < RB; ++rr) acc[i][rr] = 0.0;
    int crow[NKT];
#pragma unroll
    for (int i = 0; i < NKT; ++i) crow[i] = min(tid + 256 * i, nb - 1);  // valid row to read
    for (int d0 = 0; d0 < HD; d0 += DCH) {
      double qv[RB][DCH];
#pragma unroll
      for (int rr = 0; rr < RB; ++rr) {
        const int r = min(r0 + rr, nb - 1);
#pragma unroll
        for (int e = 0; e < DCH; ++e) qv[rr][e] = (double)qpb[(size_t)r * HD + d0 + e];
      }
#pragma unroll
      for (int i = 0; i < NKT; ++i) {
        float kv[DCH];
        if constexpr (DCH % 4 == 0) {
#pragma unroll
          for (int e = 0; e < DCH; e += 4) {
            const float4 t = *(const float4*)(kpb + (size_t)crow[i] * HD + d0 + e);
            kv[e] = t.x;
            kv[e + 1] = t.y;
            kv[e + 2] = t.z;
            kv[e + 3] = t.w;
          }
        } else {
          static_assert(DCH == 2, "feature step");
          const float2 t = *(const float2*)(kpb + (size_t)crow[i] * HD + d0);
          kv[0] = t.x;
          kv[1] = t.y;
        }
#pragma unroll
        for (int e = 0; e < DCH; ++e) {
          const double k64 = (double)kv[e];
#pragma unroll
          for (int rr = 0; rr < RB; ++rr) acc[i][rr] = fma(qv[rr][e], k64, acc[i][rr]);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < NKT; ++i) {
      const int c = tid + 256 * i;
      if (c < nb) {
#pragma unroll
        for (int rr = 0; rr < RB; ++rr) sc[rr * nb + c] = acc[i][rr];
      }
    }
  } else {
    // Large nb: LPK lanes share one key row, each lane holding 128 / LPK of
    // its features (16-byte chunks, 4 * LPK features apart), so every load of
    // the wavefront reads whole 128-byte lines; the RB query rows' matching
    // features stay in registers for the whole sweep (64 float64 values per
    // lane), and the LPK partial dot products meet in a butterfly.
    constexpr int LPK = 2 * RB, FPL = HD / LPK, CPL = FPL / 4;
    static_assert(RB * FPL == 64, "row-split scores hold 64 query values per lane");
    const int lane = tid & 63, sub = lane % LPK, grp = lane / LPK, wv = tid >> 6;
    double qv[RB][FPL];
#pragma unroll
    for (int rr = 0; rr < RB; ++rr) {
      const int r = min(r0 + rr, nb - 1);
#pragma unroll
      for (int j = 0; j < CPL; ++j) {
        const float4 t = *(const float4*)(qpb + (size_t)r * HD + 4 * LPK * j + 4 * sub);
        qv[rr][4 * j] = t.x;
        qv[rr][4 * j + 1] = t.y;
        qv[rr][4 * j + 2] = t.z;
        qv[rr][4 * j + 3] = t.w;
      }
    }
    constexpr int KPW = 64 / LPK;  // key rows per wavefront per sweep step
    for (int c0 = KPW * wv; c0 < nb; c0 += 4 * KPW) {
      const int c = c0 + grp;
      const float* krow = kpb + (size_t)min(c, nb - 1) * HD;
      double part[RB];
#pragma unroll
      for (int rr = 0; rr < RB; ++rr) part[rr] = 0.0;
#pragma unroll
      for (int j = 0; j < CPL; ++j) {
        const float4 t = *(const float4*)(krow + 4 * LPK * j + 4 * sub);
        const double kd[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
          for (int rr = 0; rr < RB; ++rr) part[rr] = fma(qv[rr][4 * j + e], kd[e], part[rr]);
      }
#pragma unroll
      for (int off = 1; off < LPK; off <<= 1)
#pragma unroll
        for (int rr = 0; rr < RB; ++rr) part[rr] += __shfl_xor(part[rr], off, 64);
      if (sub == 0 && c < nb) {
#pragma unroll
        for (int rr = 0; rr < RB; ++rr) sc[rr * nb + c] = part[rr];
      }
    }
  }
  __syncthreads();
  select_topk_rows<NCH, 4>(sc, RB, r0, bh, block_idx, nb, ksel, f0, f1, thr_mode, tau, tid);
}

// Select with the scores on the float64 matrix cores: one workgroup of NW
// wavefronts per 16 query blocks of one (b, h) (same 1-D XCD-aware grid).
// v_mfma_f64_16x16x4f64 takes 16 query rows x 16 key blocks; in step s the
// four k-slots hold features s, 32 + s, 64 + s and 96 + s (lane group g =
// lane / 16 supplies feature 32 g + s of its row), so each lane streams 32
// contiguous floats of one pooled row.  Every score sums its products in the
// same order whatever its key block, so identical key blocks tie
// bit-exactly.  Wavefront w takes key tiles w, w + NW, ... and loads the next
// tile's key rows before it multiplies the current one; lane (g, n) of a
// finished tile holds the scores of query rows g + 4 i (i < 4) against key
// block 16 T + n (the accumulator layout, checked on the chip).  Then the
// top-k phase above, one query row per wavefront at a time.
typedef double f64x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void load_row32(const float* p, float (&x)[32]) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float4 t = *(const float4*)(p + 4 * j);
    x[4 * j] = t.x;
    x[4 * j + 1] = t.y;
    x[4 * j + 2] = t.z;
    x[4 * j + 3] = t.w;
  }
}

// Score phase of the matrix-core select kernels: the 16 query rows r0 ..
// r0 + 15 of one (b, h) against all nb key blocks; store(row, c, s) takes the
// float64 score of query row r0 + row against key block c < nb.  ONEBUF: one
// register buffer of key rows and two accumulator chains (for 128 registers
// a lane, where the other wavefronts hide the loads), else two buffers and
// one chain.
template <int NW, bool ONEBUF, typename Store>
__device__ __forceinline__ void mfma_scores(const float* qpb, const float* kpb, int nb, int r0, int lane, int wave,
                                            Store&& store) {
  const int g = lane >> 4, n = lane & 15;
  float qa[32];  // A operand: row r0 + n (clamped), features 32 g + s
  load_row32(qpb + (size_t)min(r0 + n, nb - 1) * HD + 32 * g, qa);
  const int ntile = (nb + 15) / 16;
  // two register buffers of key rows: tile T + NW loads while T multiplies
  float kb[32], kn[32];
  (void)kn;
  auto tile = [&](const float(&x)[32], int T) {
    f64x4 acc = {0.0, 0.0, 0.0, 0.0};
    if constexpr (ONEBUF) {
      // steps 0..15 and 16..31 on two accumulators, added at the end (the
      // same order for every key block)
      f64x4 acc2 = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
      for (int st = 0; st < 16; ++st) {
        acc = __builtin_amdgcn_mfma_f64_16x16x4f64((double)qa[st], (double)x[st], acc, 0, 0, 0);
        acc2 = __builtin_amdgcn_mfma_f64_16x16x4f64((double)qa[st + 16], (double)x[st + 16], acc2, 0, 0, 0);
      }
      acc += acc2;
    } else {
#pragma unroll
      for (int st = 0; st < 32; ++st)
        acc = __builtin_amdgcn_mfma_f64_16x16x4f64((double)qa[st], (double)x[st], acc, 0, 0, 0);
    }
    const int c = 16 * T + n;
    if (c < nb) {
#pragma unroll
      for (int i = 0; i < 4; ++i) store(g + 4 * i, c, acc[i]);
    }
  };
  auto krow = [&](int T) { return kpb + (size_t)min(16 * T + n, nb - 1) * HD + 32 * g; };
  if constexpr (ONEBUF) {
    for (int T = wave; T < ntile; T += NW) {
      load_row32(krow(T), kb);
      tile(kb, T);
    }
  } else {
    if (wave < ntile) load_row32(krow(wave), kb);
    for (int T = wave; T < ntile; T += 2 * NW) {
      if (T + NW < ntile) load_row32(krow(T + NW), kn);
      tile(kb, T);
      if (T + NW >= ntile) break;
      if (T + 2 * NW < ntile) load_row32(krow(T + 2 * NW), kb);
      tile(kn, T + NW);
    }
  }
}

template <int NCH, int NW>
__global__ __launch_bounds__(64 * NW) void select_mfma_kernel(const float* __restrict__ q_pool,
                                                              const float* __restrict__ k_pool,
                                                              int32_t* __restrict__ block_idx, int nb, int ksel,
                                                              int f0, int f1, int thr_mode, double tau) {
  constexpr int RB = 16;
  extern __shared__ double sc[];  // [RB][nb]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n_rg = (nb + RB - 1) / RB;
  const int logical = xcd_remap(blockIdx.x, (int)gridDim.x);
  const int r0 = (logical % n_rg) * RB;
  const size_t bh = (size_t)(logical / n_rg);
  mfma_scores<NW, (NW >= 16)>(q_pool + bh * nb * HD, k_pool + bh * nb * HD, nb, r0, lane, wave,
                  [&](int row, int c, double s) { sc[row * nb + c] = s; });
  __syncthreads();
  select_topk_rows<NCH, NW>(sc, RB, r0, bh, block_idx, nb, ksel, f0, f1, thr_mode, tau, tid);
}

// Top-k phase on the high halves of the keys: sch[rr * nb + c] holds the top
// 32 bits of order_key of the float64 score, which is all the LDS has to
// keep, so two workgroups share a CU.  The bitwise search of
// select_topk_rows runs over those halves.  Where keys still tie there at the
// k-th place (scores within 2^-20 of each other, or equal), the float64
// scores of just the tied blocks are computed again, one lane each, with the
// features in ascending order (identical key blocks tie exactly again), and
// the same search over their 64-bit keys takes the rest; exact ties go lowest
// index first, and so do tied sink blocks.  Top-k mode only.
__device__ __forceinline__ double dot_f64(const float* a, const float* b) {
  double s = 0.0;
#pragma unroll 2
  for (int f = 0; f < HD; f += 4) {
    const float4 x = *(const float4*)(a + f), y = *(const float4*)(b + f);
    s = fma((double)x.x, (double)y.x, s);
    s = fma((double)x.y, (double)y.y, s);
    s = fma((double)x.z, (double)y.z, s);
    s = fma((double)x.w, (double)y.w, s);
  }
  return s;
}

// The m-th largest of the 64-bit keys (1 <= m <= number of nonzero keys; key
// of block c in lane c % 64 of slot c / 64); exact is set when exactly m keys
// are >= the result, else the result is that key itself.
template <int NCH>
__device__ __forceinline__ uint64_t kth_key64(const uint64_t (&key)[NCH], int m, bool& exact) {
  uint32_t th = 0;
  exact = false;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t cand = th | (1u << bit);
    int cnt = 0;
#pragma unroll
    for (int i = 0; i < NCH; ++i) cnt += __popcll(__ballot((uint32_t)(key[i] >> 32) >= cand));
    if (cnt >= m) {
      th = cand;
      if (cnt == m) {
        exact = true;
        return (uint64_t)th << 32;
      }
    }
  }
  int gt_hi = 0;
  uint32_t lo[NCH];
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const uint32_t h = (uint32_t)(key[i] >> 32);
    gt_hi += __popcll(__ballot(h > th));
    lo[i] = h == th ? (uint32_t)key[i] : 0u;
  }
  uint32_t tl = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t cand = tl | (1u << bit);
    int cnt = gt_hi;
#pragma unroll
    for (int i = 0; i < NCH; ++i) cnt += __popcll(__ballot(lo[i] >= cand));
    if (cnt >= m) {
      tl = cand;
      if (cnt == m) {
        exact = true;
        break;
      }
    }
  }
  return ((uint64_t)th << 32) | tl;
}

template <int NCH, int NW>
__device__ __forceinline__ void select_topk_rows_hi(const uint32_t* sch, int r0, size_t bh, const float* qpb,
                                                    const float* kpb, int32_t* __restrict__ block_idx, int nb,
                                                    int ksel, int f0, int f1, int tid) {
  const int w = tid >> 6, lane = tid & 63;
  const uint64_t lt = (1ull << lane) - 1ull;
  for (int rr = w; rr < 16; rr += NW) {
    const int r = r0 + rr;
    if (r >= nb || ksel == 0) break;
    const uint32_t* srow = sch + rr * nb;
    // every high half of a real key is > 0; sink blocks take the largest
    uint32_t key[NCH];
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int cc = i * 64 + lane;
      key[i] = cc >= nb ? 0u : (cc >= f0 && cc <= f1) ? ~0u : srow[cc];
    }
    const int kr = min(ksel, nb);
    int32_t* orow = block_idx + (bh * nb + r) * (size_t)ksel;
    uint32_t th = 0;
    bool exact = false;  // exactly kr high halves are >= th
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t cand = th | (1u << bit);
      int cnt = 0;
#pragma unroll
      for (int i = 0; i < NCH; ++i) cnt += __popcll(__ballot(key[i] >= cand));
      if (cnt >= kr) {
        th = cand;
        if (cnt == kr) {
          exact = true;
          break;
        }
      }
    }
    // th is the k-th largest high half; unless exact, the keys whose high
    // half is th are ranked by their full keys (sink blocks all alike)
    uint64_t full[NCH];
    uint64_t T2 = 0;
    bool exact2 = true;
    int need_eq = 0;
    if (!exact) {
      int gt = 0;
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        gt += __popcll(__ballot(key[i] > th));
        full[i] = 0;
        if (key[i] == th) full[i] = th == ~0u ? 1ull : order_key(dot_f64(qpb + (size_t)r * HD, kpb + (size_t)(i * 64 + lane) * HD));
      }
      const int need = kr - gt;
      T2 = kth_key64<NCH>(full, need, exact2);
      if (!exact2) {
        int gt2 = 0;
#pragma unroll
        for (int i = 0; i < NCH; ++i) gt2 += __popcll(__ballot(full[i] > T2));
        need_eq = need - gt2;  // full keys equal to T2 taken lowest index first
      }
    }
    int eq_before = 0, sel_before = 0;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      bool sel;
      if (exact) {
        sel = key[i] >= th;
      } else {
        const bool is_eq = full[i] == T2;  // T2 > 0, so only tied blocks
        const uint64_t em = __ballot(is_eq && !exact2);
        sel = key[i] > th || full[i] > T2 || (is_eq && (exact2 || eq_before + (int)__popcll(em & lt) < need_eq));
        eq_before += (int)__popcll(em);
      }
      const uint64_t sm = __ballot(sel);
      if (sel) orow[sel_before + __popcll(sm & lt)] = i * 64 + lane;
      sel_before += __popcll(sm);
    }
    for (int j = kr + lane; j < ksel; j += 64) orow[j] = -1;  // unused slots
  }
}

// Select on the matrix cores keeping only the high halves of the keys in LDS
// (16 x nb x 4 bytes): top-k mode up to 1,280 blocks, two workgroups of 8
// wavefronts per CU, so one scores while the other ranks.
template <int NCH>
__global__ __launch_bounds__(512, 4) void select_mfma_hi_kernel(const float* __restrict__ q_pool,
                                                               const float* __restrict__ k_pool,
                                                               int32_t* __restrict__ block_idx, int nb, int ksel,
                                                               int f0, int f1) {
  constexpr int RB = 16, NW = 8;
  extern __shared__ uint32_t sch[];  // [RB][nb]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n_rg = (nb + RB - 1) / RB;
  const int logical = xcd_remap(blockIdx.x, (int)gridDim.x);
  const int r0 = (logical % n_rg) * RB;
  const size_t bh = (size_t)(logical / n_rg);
  const float* qpb = q_pool + bh * nb * HD;
  const float* kpb = k_pool + bh * nb * HD;
  mfma_scores<NW, true>(qpb, kpb, nb, r0, lane, wave,
                  [&](int row, int c, double s) { sch[row * nb + c] = (uint32_t)(order_key(s) >> 32); });
  __syncthreads();
  select_topk_rows_hi<NCH, NW>(sch, r0, bh, qpb, kpb, block_idx, nb, ksel, f0, f1, tid);
}

// ------------------------------------------------------------ row order ---
// The order in which the attention grid visits one head's query blocks: by
// their first three kept blocks, then by block (a bitonic sort of 64-bit keys
// in LDS, one workgroup per head).  Every query block walks its kept blocks
// in ascending order, so workgroups that run at the same time on an XCD then
// start on the same key blocks and meet in its L2 (measured inside whole
// steps: attention 2.7% faster at 295 blocks, 1.6% at 1,045).  Conditioning
// sink query blocks [f0, f1] (dense rows, the longest) come first.  The
// attention calls on a reblocked row order keep that order instead.
__global__ __launch_bounds__(1024) void row_order_kernel(const int32_t* __restrict__ block_idx,
                                                         int32_t* __restrict__ order, int nb, int krow, int f0,
                                                         int f1) {
  __shared__ uint64_t key[BSA_MAX_BLOCKS];
  const size_t bh = blockIdx.x;
  const int tid = threadIdx.x;
  int n2 = 1;
  while (n2 < nb) n2 <<= 1;
  for (int i = tid; i < n2; i += 1024) {
    uint64_t kv = ~0ull;  // padding sorts last
    if (i < nb) {
      const int32_t* row = block_idx + (bh * nb + i) * (size_t)krow;
      kv = (uint64_t)i;  // bits [0, 11): the block; three 12-bit fields above
      if (i < f0 || i > f1) {
        // a kept block c enters as c + 1 >= 1, so these sort after the sink rows
        kv |= (uint64_t)1 << 47;
#pragma unroll
        for (int j = 0; j < 3; ++j)
          if (j < krow) kv |= (uint64_t)(row[j] + 1) << (11 + 12 * (2 - j));  // -1 padding -> 0
      }
    }
    key[i] = kv;
  }
  __syncthreads();
  for (int size = 2; size <= n2; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = tid; i < (n2 >> 1); i += 1024) {
        const int lo = 2 * i - (i & (stride - 1)), hi = lo + stride;
        const uint64_t a = key[lo], b = key[hi];
        if ((a > b) == ((lo & size) == 0)) {
          key[lo] = b;
          key[hi] = a;
        }
      }
      __syncthreads();
    }
  }
  for (int i = tid; i < nb; i += 1024) order[bh * nb + i] = (int32_t)(key[i] & 2047u);
}

// ------------------------------------------------------------- attention ---
// One workgroup (4 wavefronts, 2 workgroups per CU) per (b, h, query block r):
// 128 query rows, wavefront w owning queries [32w, 32w + 32).  The keys are
// walked in half tiles of 64: the two halves of every selected block, then
// the summary rows in groups of 64.
//
// Software pipeline, per half tile t (one barrier each):
//   - direct global->LDS loads of K(t+2) and V(t+1) are issued first;
//   - the MFMAs of S(t+1) = K(t+1) Q^T run interleaved with the softmax of
//     S(t) (computed one step earlier), so the matrix cores and the vector
//     ALUs of one wavefront work at the same time;
//   - then O^T += V^T(t) P(t)^T, with P(t) taken straight from the S^T
//     accumulator layout and the V^T operand read from the row-major V tile
//     by transposing LDS reads.
// K is therefore staged two half tiles ahead and V one ahead, in two LDS
// buffers each (64 KB per workgroup).  Lane l holds query 32w + l%32; lanes l
// and l^32 hold the two halves of its 64 keys.
//
// The running max only moves when a tile's max exceeds it by more than
// LAZY_MAX (base-2 units), so O is rescaled rarely; probabilities stay below
// 2^LAZY_MAX, far from float or bfloat16 overflow.

constexpr int HT = 64;            // keys per half tile
constexpr float LAZY_MAX = 8.0f;

// K half tile: 64 rows x 256 B of 16-byte chunks; chunk c of row `row` at
// position c ^ (row & 15), so the K operand reads (16 lanes x 16 B from 16
// consecutive rows) touch all 64 banks.
__device__ __forceinline__ int swz_k(int row, int chunk) { return row * HD + ((chunk ^ (row & 15)) << 3); }
// V half tile, laid out for transposing reads (ds_read_b64_tr_b16 takes, in
// each group of 16 lanes, 4 rows x 16 columns: lane 4e + c supplies row e's
// columns 4c..4c+3, lane i receives column i): 128-byte blocks of 4 keys x
// 16 features (row-major), four blocks (key quads 4g, feature halves h1) per
// 512-byte unit, one unit per (key slice kk of 16, half of it, feature block
// db of 32).  Key 16 kk + 8 half + 4 g + e, feature chunk 4 db + 2 h1 + c2
// (8 features) sits at 16-byte slot 32 (8 kk + 4 half + db) + 8 (2 g + h1) +
// 2 e + c2, so every transposing read covers one unit: 512 contiguous bytes
// (measured about 20% faster per read than a bank-spread row-major pattern).
__device__ __forceinline__ int vslot(int key, int ch) {
  const int u = 8 * (key >> 4) + 4 * ((key >> 3) & 1) + (ch >> 2);
  return 32 * u + 8 * (2 * ((key >> 2) & 1) + ((ch >> 1) & 1)) + 2 * (key & 3) + (ch & 1);
}

__device__ __forceinline__ bf16x8 ld_bf16x8(const uint16_t* p) { return *(const bf16x8*)p; }

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4* lds_bf16x4_ptr;

// Transposing LDS read (ds_read_b64_tr_b16).  Within each group of 16 lanes,
// lane 4e + c supplies the address of columns [4c, 4c + 4) of row e, and
// lane i receives column i of rows 0..3 (element e from row e).
__device__ __forceinline__ bf16x4 ld_tr4(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_ptr)(p));
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// value of lane l ^ 32 (a VALU lane swap, no LDS round trip)
__device__ __forceinline__ float other_half(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  // one of the two results holds this lane's half, the other the partner's
  const float a = __uint_as_float(r[0]), b = __uint_as_float(r[1]);
  return (a == x) ? b : a;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  // raw buffer: byte offsets at or beyond `bytes` read as zero
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

struct TileSrc {
  uint32_t off;    // byte offset of the half tile's first row (K and V, or sum_k and sum_v)
  int nvalid;      // rows of the half tile that exist (may be <= 0)
  int c0;          // summary tiles: first summary block
  bool summary;
};

__global__ __launch_bounds__(256, 2) void attn_fwd_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ sum_k, const uint16_t* __restrict__ sum_v, const float* __restrict__ sum_bias,
    const int32_t* __restrict__ block_idx, const int32_t* __restrict__ tok_idx, const int32_t* __restrict__ perm,
    const int32_t* __restrict__ order, uint16_t* __restrict__ out, int N, int nb, int krow, float scale_log2,
    int total_wg, int chunk, int f0, int f1, int E) {
  // LDS buffers as distinct variables, so the compiler can tell the DMA
  // targets from the buffers being read
  __shared__ __attribute__((aligned(16))) uint16_t ks0[HT * HD], ks1[HT * HD];
  __shared__ __attribute__((aligned(16))) uint16_t vs0[HD * HT], vs1[HD * HT];
  __shared__ float addv0[HT], addv1[HT];
  __shared__ uint32_t selmask[BSA_MAX_BLOCKS / 32];
  __shared__ int32_t sidx[BSA_MAX_BLOCKS];  // this query block's selected blocks
  __shared__ int32_t tokl[BSA_MAX_EXTRA];    // this query block's extra tokens

  // Workgroup -> (b, h, position in the head's visiting order).  Workgroups
  // are dealt to the 8 XCDs round-robin.  With chunk = 0 each XCD takes a
  // contiguous range of (head, position), so the longer dense sink rows,
  // first in each head's order, spread over the XCDs and start first.
  // With chunk > 0 XCD x takes positions [x chunk, x chunk + chunk) of
  // every head in turn, so the XCDs all work on the same one or two heads at
  // a time and their L2 misses meet in the memory-side cache, while each L2
  // still sees neighbouring query blocks; padding workgroups past nb leave at
  // once.
  int rr;
  size_t bh;
  if (chunk > 0) {
    const int x = blockIdx.x & 7, j = blockIdx.x >> 3;
    rr = x * chunk + j % chunk;
    bh = (size_t)(j / chunk);
    if (rr >= nb) return;  // uniform over the workgroup, before any barrier
  } else {
    const int logical = xcd_remap(blockIdx.x, total_wg);
    rr = logical % nb;
    bh = (size_t)(logical / nb);
  }
  // position rr of the head's visiting order (row_order_kernel), else (no
  // selection) rr blocks after the first sink block
  const int r = order ? order[bh * nb + rr] : (rr + f0) % nb;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keep in SGPRs
  const int g = lane >> 5, ln = lane & 31;

  const float* biasb = sum_bias ? sum_bias + bh * (size_t)nb : nullptr;
  const int32_t* irow = block_idx + (bh * nb + r) * (size_t)krow;
  // a conditioning sink query block attends to every key block exactly
  const bool dense_row = r >= f0 && r <= f1;
  const int kslots = dense_row ? nb : krow;
  // per-head buffer descriptors: K, V, summary K, summary V (rows past the
  // end of a buffer read as zeros)
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(k + bh * (size_t)N * HD, (uint32_t)N * HD * 2);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(v + bh * (size_t)N * HD, (uint32_t)N * HD * 2);
  const __amdgpu_buffer_rsrc_t rsk =
      make_rsrc(sum_k ? sum_k + bh * (size_t)nb * HD : k, sum_k ? (uint32_t)nb * HD * 2 : 0u);
  const __amdgpu_buffer_rsrc_t rsv =
      make_rsrc(sum_v ? sum_v + bh * (size_t)nb * HD : v, sum_v ? (uint32_t)nb * HD * 2 : 0u);

  // Q fragments (B operand of S^T = K Q^T): query qi, features 16kk + 8g + [0, 8).
  // With a row order perm, query qi (a position) is row perm[qi] of q and
  // of out; k and v already hold their rows in the new order.
  const int qi = r * BLK + 32 * wave + ln;
  bf16x8 qf[8];
  {
    const int qpos = min(qi, N - 1);
    const uint16_t* qrow = q + (bh * (size_t)N + (size_t)(perm ? perm[bh * N + qpos] : qpos)) * HD;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      bf16x8 t = ld_bf16x8(qrow + 16 * kk + 8 * g);
      if (qi >= N) t = bf16x8{};
      qf[kk] = t;
    }
  }

  const int nwords = (nb + 31) >> 5;
  for (int i = tid; i < nwords; i += 256) selmask[i] = 0u;
  __syncthreads();
  // the row's kept blocks: a prefix of its slots, -1 padding after them
  // (threshold selection keeps a different number per row)
  int kcount = 0;
  for (int base = 0; base < kslots; base += 256) {
    const int i = base + tid;
    const int c = i < kslots ? (dense_row ? i : irow[i]) : -1;
    if (c >= 0) {
      sidx[i] = c;
      atomicOr(&selmask[c >> 5], 1u << (c & 31));
    }
    kcount += __syncthreads_count(c >= 0);
  }
  const int ksel = __builtin_amdgcn_readfirstlane(kcount);
  __syncthreads();

  const int n_exact = 2 * ksel;
  // summary half tiles: only those holding rows below nb (a group of 128
  // summary rows past the end contributes nothing)
  const int ntiles = n_exact + ((ksel < nb) ? (nb + HT - 1) / HT : 0);

  // block index of half tile t (exact tiles), read from LDS; issued one step
  // before describe() needs it
  auto tile_block = [&](int t) {
    t = min(t, ntiles - 1);
    return t < n_exact ? sidx[t >> 1] : 0;
  };
  auto describe = [&](int t, int c) {
    t = min(t, ntiles - 1);  // past the end: the last half tile again (never used)
    TileSrc d;
    const int h = t & 1;
    if (t < n_exact) {
      const int row0 = c * BLK + h * HT;
      d.off = (uint32_t)row0 * (HD * 2);
      d.nvalid = min(HT, N - row0);
      d.c0 = 0;
      d.summary = false;
    } else {
      const int st = (t - n_exact) >> 1;
      const int row0 = st * BLK + h * HT;
      d.off = (uint32_t)row0 * (HD * 2);
      d.nvalid = min(HT, nb - row0);
      d.c0 = row0;
      d.summary = true;
    }
    return d;
  };

  // Direct global -> LDS loads.  Instruction j of wavefront w fills the 64
  // consecutive 16-byte LDS slots P = (4w + j) * 64 + lane; each lane
  // fetches the global chunk that the tile's layout places there.  K: row
  // 16w + 4j + lane/16 at position lane % 16, offset kbase + 1024 j +
  // (kx ^ 64 j).  V (slot -> key, chunk: the inverse of vslot): key
  // 16 w + 8 (j / 2) + 4 ((lane / 16) & 1) + (lane / 2) % 4, chunk
  // 4 (2 (j & 1) + lane / 32) + 2 ((lane / 8) & 1) + lane % 2, offset vbase +
  // 2048 (j / 2) + 128 (j & 1).  Rows past the end of the buffer (ragged
  // tails) arrive as zeros.
  const uint32_t kbase = (uint32_t)((16 * wave + (lane >> 4)) * (HD * 2));
  const uint32_t kx = (uint32_t)(((lane & 15) ^ (lane >> 4)) * 16);
  const uint32_t vbase = (uint32_t)((16 * wave + 4 * ((lane >> 4) & 1) + ((lane >> 1) & 3)) * (HD * 2) +
                                    (4 * (lane >> 5) + 2 * ((lane >> 3) & 1) + (lane & 1)) * 16);
  auto kvo = [&](int j) { return kbase + 1024u * j + (kx ^ (64u * j)); };
  auto load_k1 = [&](const TileSrc& d, uint16_t* ksd, int j) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(d.summary ? rsk : rk, (lds_ptr_t)(ksd + (4 * wave + j) * 512),
                                             16, (int)(d.off + kvo(j)), 0, 0, 0);
  };
  auto load_v1 = [&](const TileSrc& d, uint16_t* vsd, int j) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(d.summary ? rsv : rv, (lds_ptr_t)(vsd + (4 * wave + j) * 512),
                                             16, (int)(d.off + vbase + 2048u * (j >> 1) + 128u * (j & 1)), 0, 0, 0);
  };
  auto load_k = [&](const TileSrc& d, uint16_t* ksd) {
#pragma unroll
    for (int j = 0; j < 4; ++j) load_k1(d, ksd, j);
  };
  auto load_v = [&](const TileSrc& d, uint16_t* vsd) {
#pragma unroll
    for (int j = 0; j < 4; ++j) load_v1(d, vsd, j);
  };
  // additive logit term of each key of a half tile (base-2 units)
  // Only summary tiles and the short halves of the last block need it; full
  // exact half tiles skip it (their softmax reads no additive term).
  auto mask_value = [&](const TileSrc& d) {
    float a = 0.f;
    if (tid < HT) {
      if (!d.summary) {
        a = tid < d.nvalid ? 0.f : -INFINITY;
      } else {
        const int c = d.c0 + tid;
        const bool skipped = c < nb && !((selmask[c >> 5] >> (c & 31)) & 1u);
        a = skipped ? biasb[c] * LOG2E : -INFINITY;
      }
    }
    return a;
  };
  auto store_mask = [&](const TileSrc& d, float a, float* addvd) {
    if (tid < HT && (d.summary || d.nvalid < HT)) {
      // the lane index recomputed here (wavefront 0: lane == tid) instead of
      // an address kept across the loop, which the register allocator would
      // spill: its reload waits for every direct-to-LDS load in flight
      int l;
      asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
      addvd[l] = a;
    }
  };

  // V^T operand of O^T += V^T P^T for feature block db (32 features) and
  // key slice kk (16 keys), from the V tile by two transposing reads, of the
  // units (kk, half 0, db) and (kk, half 1, db): lane l = 32 g + 16 h1 + i
  // addresses element 4 l of the unit, i.e. key 16 kk + 8 half + 4 g + i / 4,
  // features 32 db + 16 h1 + 4 (i % 4) .. +3, and receives feature
  // 32 db + 16 h1 + i = 32 db + ln of keys 16 kk + 4 g + {0..3} and
  // 16 kk + 8 + 4 g + {0..3}: exactly the eight keys, in the same order, that
  // its P operand (the S^T accumulator of query ln) holds.  The address is
  // the lane's 4 l plus compile-time offsets.
  auto v_operand_db = [&](const uint16_t* vsc, int db, int kk) {
    const uint16_t* p = vsc + 4 * lane + 256 * (8 * kk + db);
    const bf16x4 a = ld_tr4(p), b = ld_tr4(p + 1024);
    return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  };

  f32x16 o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) o[db] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;
  f32x16 sA[2], sB[2];
  if (E > 0 && !dense_row) {
    // Extra tokens first, 64 at a time: their K and V rows gathered straight
    // into LDS in the tile layout by the direct-to-LDS loads (each lane reads
    // the row of its slot's token; the loads of group g + 1 fly while group g
    // is computed, in the other buffer pair), then S^T = K Q^T, a softmax
    // update with the exact max and O^T += V^T P^T.  The state (o, m_run,
    // l_run) carries into the online softmax of the main loop.
    const int t_in = tid < E ? tok_idx[(bh * nb + r) * (size_t)E + tid] : -1;
    tokl[tid] = t_in;
    const int nval = __syncthreads_count(t_in >= 0);  // valid tokens come first
    // byte offset of row i of the token list; past the valid tokens, the end
    // of the buffer (those rows read as zeros)
    const uint32_t past_end = (uint32_t)N * (HD * 2);
    auto tok_off = [&](int i) { return i < nval ? (uint32_t)tokl[i] * (HD * 2) : past_end; };
    // the slot -> (row, chunk) maps of the tile loads (see load_k1, load_v1)
    const int krow0 = 16 * wave + (lane >> 4);
    const uint32_t kxg = (uint32_t)(((lane & 15) ^ (lane >> 4)) * 16);
    const int vrow0 = 16 * wave + 4 * ((lane >> 4) & 1) + ((lane >> 1) & 3);
    const uint32_t vch = (uint32_t)((4 * (lane >> 5) + 2 * ((lane >> 3) & 1) + (lane & 1)) * 16);
    auto gather = [&](int base, uint16_t* kd, uint16_t* vd) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_ptr_t)(kd + (4 * wave + j) * 512), 16,
                                                 (int)(tok_off(base + krow0 + 4 * j) + (kxg ^ (64u * j))), 0, 0, 0);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_ptr_t)(vd + (4 * wave + j) * 512), 16,
                                                 (int)(tok_off(base + vrow0 + 8 * (j >> 1)) + vch + 128u * (j & 1)),
                                                 0, 0, 0);
    };
    const int ngroups = (nval + HT - 1) / HT;
    if (ngroups > 0) gather(0, ks0, vs0);
    for (int gi = 0; gi < ngroups; ++gi) {
      const int base = gi * HT;
      const uint16_t* kc = (gi & 1) ? ks1 : ks0;
      const uint16_t* vc = (gi & 1) ? vs1 : vs0;
      if (gi + 1 < ngroups) {
        // the next group into the pair the previous group read (free since
        // the barrier that ended it); then wait for this group's 8 loads only
        gather(base + HT, (gi & 1) ? ks0 : ks1, (gi & 1) ? vs0 : vs1);
        asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
      } else {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      }
      __syncthreads();
      // S^T: sA[mb] element ii is key base + 32 mb + 8 (ii / 4) + 4 g + ii % 4
      sA[0] = f32x16{};
      sA[1] = f32x16{};
#pragma unroll
      for (int i = 0; i < 16; ++i)
        sA[i & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            ld_bf16x8(kc + swz_k(32 * (i & 1) + ln, 2 * (i >> 1) + g)), qf[i >> 1], sA[i & 1], 0, 0, 0);
      float mx = -INFINITY;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int ii = 0; ii < 16; ++ii) {
          const int key = base + 32 * mb + 8 * (ii >> 2) + 4 * g + (ii & 3);
          const float x = key < nval ? sA[mb][ii] * scale_log2 : -INFINITY;
          sA[mb][ii] = x;
          mx = fmaxf(mx, x);
        }
      mx = fmaxf(mx, other_half(mx));
      const float m_new = fmaxf(m_run, mx);  // finite: the group holds a token
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      // P slice kk: keys 16 kk + 8 (e / 4) + 4 g + e % 4, e = 0..7
      bf16x8 pb[4];
      float psum = 0.f;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        typedef uint16_t u16x8_t __attribute__((ext_vector_type(8)));
        u16x8_t pu;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint16_t pbits = f2bf(__builtin_amdgcn_exp2f(sA[kk >> 1][8 * (kk & 1) + e] - m_new));
          pu[e] = pbits;
          psum += bf2f(pbits);
        }
        pb[kk] = __builtin_bit_cast(bf16x8, pu);
      }
      l_run = l_run * alpha + psum;
#pragma unroll
      for (int db = 0; db < 4; ++db) o[db] *= alpha;
#pragma unroll
      for (int i = 0; i < 16; ++i)
        o[i & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v_operand_db(vc, i & 3, i >> 2), pb[i >> 2], o[i & 3],
                                                           0, 0, 0);
      __syncthreads();
    }
  }

  // ---------------------------------------------------------------------
  // S^T(t) = K Q^T : s[mb] holds keys 32mb + 8(i/4) + 4g + i%4 of the half
  // tile.  MFMA number i of a half tile uses mb = i & 1, kk = i >> 1, so the
  // two accumulators alternate.
  // element offset of K slice kk for key row ln (key block half mb adds 32
  // rows): swz_k(ln, 2 kk + g); eight per lane, computed once (left to
  // itself the compiler keeps one address register per read, and the
  // register pressure spilled a value whose reload waits for every load in
  // flight; measured 0.7% faster at 768p)
  int koff[8];
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) koff[kk] = swz_k(ln, 2 * kk + g);
  auto k_operand = [&](const uint16_t* ksc, int i) {
    return ld_bf16x8(ksc + 32 * HD * (i & 1) + koff[i >> 1]);
  };
  auto v_operand = [&](const uint16_t* vsc, int i) {  // i = 4 kk + db
    return v_operand_db(vsc, i & 3, i >> 2);
  };

  // prologue S(0), plain order
  auto qk_plain = [&](const uint16_t* ksc, f32x16* s) {
    s[0] = f32x16{};
    s[1] = f32x16{};
#pragma unroll
    for (int i = 0; i < 16; ++i)
      s[i & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k_operand(ksc, i), qf[i >> 1], s[i & 1], 0, 0, 0);
  };

  // Region A of a half tile: the 16 MFMAs of S(t+1) = K(t+1) Q^T, each
  // followed by one slice of the softmax of S(t).  Slot work:
  //   0-3   scale (+ additive term) and running max over 8 of the 32 values
  //   4     exchange the max with the partner lane (l ^ 32)
  //   5     new reference max, rescale factor
  //   6-13  exponentials of 4 values, bf16 packing, row sum
  // Returns the O rescale factor (1 unless the reference max moved).
  auto region_a = [&](const uint16_t* kn, f32x16* sn, f32x16* sc, bool need_add,
                      const float* addvc, bf16x8* pb, const TileSrc& dk, uint16_t* kd,
                      const TileSrc& dv, uint16_t* vd, const uint16_t* vc, bf16x8* vpre) -> float {
    // K operands read three slots ahead (0.4-0.7% faster than two)
    bf16x8 kop0 = k_operand(kn, 0), kop1 = k_operand(kn, 1), kop2 = k_operand(kn, 2), kop3;
    float mx = -INFINITY, m_use = 0.f, alpha = 1.f, psum = 0.f;
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (i + 3 < 16) kop3 = k_operand(kn, i + 3);
      sn[i & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop0, qf[i >> 1], i < 2 ? f32x16{} : sn[i & 1],
                                                          0, 0, 0);
      if (i < 4) {
        // values v = 8i .. 8i+7 : mb = i >> 1, elements 8(i&1) .. +7
        const int mb = i >> 1, e0 = 8 * (i & 1);
        float m = -INFINITY;
        if (need_add) {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int ii = e0 + e;
            const float x = fmaf(sc[mb][ii], scale_log2, addvc[32 * mb + 8 * (ii >> 2) + 4 * g + (ii & 3)]);
            sc[mb][ii] = x;
            m = fmaxf(m, x);
          }
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) m = fmaxf(m, sc[mb][e0 + e]);
        }
        mx = (i == 0) ? m : fmaxf(mx, m);
      } else if (i == 4) {
        if (!need_add) mx *= scale_log2;
        mx = fmaxf(mx, other_half(mx));
      } else if (i == 5) {
        const float m_new = (mx > m_run + LAZY_MAX) ? mx : m_run;
        m_use = (m_new == -INFINITY) ? 0.f : m_new;
        alpha = __builtin_amdgcn_exp2f(m_run - m_use);
        m_run = m_new;
        psum = l_run * alpha;
      } else if (i >= 6 && i < 14) {
        // half slice j: keys of P slice kk = j >> 1, elements 4(j&1) .. +3
        const int j = i - 6, kk = j >> 1, e0 = 4 * (j & 1);
        const int mb = kk >> 1, base = 8 * (kk & 1) + e0;
        float p[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float x = sc[mb][base + e];
          p[e] = need_add ? __builtin_amdgcn_exp2f(x - m_use)
                          : __builtin_amdgcn_exp2f(fmaf(x, scale_log2, -m_use));
        }
        const bf16x2 p01 = __builtin_convertvector((float __attribute__((ext_vector_type(2)))){p[0], p[1]}, bf16x2);
        const bf16x2 p23 = __builtin_convertvector((float __attribute__((ext_vector_type(2)))){p[2], p[3]}, bf16x2);
        pb[kk][e0 + 0] = p01[0];
        pb[kk][e0 + 1] = p01[1];
        pb[kk][e0 + 2] = p23[0];
        pb[kk][e0 + 3] = p23[1];
        psum = __builtin_amdgcn_fdot2_f32_bf16(p01, one, psum, false);
        psum = __builtin_amdgcn_fdot2_f32_bf16(p23, one, psum, false);
      }
      // spread the 8 direct-to-LDS loads of the next half tiles over the
      // region (one every second slot) instead of issuing them back to back
      if ((i & 1) == 0) {
        const int j = i >> 1;
        if (j < 4)
          load_k1(dk, kd, j);
        else
          load_v1(dv, vd, j - 4);
      }
      kop0 = kop1;
      kop1 = kop2;
      kop2 = kop3;
      // the first two V^T operands of region B, read in the last two slots
      // (V^T(t) has been in LDS since the step began; 0.3-0.5% faster)
      if (i >= 14) vpre[i - 14] = v_operand(vc, i - 14);
      // no scheduling fence here: the compiler's own interleaving of the
      // slots measures about 1.5% faster than a fixed slot order
    }
    l_run = psum;
    return alpha;
  };

  // Region B: O^T += V^T(t) P(t)^T, 16 MFMAs (db fastest: 4 independent chains)
  auto region_b = [&](const uint16_t* vc, const bf16x8* pb, const bf16x8* vpre, auto&& bookkeeping) {
    // operands read three slots ahead (region B has no VALU work to hide
    // the LDS latency behind); the first two come from region A
    bf16x8 vop0 = vpre[0], vop1 = vpre[1], vop2 = v_operand(vc, 2), vop3;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (i + 3 < 16) vop3 = v_operand(vc, i + 3);
      o[i & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop0, pb[i >> 2], o[i & 3], 0, 0, 0);
      // the next step's descriptors and key mask, in the issue slots this
      // MFMA-only region leaves free
      if (i == 4) bookkeeping();
      vop0 = vop1;
      vop1 = vop2;
      vop2 = vop3;
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // prologue: K(0), K(1), V(0) and the masks of tile 0; S(0)
  TileSrc d0 = describe(0, tile_block(0)), d1 = describe(1, tile_block(1)), d2 = describe(2, tile_block(2));
  load_k(d0, ks0);
  load_k(d1, ks1);
  load_v(d0, vs0);
  store_mask(d0, mask_value(d0), addv0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  qk_plain(ks0, sA);
  __syncthreads();  // every wavefront is done with ks0 before K(2) lands there

  // half tile t: d0 = tile t, d1 = t+1, d2 = t+2.  Reads K(t+1) from kn and
  // V(t) from vc; loads K(t+2) into kd and V(t+1) into vd.
  auto step = [&](f32x16* sc, f32x16* sn, const uint16_t* kn, const uint16_t* vc,
                  uint16_t* kd, uint16_t* vd, const float* addvc, float* addvn, int t) {
    const bool need_add = d0.summary || d0.nvalid < HT;
    // early: the block index of half tile t+3 and the mask of half tile t+1
    const int c3 = tile_block(t + 3);
    const float mask1 = mask_value(d1);
    bf16x8 pb[4], vpre[2];
    float alpha;
    // the softmax-heavy region issues at raised priority so its VALU work
    // is not starved by the other wavefront's MFMA-only region on this SIMD
    __builtin_amdgcn_s_setprio(3);
    if (need_add)
      alpha = region_a(kn, sn, sc, true, addvc, pb, d2, kd, d1, vd, vc, vpre);
    else
      alpha = region_a(kn, sn, sc, false, addvc, pb, d2, kd, d1, vd, vc, vpre);
    if (__ballot(alpha != 1.0f)) {
#pragma unroll
      for (int db = 0; db < 4; ++db) o[db] *= alpha;
    }
    __builtin_amdgcn_s_setprio(0);
    region_b(vc, pb, vpre, [&]() {
      store_mask(d1, mask1, addvn);
      d0 = d1;
      d1 = d2;
      d2 = describe(t + 3, c3);
    });
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  };

  for (int t = 0; t < ntiles; t += 2) {
    step(sA, sB, ks1, vs0, ks0, vs1, addv0, addv1, t);
    if (t + 1 < ntiles) step(sB, sA, ks0, vs1, ks1, vs0, addv1, addv0, t + 1);
  }

  const float l_tot = l_run + other_half(l_run);
  const float inv = 1.f / l_tot;
  if (qi < N) {
    uint16_t* orow = out + (bh * (size_t)N + (size_t)(perm ? perm[bh * N + qi] : qi)) * HD;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d0o = 32 * db + 8 * r4 + 4 * g;
        const uint32_t w0 = (uint32_t)f2bf(o[db][4 * r4 + 0] * inv) |
                            ((uint32_t)f2bf(o[db][4 * r4 + 1] * inv) << 16);
        const uint32_t w1 = (uint32_t)f2bf(o[db][4 * r4 + 2] * inv) |
                            ((uint32_t)f2bf(o[db][4 * r4 + 3] * inv) << 16);
        *(uint2*)(orow + d0o) = make_uint2(w0, w1);
      }
    }
  }
}

// ---------------------------------------------------------- extra tokens ---
// Besides its kept blocks, each query block r reads exactly the E tokens j of
// the blocks it skipped with the largest q_pool[r] . k_j, equal scores going
// to the lower token; every skipped block keeps its summary row.
// Source: "H3 Sparse Attention" (WAS Node Suite node page), section "The
// inputs that matter" (extra_tokens: per query block, individually
// highest-scoring tokens on top of its selected blocks; 256 by default).
//
// token_select_kernel: one workgroup of 8 wavefronts (two per SIMD) per 32
// query blocks of one (b, h), on a 1-D grid remapped like the select kernel.
//  - Scores on the matrix cores (16x16x32 bf16): C^T = K Qs^T, Qs holding
//    every pooled query split exactly into three bfloat16 terms (hi + mid +
//    lo equals the float32 value), so each product is exact and the sums are
//    float32.  Wavefront w scores tokens 32 (w % 4) + [0, 32) of every block
//    against query blocks 16 (w / 4) + [0, 16); lane l of an accumulator
//    holds query block l % 16 and 4 tokens.  The feature order inside the
//    products is free, so each load reads 64 contiguous bytes of a token row.
//  - Each query block keeps a candidate list in LDS of 64-bit keys: the
//    order-preserving float32 score above, the complemented token index below
//    (so equal scores rank the lower token higher).  A token enters when the
//    upper half of its key reaches the row's threshold.  Before a step whose
//    128 new tokens could overflow a list, the list is cut to its `keep`
//    largest keys and the threshold rises to the smallest kept one; every key
//    dropped is below `keep` kept ones.
//  - Two phases.  First the sample blocks (one in TS_STRIDE), keeping the m
//    best of each row in its list: the m-th key T_m is a lower bound of the
//    row's E-th key whenever at least E candidates reach T_m.  Then the
//    other blocks with the threshold fixed at T_m: wavefront w scores token
//    eighth w of each block against all 32 query blocks (two B operands, so
//    each token is loaded once per workgroup: the loads, 16 rows x 64 bytes
//    per instruction, bound this phase) and appends the keys reaching T_m to
//    its own workspace segment per (query block, token eighth), with no
//    lists, atomics or barriers; a merge takes the E best of a row's phase-1
//    keys and segments.  A row with fewer than
//    E keys reaching T_m (an unrepresentative sample) or with an overflowing
//    segment is redone from an empty list over every block by the
//    list-and-cut sweep.  With one block in S sampled, m = E/S + 8 sqrt(E/S)
//    sets T_m near the 2E- to 3E-th score (S = 8: for E = 256 the fewest
//    candidates reaching T_m measured on the 768p inputs was 1.6 E, the most
//    5 E).  S = 12 measured 6% faster than 8 there (a shorter sample phase),
//    16 slower.  Small E (< 64) runs the list-and-cut sweep over every block
//    directly.
//  - In the list-and-cut sweep each step handles one key block (32 tokens
//    per wavefront); inserts need no atomics: each token quarter publishes
//    its per-row counts, and after a barrier every lane derives positions.
//  - At the end each list is cut to E and written in ascending token order
//    (a token's slot is the number of kept tokens below it), -1 after.
//  - One workgroup per CU (its LDS), so the groups run in rounds of 256.
//    The groups past the last whole round split their key blocks into up to
//    8 ranges (parts), so that round fills the chip.  A part runs all of the
//    above over its own range, samples one block in 6 (so that few blocks
//    still give a safe threshold) and leaves its E best keys per row in the
//    workspace.  token_merge_kernel then takes each row's E best over its
//    parts.  Every score is computed as in a whole group, so the tokens are
//    the same.

constexpr int TS_ROWS = 32;    // query blocks per workgroup
constexpr int TS_CAP = 512;    // candidate keys per query block
constexpr int TS_STRIDE = 12;  // blocks c with c % TS_STRIDE == 3 form the sample
constexpr int TS_STRIDE_PART = 6;  // the same for a part of a group
constexpr int TS_SEGS = 8;     // workspace segments per query block in phase 2 (token eighths)
constexpr int SEG_CAP = 256;   // keys per segment
constexpr int TS_MAX_PARTS = 8;  // parts a group of the last dispatch round may split into
constexpr int TS_CUS = 256;      // compute units of the chip: one token-select workgroup each

__device__ __forceinline__ uint32_t order_key32(float s) {
  if (s == 0.f) s = 0.f;  // -0 ties with +0
  const uint32_t u = __float_as_uint(s);
  return (u >> 31) ? ~u : (u | 0x80000000u);
}

// The `keep` largest of the distinct keys (hi, lo) a wavefront holds, PER
// per lane (empty slots hi = 0, real keys have hi != 0; keep <= number of
// real keys): kept are those with hi > T, or hi == T and (exact or lo >= L).
// An MSB-first bitwise search on the upper halves (the score keys) stops as
// soon as exactly `keep` keys reach the candidate; only when several keys
// share the upper half at the boundary does a second search order those by
// their lower halves (larger = lower token).
//
// lb, when nonzero, is a lower bound of the keep-th largest upper half: the
// bits above the highest one on which it and the largest upper half differ
// are then taken at once.
template <int PER>
__device__ void top_keys(const uint32_t (&hi)[PER], const uint32_t (&lo)[PER], int keep, uint32_t& T,
                         uint32_t& L, bool& exact, uint32_t lb = 0u) {
  T = 0u;
  exact = false;
  int top = 31;
  if (lb != 0u) {
    uint32_t mx = 0u;
#pragma unroll
    for (int j = 0; j < PER; ++j) mx = max(mx, hi[j]);
    mx = wave_max32(mx);
    const uint32_t x = lb ^ mx;
    top = x == 0u ? -1 : 31 - __clz(x);
    T = top < 0 ? mx : mx & ~((2u << top) - 1u);
  }
  for (int bit = top; bit >= 0; --bit) {
    const uint32_t cand = T | (1u << bit);
    int c = 0;
#pragma unroll
    for (int j = 0; j < PER; ++j) c += __popcll(__ballot(hi[j] >= cand));
    if (c >= keep) {
      T = cand;
      if (c == keep) {
        exact = true;
        break;
      }
    }
  }
  L = 0u;
  if (!exact) {
    int gt = 0;
#pragma unroll
    for (int j = 0; j < PER; ++j) gt += __popcll(__ballot(hi[j] > T));
    const int need = keep - gt;
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t cand = L | (1u << bit);
      int c = 0;
#pragma unroll
      for (int j = 0; j < PER; ++j) c += __popcll(__ballot(hi[j] == T && lo[j] >= cand));
      if (c >= need) {
        L = cand;
        if (c == need) break;
      }
    }
  }
}

// Writes the kept keys to list[0, keep) in (slot, lane) order and returns
// the smallest kept key.
template <int PER>
__device__ uint64_t write_kept(uint64_t* list, const uint32_t (&hi)[PER], const uint32_t (&lo)[PER],
                               uint32_t T, uint32_t L, bool exact, int lane) {
  const uint64_t lt = (1ull << lane) - 1ull;
  int before = 0;
  uint64_t kmin = ~0ull;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const bool sel = hi[j] > T || (hi[j] == T && (exact || lo[j] >= L));
    const uint64_t m = __ballot(sel);
    const uint64_t kv = ((uint64_t)hi[j] << 32) | lo[j];
    if (sel) {
      list[before + __popcll(m & lt)] = kv;
      kmin = kv < kmin ? kv : kmin;
    }
    before += __popcll(m);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const uint64_t o = __shfl_xor(kmin, off, 64);
    kmin = o < kmin ? o : kmin;
  }
  return kmin;
}

// Cuts a candidate list (n distinct keys, each with a nonzero upper half;
// keep <= n <= TS_CAP) to its `keep` largest keys and returns the smallest
// kept key.  One wavefront.
__device__ uint64_t cut_list(uint64_t* list, int n, int keep, int lane) {
  constexpr int PER = TS_CAP / 64;
  uint32_t hi[PER], lo[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int x = lane + 64 * j;
    const uint64_t kv = x < n ? list[x] : 0ull;
    hi[j] = (uint32_t)(kv >> 32);
    lo[j] = (uint32_t)kv;
  }
  uint32_t T, L;
  bool exact;
  top_keys<PER>(hi, lo, keep, T, L, exact);
  return write_kept<PER>(list, hi, lo, T, L, exact, lane);
}

// The tokens of n <= E kept keys in ascending order, -1 after, into orow[0, E).
// A token's slot is the number of kept tokens below it, i.e. of kept keys
// with a larger lower half.  One wavefront.
__device__ void write_tokens(const uint64_t* keys, int n, int E, int32_t* orow, int lane) {
  uint32_t lo[BSA_MAX_EXTRA / 64];
  int rank[BSA_MAX_EXTRA / 64];
#pragma unroll
  for (int j = 0; j < BSA_MAX_EXTRA / 64; ++j) {
    const int y = lane + 64 * j;
    lo[j] = y < n ? (uint32_t)keys[y] : 0u;
    rank[j] = 0;
  }
  for (int y = 0; y < n; ++y) {
    const uint32_t o = (uint32_t)keys[y];
#pragma unroll
    for (int j = 0; j < BSA_MAX_EXTRA / 64; ++j) rank[j] += o > lo[j];
  }
#pragma unroll
  for (int j = 0; j < BSA_MAX_EXTRA / 64; ++j) {
    const int y = lane + 64 * j;
    if (y < n) orow[rank[j]] = (int32_t)(0xFFFFFFFFu - lo[j]);
  }
  for (int y = n + lane; y < E; y += 64) orow[y] = -1;
}

typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));

typedef float f32x4 __attribute__((ext_vector_type(4)));

// 8 wavefronts, two per SIMD, so one wavefront's inserts, cuts and barrier
// waits overlap the other's matrix work.  Wavefront w takes the 32 tokens
// [32 (w % 4), +32) of each step's block against the 16 query blocks
// 16 (w / 4) + [0, 16), as two 16x16x32 MFMA tiles.
constexpr int TS_THREADS = 512;

__global__ __launch_bounds__(TS_THREADS, 1) void token_select_kernel(
    const float* __restrict__ q_pool, const uint16_t* __restrict__ k,
    const int32_t* __restrict__ block_idx, int32_t* __restrict__ token_idx,
    uint64_t* __restrict__ gseg, uint64_t* __restrict__ pseg, uint64_t* __restrict__ plist,
    int32_t* __restrict__ pcount, int N, int nb, int krow, int E, int m_whole, int m_part, int f0, int f1,
    int n_whole, int parts) {
  // row strides padded by one element, so that lanes of different rows at
  // equal positions fall into different LDS banks
  __shared__ uint64_t list[TS_ROWS][TS_CAP + 1];
  __shared__ uint32_t skip[TS_ROWS][BSA_MAX_BLOCKS / 32 + 1];  // bit c: row skipped block c
  __shared__ uint16_t order[BSA_MAX_BLOCKS];                    // sample blocks first, then the rest
  __shared__ uint64_t tm[TS_ROWS];                              // T_m, 0 for none
  // list sizes and the keys each token quarter inserts in a step, both
  // double-buffered by step parity: a step reads one copy and writes the
  // other, so no wavefront overwrites a value another still reads
  __shared__ int cnt[2][TS_ROWS];
  __shared__ int cw[2][TS_SEGS][TS_ROWS];
  __shared__ int nge[TS_ROWS];        // rows to redo (phase 2 could not decide them)
  __shared__ int segcnt[TS_SEGS][TS_ROWS];  // keys per workspace segment, -1 when it overflowed
  __shared__ uint32_t thr[TS_ROWS];
  __shared__ int redo;

  // workgroups [0, n_whole) take whole groups; the rest take one part (a
  // range of key blocks) each of the last groups, `parts` per group
  const int ngrp = (nb + TS_ROWS - 1) / TS_ROWS;
  const int wg = (int)blockIdx.x;
  const int pidx = wg - n_whole;  // part workgroup index, < 0 for a whole group
  const int logical = pidx < 0 ? xcd_remap(wg, n_whole) : n_whole + pidx / parts;
  const int c_lo = pidx < 0 ? 0 : (pidx % parts) * nb / parts;
  const int c_hi = pidx < 0 ? nb : (pidx % parts + 1) * nb / parts;
  const int nbr = c_hi - c_lo;  // key blocks this workgroup visits
  const int r0 = (logical % ngrp) * TS_ROWS;
  const size_t bh = (size_t)(logical / ngrp);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, q4 = lane >> 4;
  const int nwords = (nb + 31) >> 5;
  // sample blocks c % S == 3 below c: S = TS_STRIDE for a whole group, the
  // denser TS_STRIDE_PART for a part (its range holds few blocks, and a
  // sample of a few blocks misjudges a row's threshold more often), each with
  // its own m
  const int S = pidx < 0 ? TS_STRIDE : TS_STRIDE_PART;
  const int m = pidx < 0 ? m_whole : m_part;
  auto n_sample_below = [&](int c) { return (c + S - 4) / S; };
  const int n1 = m > 0 ? n_sample_below(c_hi) - n_sample_below(c_lo) : 0;  // sample blocks
  // workspace segments of row xr of the group (TS_SEGS x SEG_CAP keys)
  auto seg_row = [&](int xr) {
    return pidx < 0 ? gseg + (bh * nb + (size_t)min(r0 + xr, nb - 1)) * TS_SEGS * SEG_CAP
                    : pseg + ((size_t)pidx * TS_ROWS + xr) * TS_SEGS * SEG_CAP;
  };

  // candidates of row r0 + i: the blocks it did not keep; none for a sink
  // query block (it attends to every block exactly) or past the last row
  for (int x = tid; x < TS_ROWS * nwords; x += TS_THREADS) {
    const int i = x / nwords, wd = x % nwords, r = r0 + i;
    uint32_t mk = 0u;
    if (r < nb && !(r >= f0 && r <= f1)) {
      // the bits of blocks [c_lo, c_hi) in word wd
      const int lo = max(c_lo - 32 * wd, 0), hi = min(c_hi - 32 * wd, 32);
      if (hi > lo) mk = (hi == 32 ? 0xFFFFFFFFu : ((1u << hi) - 1u)) & ~((1u << lo) - 1u);
    }
    skip[i][wd] = mk;
  }
  if (tid < TS_ROWS) {
    cnt[0][tid] = 0;
    nge[tid] = 0;
    thr[tid] = 0u;
    tm[tid] = 0ull;
  }
  if (tid == 0) redo = 0;
  // visiting order of the blocks [c_lo, c_hi): the sample blocks (c % S ==
  // 3) first, then the others, each in block order
  for (int c = c_lo + tid; c < c_hi; c += TS_THREADS) {
    const bool smp = n1 > 0 && c % S == 3;
    const int below = n1 > 0 ? n_sample_below(c) - n_sample_below(c_lo) : 0;  // sample blocks in [c_lo, c)
    order[smp ? below : n1 + (c - c_lo) - below] = (uint16_t)c;
  }
  __syncthreads();
  for (int x = tid; x < TS_ROWS * krow; x += TS_THREADS) {
    const int i = x / krow, r = r0 + i;
    if (r < nb) {
      const int c = block_idx[(bh * nb + r) * (size_t)krow + (x - i * krow)];
      if (c >= 0) atomicAnd(&skip[i][c >> 5], ~(1u << (c & 31)));
    }
  }

  // B operand of query block r0 + qr: features 32 s + 8 q4 + [0, 8) for
  // k-step s, as three exact bfloat16 terms
  auto split_q = [&](int qr, bf16x8(&qs)[3][4]) {
    const float* qp = q_pool + (bh * nb + min(r0 + qr, nb - 1)) * HD + 8 * q4;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      u16x8 hi, mid, lo;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = qp[32 * s + e];
        const uint16_t h = f2bf(x);
        const float r1 = x - bf2f(h);  // exact
        const uint16_t md = f2bf(r1);
        const float r2 = r1 - bf2f(md);  // exact, at most 8 significant bits
        hi[e] = h;
        mid[e] = md;
        lo[e] = f2bf(r2);
      }
      qs[0][s] = __builtin_bit_cast(bf16x8, hi);
      qs[1][s] = __builtin_bit_cast(bf16x8, mid);
      qs[2][s] = __builtin_bit_cast(bf16x8, lo);
    }
  };
  __syncthreads();

  // A operand (K) of a tile: tile row j of key block c, features 32 s +
  // 8 q4 + [0, 8) for k-step s (so each load instruction reads 64 contiguous
  // bytes of every row it touches).  Past the end of the sequence the last
  // row is read again: such a token's scores fill only its own accumulator
  // row and it is never inserted, so the loaded data needs no zeroing (and a
  // load needs no wait until the MFMAs that read it).
  const uint16_t* kb = k + bh * (size_t)N * HD;

  // value of lane l ^ 16 and of lane l ^ 32 (VALU lane swaps)
  auto lane_x16 = [&](int x) {
    const auto r = __builtin_amdgcn_permlane16_swap((unsigned)x, (unsigned)x, false, false);
    return (int)((lane & 16) ? r[0] : r[1]);
  };
  auto lane_x32 = [&](int x) {
    const auto r = __builtin_amdgcn_permlane32_swap((unsigned)x, (unsigned)x, false, false);
    return (int)((lane & 32) ? r[0] : r[1]);
  };

  // Token eighths (every phase): wavefront w scores tokens 8 j + w (j < 16)
  // of a key block against all 32 query blocks of the group, with two B
  // operands, so each token is loaded once per workgroup.  Tile row j is
  // token 8 j + w, so lane l holds tokens 8 (4 q4 + v) + w (v < 4) against
  // query blocks l16 and 16 + l16 (row halves h = 0, 1).  Taking every
  // eighth token (not 16 adjacent ones, which tend to score alike) spreads a
  // row's keys evenly over its workspace segments in phase 2.
  const int te = wave;
  auto load8 = [&](int c, uint4* kt) {  // key block c
    const uint16_t* src = kb + (size_t)min(c * BLK + 8 * l16 + te, N - 1) * HD + 8 * q4;
#pragma unroll
    for (int s = 0; s < 4; ++s) kt[s] = *(const uint4*)(src + 32 * s);
  };
  // each score's chain: k-steps in order, small terms first; the two row
  // halves' chains alternate
  auto mfma_rows = [&](const uint4* kt, f32x4* acc, const bf16x8(&qh)[2][3][4]) {
    acc[0] = f32x4{};
    acc[1] = f32x4{};
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int term = 2; term >= 0; --term)
#pragma unroll
        for (int h = 0; h < 2; ++h)
          acc[h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kt[s]), qh[h][term][s],
                                                           acc[h], 0, 0, 0);
  };

  // One sweep over order[i0, i1) with lists cut to `keep`.  List sizes start
  // and end in cnt[0] (a sweep runs a multiple of 4 steps).
  auto sweep = [&](int i0, int i1, int keep) {
    bf16x8 qh[2][3][4];
    split_q(l16, qh[0]);
    split_q(16 + l16, qh[1]);
    uint32_t thr_reg[2] = {thr[l16], thr[16 + l16]};
    // Step i (software pipeline): the MFMAs of tile i+1 and the loads of tile
    // i+3 go out first; the keys of tile i (scored by the previous step) are
    // filtered by the row threshold and each token eighth publishes how many
    // it inserts per row; between the two barriers the lists that would
    // overflow are cut; then every lane writes its keys at positions given by
    // the list size and the counts of the eighths before it (no atomics).
    // Every step issues the same loads and waits (no branch around them), so
    // each tile's MFMAs wait only for that tile's own loads, issued two steps
    // earlier.
    auto step = [&](int i, const f32x4* acc, f32x4* accn, const uint4* kn, uint4* kl) {
      const int par = (i - i0) & 1;
      mfma_rows(kn, accn, qh);
      __builtin_amdgcn_sched_barrier(0);
      load8((int)order[min(i + 3, i1 - 1)], kl);
      // keys of tile i: value v of row half h is token tb + 8 v.  A score's
      // key reaches the threshold key exactly when the score reaches the
      // float with that key (the key map is monotone; -0 counts as +0)
      const int c = order[min(i, i1 - 1)];
      const int tb = c * BLK + 32 * q4 + te;
      uint32_t mask[2];
      int before[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int xr = 16 * h + l16;
        const float thr_f = thr_reg[h] == 0u ? -INFINITY
                            : (thr_reg[h] >> 31) ? __uint_as_float(thr_reg[h] & 0x7FFFFFFFu)
                                                 : __uint_as_float(~thr_reg[h]);
        uint32_t mk = 0u;
        if (i < i1 && ((skip[xr][c >> 5] >> (c & 31)) & 1u)) {
#pragma unroll
          for (int v = 0; v < 4; ++v) mk |= (acc[h][v] >= thr_f ? 1u : 0u) << v;
          if (tb + 24 >= N) {  // the last block: tokens past the end
#pragma unroll
            for (int v = 0; v < 4; ++v) mk &= tb + 8 * v < N ? ~0u : ~(1u << v);
          }
        }
        mask[h] = mk;
        // the row's four lanes of this wavefront (q4 = 0..3): their total and
        // this lane's offset among them (lane swaps across 16 and 32)
        const int pc = __popc(mk);
        const int p16 = lane_x16(pc), pair = pc + p16, p32 = lane_x32(pair);
        before[h] = ((q4 & 1) ? p16 : 0) + ((q4 & 2) ? p32 : 0);
        if (q4 == 0) cw[par][te][xr] = pair + p32;
      }
      __syncthreads();
      // a list whose keys this step could overflow is cut first; a wavefront
      // cuts only its own rows (x = wave mod 8)
      const int lr = lane & (TS_ROWS - 1);
      int grow = 0;
#pragma unroll
      for (int q = 0; q < TS_SEGS; ++q) grow += cw[par][q][lr];
      const uint64_t full = __ballot(lane < TS_ROWS && cnt[par][lr] + grow > TS_CAP);
      if (full) {
        for (int x = wave; x < TS_ROWS; x += TS_THREADS / 64) {
          if ((full >> x) & 1ull) {
            const uint64_t T = cut_list(list[x], cnt[par][x], keep, lane);
            if (lane == 0) {
              cnt[par][x] = keep;
              thr[x] = (uint32_t)(T >> 32);
            }
          }
        }
      }
      __syncthreads();
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int xr = 16 * h + l16;
        thr_reg[h] = thr[xr];
        int pos = cnt[par][xr] + before[h], tot = 0;
#pragma unroll
        for (int q = 0; q < TS_SEGS; ++q) {
          const int cq = cw[par][q][xr];
          pos += q < te ? cq : 0;
          tot += cq;
        }
        if (te == 0 && q4 == 0) cnt[par ^ 1][xr] = cnt[par][xr] + tot;
        for (uint32_t mm = mask[h]; mm != 0u; mm &= mm - 1u) {  // set bits, lowest first
          const int v = __builtin_ctz(mm);
          float sv = acc[h][0];
#pragma unroll
          for (int u = 1; u < 4; ++u) sv = v == u ? acc[h][u] : sv;
          const uint32_t t = (uint32_t)(tb + 8 * v);
          list[xr][pos++] = ((uint64_t)order_key32(sv) << 32) | (uint64_t)(0xFFFFFFFFu - t);
        }
      }
    };
    f32x4 accA[2], accB[2];
    uint4 kA[4], kB[4], kC[4], kD[4];
    load8((int)order[min(i0, i1 - 1)], kA);
    load8((int)order[min(i0 + 1, i1 - 1)], kB);
    load8((int)order[min(i0 + 2, i1 - 1)], kC);
    mfma_rows(kA, accA, qh);
    for (int i = i0; i < i1; i += 4) {
      step(i, accA, accB, kB, kD);
      step(i + 1, accB, accA, kC, kA);
      step(i + 2, accA, accB, kD, kB);
      step(i + 3, accB, accA, kA, kC);
    }
    __syncthreads();
  };

  if (n1 > 0) {
    // phase 1: the sample, keeping the m best of each row
    sweep(0, n1, m);
    for (int x = wave; x < TS_ROWS; x += TS_THREADS / 64) {
      const int n = cnt[0][x];
      if (n >= m) {
        const uint64_t T = cut_list(list[x], n, m, lane);
        if (lane == 0) {
          cnt[0][x] = m;
          tm[x] = T;
          thr[x] = (uint32_t)(T >> 32);
        }
      }
    }
    __syncthreads();
  }
  if (n1 > 0) {
    // Phase 2 (filter): with the rows' thresholds fixed at T_m, every key
    // reaching its row's T_m goes to the wavefront's own workspace segment
    // for that row (token eighth), at positions the row's four lanes agree
    // on; no lists, no atomics, no barriers.  Strided eighths: fullest
    // segment 193 of 256 keys at 768p, E = 256, against 257 (an overflow)
    // with 16 adjacent tokens per eighth.
    {
      bf16x8 qh[2][3][4];
      split_q(l16, qh[0]);
      split_q(16 + l16, qh[1]);
      float thr_f[2];
      uint64_t* seg[2];
      int scount[2] = {0, 0};  // the same in the row's four lanes
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t th = (uint32_t)(tm[16 * h + l16] >> 32);
        thr_f[h] = th == 0u ? -INFINITY : (th >> 31) ? __uint_as_float(th & 0x7FFFFFFFu) : __uint_as_float(~th);
        seg[h] = seg_row(16 * h + l16) + te * SEG_CAP;
      }
      auto fstep = [&](int i, const f32x4* acc, f32x4* accn, const uint4* kn, uint4* kl) {
        mfma_rows(kn, accn, qh);
        __builtin_amdgcn_sched_barrier(0);
        load8((int)order[min(max(i + 3, n1), nbr - 1)], kl);
        const int c = order[min(max(i, n1), nbr - 1)];
        const int tb = c * BLK + 32 * q4 + te;  // value v: token tb + 8 v
        const bool in_range = i >= n1 && i < nbr;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int xr = 16 * h + l16;
          uint32_t mask = 0u;
          if (in_range && ((skip[xr][c >> 5] >> (c & 31)) & 1u)) {
#pragma unroll
            for (int v = 0; v < 4; ++v) mask |= (acc[h][v] >= thr_f[h] ? 1u : 0u) << v;
            if (tb + 24 >= N) {  // the last block: tokens past the end
#pragma unroll
              for (int v = 0; v < 4; ++v) mask &= tb + 8 * v < N ? ~0u : ~(1u << v);
            }
          }
          const int pc = __popc(mask);
          const int p16 = lane_x16(pc), pair = pc + p16, p32 = lane_x32(pair);
          int pos = scount[h] + ((q4 & 1) ? p16 : 0) + ((q4 & 2) ? p32 : 0);
          for (uint32_t mm = mask; mm != 0u; mm &= mm - 1u) {  // set bits, lowest first
            const int v = __builtin_ctz(mm);
            float sv = acc[h][0];
#pragma unroll
            for (int u = 1; u < 4; ++u) sv = v == u ? acc[h][u] : sv;
            const uint32_t t = (uint32_t)(tb + 8 * v);
            if (pos < SEG_CAP) seg[h][pos] = ((uint64_t)order_key32(sv) << 32) | (uint64_t)(0xFFFFFFFFu - t);
            ++pos;
          }
          scount[h] += pair + p32;
        }
      };
      // the pipeline fills inside the loop (three steps on zeroed buffers
      // before tile n1), so no load is in flight when the loop is entered
      // and every tile's MFMAs wait only for that tile's own loads
      f32x4 accA[2] = {f32x4{}, f32x4{}}, accB[2] = {f32x4{}, f32x4{}};
      uint4 kA[4], kB[4], kC[4], kD[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) kA[j] = kB[j] = kC[j] = kD[j] = make_uint4(0u, 0u, 0u, 0u);
      for (int i = n1 - 3; i < nbr; i += 4) {
        fstep(i, accA, accB, kB, kD);
        fstep(i + 1, accB, accA, kC, kA);
        fstep(i + 2, accA, accB, kD, kB);
        fstep(i + 3, accB, accA, kA, kC);
      }
      if (q4 == 0) {
#pragma unroll
        for (int h = 0; h < 2; ++h) segcnt[te][16 * h + l16] = scount[h] <= SEG_CAP ? scount[h] : -1;
      }
    }
    __syncthreads();
    // Merge: each row's phase-1 keys and its eight segments; the E best of
    // them are the row's answer when at least E keys reach T_m (then no key
    // below T_m can be among the E best) and no segment overflowed.
    for (int x = wave; x < TS_ROWS; x += TS_THREADS / 64) {
      const int r = r0 + x;
      bool bad = false;
      if (r < nb) {
        int c[TS_SEGS], total = cnt[0][x];
        const int n0 = total;
#pragma unroll
        for (int q = 0; q < TS_SEGS; ++q) {
          c[q] = segcnt[q][x];
          bad |= c[q] < 0;
          total += max(c[q], 0);
        }
        if (!bad) {
          // fixed register slots: the phase-1 keys, then SPER per segment
          constexpr int LPER = TS_CAP / 64, SPER = SEG_CAP / 64;
          constexpr int PER = LPER + TS_SEGS * SPER;
          uint32_t hi[PER], lo[PER];
          const uint64_t tmx = tm[x];
          const uint64_t* sb = seg_row(x);
          int nge_l = 0;
#pragma unroll
          for (int j = 0; j < PER; ++j) {
            uint64_t kv = 0ull;
            if (j < LPER) {
              const int y = lane + 64 * j;
              if (y < n0) kv = list[x][y];
            } else {
              const int q = (j - LPER) / SPER, y = lane + 64 * ((j - LPER) % SPER);
              if (y < c[q]) kv = sb[q * SEG_CAP + y];
            }
            hi[j] = (uint32_t)(kv >> 32);
            lo[j] = (uint32_t)kv;
            nge_l += (kv != 0ull && kv >= tmx);
          }
          int nge_w = nge_l;
#pragma unroll
          for (int off = 32; off > 0; off >>= 1) nge_w += __shfl_xor(nge_w, off, 64);
          if (tmx != 0ull && nge_w < E) {
            bad = true;
          } else {
            const int keep = min(E, total);
            if (keep > 0) {
              // at least E keys reach T_m, so the E-th largest does too
              uint32_t T, L;
              bool exact;
              top_keys<PER>(hi, lo, keep, T, L, exact, (uint32_t)(tmx >> 32));
              write_kept<PER>(list[x], hi, lo, T, L, exact, lane);
            }
            if (lane == 0) cnt[0][x] = keep;
          }
        }
      }
      if (lane == 0) nge[x] = bad ? 1 : 0;
    }
    __syncthreads();
    // rows phase 2 could not decide are redone from an empty list over
    // every block with the list-and-cut sweep
    if (tid < TS_ROWS && nge[tid]) atomicOr(&redo, 1);
    __syncthreads();
    if (redo) {
      for (int x = tid; x < TS_ROWS * nwords; x += TS_THREADS) {
        const int i = x / nwords;
        if (!nge[i]) skip[i][x % nwords] = 0u;
      }
      __syncthreads();
      if (tid < TS_ROWS) {
        if (nge[tid]) {
          cnt[0][tid] = 0;
          thr[tid] = 0u;
        }
        tm[tid] = 0ull;
      }
      __syncthreads();
      sweep(0, nbr, E);
    }
  } else {
    // small E (or a part without sample blocks): one list-and-cut sweep over
    // every block
    sweep(0, nbr, E);
  }

  for (int x = wave; x < TS_ROWS; x += TS_THREADS / 64) {
    const int r = r0 + x;
    if (r >= nb) break;
    int n = cnt[0][x];
    if (n > E) {
      cut_list(list[x], n, E, lane);
      n = E;
    }
    if (pidx < 0) {
      write_tokens(list[x], n, E, token_idx + (bh * nb + r) * (size_t)E, lane);
    } else {
      // a part: its E best keys, for token_merge_kernel
      uint64_t* prow = plist + ((size_t)pidx * TS_ROWS + x) * E;
      for (int y = lane; y < n; y += 64) prow[y] = list[x][y];
      if (lane == 0) pcount[pidx * TS_ROWS + x] = n;
    }
  }
}

// One query block of the last groups: the E best keys of its parts' lists
// (disjoint key ranges, so every key is distinct), written as tokens in
// ascending order.  One wavefront a row, 8 rows a workgroup.
__global__ __launch_bounds__(512) void token_merge_kernel(const uint64_t* __restrict__ plist,
                                                          const int32_t* __restrict__ pcount,
                                                          int32_t* __restrict__ token_idx, int nb, int E,
                                                          int n_whole, int parts, int n_rows) {
  constexpr int EPL = BSA_MAX_EXTRA / 64, PER = TS_MAX_PARTS * EPL;
  __shared__ uint64_t kept[8][BSA_MAX_EXTRA];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int xa = blockIdx.x * 8 + wave;  // row slot over the last groups
  if (xa >= n_rows) return;
  const int ngrp = (nb + TS_ROWS - 1) / TS_ROWS;
  const int logical = n_whole + xa / TS_ROWS, x = xa % TS_ROWS;
  const int r = (logical % ngrp) * TS_ROWS + x;
  if (r >= nb) return;
  const size_t bh = (size_t)(logical / ngrp);
  uint32_t hi[PER], lo[PER];
  int total = 0;
#pragma unroll
  for (int q = 0; q < TS_MAX_PARTS; ++q) {
    const int pidx = (xa / TS_ROWS) * parts + q;
    const int n = q < parts ? pcount[pidx * TS_ROWS + x] : 0;
    const uint64_t* prow = plist + ((size_t)pidx * TS_ROWS + x) * E;
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
      const int y = lane + 64 * j;
      const uint64_t kv = y < n ? prow[y] : 0ull;
      hi[q * EPL + j] = (uint32_t)(kv >> 32);
      lo[q * EPL + j] = (uint32_t)kv;
    }
    total += n;
  }
  const int keep = min(E, total);
  if (keep > 0) {
    uint32_t T, L;
    bool exact;
    top_keys<PER>(hi, lo, keep, T, L, exact);
    write_kept<PER>(kept[wave], hi, lo, T, L, exact, lane);
  }
  write_tokens(kept[wave], keep, E, token_idx + (bh * nb + r) * (size_t)E, lane);
}

// ------------------------------------------------------------------ host ---
struct Geometry {
  int64_t B, H, N, nb, k;
  int64_t f0, f1;  // conditioning sink blocks [f0, f1]; f1 < f0 when there are none
  bool threshold;
  double tau;
  bool reweight;
  int anchor_rows;
  double scale;
  int E;  // extra tokens per query block
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Scratch of each call, always from the start of the workspace: no call
// reads anything that another call left there.
//   pool (reweight only): float64 anchor partial sums [B, H, nb, 128], then
//     the anchor [B, H, 128] at pool_anchor_off();
//   forward: the visiting order of each head's query blocks, int32 [B, H, nb];
//   select_tokens: key segments, u64 [B, H, nb, TS_SEGS, SEG_CAP]; then, when
//     the last groups split into parts (token_split), each part's segments
//     u64 [parts total, TS_ROWS, TS_SEGS, SEG_CAP], its E best keys per row
//     u64 [parts total, TS_ROWS, E] and their counts int32 [parts total,
//     TS_ROWS].
size_t pool_anchor_off(const Geometry& g) { return align256((size_t)(g.B * g.H * g.nb) * HD * sizeof(double)); }
size_t pool_ws(const Geometry& g) {
  return g.reweight ? pool_anchor_off(g) + align256((size_t)(g.B * g.H) * HD * sizeof(double)) : 0;
}
size_t forward_ws(const Geometry& g) { return align256((size_t)(g.B * g.H * g.nb) * sizeof(int32_t)); }
// Token selection runs one workgroup per CU; groups of TS_ROWS query blocks
// past the last whole dispatch round split their key blocks into `parts`
// ranges (a workgroup each, merged by token_merge_kernel), so that the last
// round fills the chip.  The first n_whole groups run whole.
void token_split(const Geometry& g, int* n_whole, int* parts) {
  const int G = (int)(((g.nb + TS_ROWS - 1) / TS_ROWS) * g.H * g.B);
  const int tail = G > TS_CUS ? G % TS_CUS : 0;
  int P = tail > 0 ? std::min(TS_MAX_PARTS, std::min(TS_CUS / tail, (int)g.nb)) : 1;
  if (P < 2) P = 1;
  *parts = P;
  *n_whole = P > 1 ? G - tail : G;
}
size_t tokens_seg_bytes(const Geometry& g) {
  return align256((size_t)(g.B * g.H * g.nb) * TS_SEGS * SEG_CAP * sizeof(uint64_t));
}
size_t tokens_ws(const Geometry& g) {
  if (g.E == 0) return 0;
  int n_whole, parts;
  token_split(g, &n_whole, &parts);
  const size_t G = (size_t)((g.nb + TS_ROWS - 1) / TS_ROWS) * g.H * g.B;
  const size_t prow = parts > 1 ? (G - n_whole) * parts * TS_ROWS : 0;  // part rows
  return tokens_seg_bytes(g) + align256(prow * TS_SEGS * SEG_CAP * sizeof(uint64_t)) +
         align256(prow * g.E * sizeof(uint64_t)) + align256(prow * sizeof(int32_t));
}
size_t ws_total(const Geometry& g) { return std::max(pool_ws(g), std::max(forward_ws(g), tokens_ws(g))); }

int make_geometry(const bsa_problem* p, Geometry* g) {
  if (!p) return BSA_ERR_INVALID;
  if (p->head_dim != BSA_HEAD_DIM || p->block_size != BSA_BLOCK) return BSA_ERR_UNSUPPORTED;
  if (p->batch < 1 || p->heads < 1 || p->seq_len < 1 || p->top_k < 0) return BSA_ERR_INVALID;
  if (p->batch > 65535 || p->heads > 65535) return BSA_ERR_INVALID;
  if (p->summary != BSA_SUMMARY_MEAN && p->summary != BSA_SUMMARY_REWEIGHT) return BSA_ERR_INVALID;
  if (p->anchor_rows < 0 || p->anchor_rows > p->seq_len) return BSA_ERR_INVALID;
  if (!(p->scale >= 0.f) || !isfinite(p->scale)) return BSA_ERR_INVALID;
  if (p->sink_start < 0 || p->sink_rows < 0 || (int64_t)p->sink_start + p->sink_rows > p->seq_len)
    return BSA_ERR_INVALID;
  if (p->select_mode != BSA_SELECT_TOPK && p->select_mode != BSA_SELECT_THRESHOLD) return BSA_ERR_INVALID;
  if (!isfinite(p->select_tau)) return BSA_ERR_INVALID;
  if (p->extra_tokens < 0 || p->extra_tokens > BSA_MAX_EXTRA) return BSA_ERR_INVALID;
  g->E = p->extra_tokens;
  g->threshold = p->select_mode == BSA_SELECT_THRESHOLD;
  g->tau = (double)p->select_tau;
  g->B = p->batch;
  g->H = p->heads;
  g->N = p->seq_len;
  g->nb = (g->N + BLK - 1) / BLK;
  if (g->nb > BSA_MAX_BLOCKS) return BSA_ERR_UNSUPPORTED;
  if (p->sink_rows > 0) {
    g->f0 = p->sink_start / BLK;
    g->f1 = ((int64_t)p->sink_start + p->sink_rows - 1) / BLK;
  } else {
    g->f0 = 0;
    g->f1 = -1;
  }
  const int64_t n_sink = g->f1 - g->f0 + 1, rest = g->nb - n_sink;
  g->k = n_sink + (p->top_k < rest ? p->top_k : rest);
  g->reweight = p->summary == BSA_SUMMARY_REWEIGHT;
  g->anchor_rows = p->anchor_rows == 0 ? p->seq_len : p->anchor_rows;
  g->scale = p->scale == 0.f ? 1.0 / sqrt((double)HD) : (double)p->scale;
  // the attention launch is a 1-D grid of 256-thread workgroups (at most
  // 8 ceil(nb / 8) per head), and a grid dimension counts work-items in 32 bits
  if (g->B * g->H * (8 * ((g->nb + 7) / 8)) * 256 >= (1ll << 32)) return BSA_ERR_UNSUPPORTED;
  // every per-head tensor of the attention kernel is addressed with 32-bit
  // byte offsets (buffer descriptors): N rows of 256 bytes fit for N <= 2^24
  return BSA_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// hipGetLastError reports the last failure of any runtime call on this thread,
// also one made by other code in the process before this library was called.
// Each entry point drops such an error before its launches, so the status it
// returns is that of its own launches; the name of the last failure it saw is
// kept per thread for bsa_hip_error_str.
void drop_stale_error() { (void)hipGetLastError(); }

int launch_status() {
  const hipError_t e = hipGetLastError();
  if (e == hipSuccess) return BSA_OK;
  bsa_note_hip_error(e);
  return BSA_ERR_HIP;
}

template <int NKT, int RB, bool ROWSPLIT>
int launch_select(const Geometry& g, const float* q_pool, const float* k_pool, int32_t* block_idx,
                  hipStream_t stream) {
  const dim3 grid((unsigned)(((g.nb + RB - 1) / RB) * g.H * g.B));
  const size_t lds = (size_t)RB * g.nb * sizeof(double);
  if (lds > 48 * 1024) {
    // allow the score rows of large sequences beyond the default dynamic LDS cap
    if (hipFuncSetAttribute((const void*)select_kernel<NKT, RB, ROWSPLIT>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
      return BSA_ERR_HIP;
  }
  hipLaunchKernelGGL((select_kernel<NKT, RB, ROWSPLIT>), grid, dim3(256), lds, stream, q_pool, k_pool, block_idx,
                     (int)g.nb, (int)g.k, (int)g.f0, (int)g.f1, g.threshold ? 1 : 0, g.tau);
  return launch_status();
}

template <int NCH, int NW>
int launch_select_mfma(const Geometry& g, const float* q_pool, const float* k_pool, int32_t* block_idx,
                       hipStream_t stream) {
  const dim3 grid((unsigned)(((g.nb + 15) / 16) * g.H * g.B));
  const size_t lds = (size_t)16 * g.nb * sizeof(double);
  if (lds > 48 * 1024) {
    if (hipFuncSetAttribute((const void*)select_mfma_kernel<NCH, NW>, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)lds) != hipSuccess)
      return BSA_ERR_HIP;
  }
  hipLaunchKernelGGL((select_mfma_kernel<NCH, NW>), grid, dim3(64 * NW), lds, stream, q_pool, k_pool, block_idx,
                     (int)g.nb, (int)g.k, (int)g.f0, (int)g.f1, g.threshold ? 1 : 0, g.tau);
  return launch_status();
}

template <int NCH>
int launch_select_mfma_hi(const Geometry& g, const float* q_pool, const float* k_pool, int32_t* block_idx,
                          hipStream_t stream) {
  const dim3 grid((unsigned)(((g.nb + 15) / 16) * g.H * g.B));
  const size_t lds = (size_t)16 * g.nb * sizeof(uint32_t);
  if (lds > 48 * 1024) {
    if (hipFuncSetAttribute((const void*)select_mfma_hi_kernel<NCH>, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)lds) != hipSuccess)
      return BSA_ERR_HIP;
  }
  hipLaunchKernelGGL((select_mfma_hi_kernel<NCH>), grid, dim3(512), lds, stream, q_pool, k_pool, block_idx,
                     (int)g.nb, (int)g.k, (int)g.f0, (int)g.f1);
  return launch_status();
}

// Whether a row can skip a block, i.e. the summary rows take part: top-k
// with k < nb, or threshold selection (rows keep at most k blocks).
bool uses_summaries(const Geometry& g) { return g.k < g.nb || g.threshold; }

int check_forward(const Geometry& g, const void* q, const void* k, const void* v, const void* sum_k,
                  const void* sum_v, const float* sum_bias, const int32_t* block_idx, const void* out,
                  const void* workspace, size_t workspace_bytes) {
  if (!q || !k || !v || !out) return BSA_ERR_INVALID;
  if (g.k > 0 && !block_idx) return BSA_ERR_INVALID;
  if (uses_summaries(g) && (!sum_k || !sum_v || !sum_bias)) return BSA_ERR_INVALID;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || (sum_k && !aligned16(sum_k)) ||
      (sum_v && !aligned16(sum_v)) || ((uintptr_t)sum_bias & 3u) || ((uintptr_t)block_idx & 3u))
    return BSA_ERR_INVALID;
  // the workspace is optional here (it only holds the visiting order)
  if (workspace && (workspace_bytes < forward_ws(g) || ((uintptr_t)workspace & 255u))) return BSA_ERR_WORKSPACE;
  return BSA_OK;
}

int launch_attention(const Geometry& g, const void* q, const void* k, const void* v, const void* sum_k,
                     const void* sum_v, const float* sum_bias, const int32_t* block_idx, const int32_t* tok_idx,
                     const int32_t* perm, void* out, int32_t* order_buf, hipStream_t stream) {
  // The head-synchronous map (8 chunks of ceil(nb / 8) query blocks per head)
  // once the K and V of eight heads, one per XCD, would pass 192 MiB
  // (nb > 384); below that, and with sinks, one contiguous range per XCD.
  // Measured inside whole steps: 4.9% faster at 1,045 blocks, 0.7% at 574,
  // 0.7% slower at 295 (there the XCDs' own heads still share the
  // memory-side cache, and a 37-block chunk puts two heads in each L2).
  const int chunk = (g.f1 < g.f0 && g.nb > 384) ? (int)((g.nb + 7) / 8) : 0;
  const int total = chunk > 0 ? (int)(g.B * g.H * 8 * chunk) : (int)(g.B * g.H * g.nb);
  const float scale_log2 = (float)(g.scale * 1.4426950408889634);
  // the visiting order by kept blocks, sink query blocks first; not on a
  // reblocked row order, whose neighbouring query blocks already share their
  // key blocks (there the sort measured 1.7% slower, elsewhere 1.1-2.7% faster)
  int32_t* order = nullptr;
  if (g.k > 0 && block_idx && !perm && order_buf) {
    order = order_buf;
    hipLaunchKernelGGL(row_order_kernel, dim3((unsigned)(g.B * g.H)), dim3(1024), 0, stream, block_idx, order,
                       (int)g.nb, (int)g.k, (int)g.f0, (int)g.f1);
  }
  const bool summ = uses_summaries(g);
  hipLaunchKernelGGL(attn_fwd_kernel, dim3((unsigned)total), dim3(256), 0, stream, (const uint16_t*)q,
                     (const uint16_t*)k, (const uint16_t*)v, summ ? (const uint16_t*)sum_k : nullptr,
                     summ ? (const uint16_t*)sum_v : nullptr, summ ? sum_bias : nullptr, block_idx, tok_idx, perm,
                     order, (uint16_t*)out, (int)g.N, (int)g.nb, (int)g.k, scale_log2, total, chunk, (int)g.f0,
                     (int)g.f1, tok_idx ? g.E : 0);
  return launch_status();
}

int check_pool(const Geometry& g, const void* q, const void* k, const void* v, const float* q_pool,
               const float* k_pool, const void* sum_k, const void* sum_v, const float* sum_bias,
               const void* workspace, size_t workspace_bytes) {
  if (!q || !k || !v || !q_pool || !k_pool || !sum_k || !sum_v || !sum_bias) return BSA_ERR_INVALID;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(q_pool) || !aligned16(k_pool) ||
      !aligned16(sum_k) || !aligned16(sum_v) || ((uintptr_t)sum_bias & 3u))
    return BSA_ERR_INVALID;
  if (g.reweight && (!workspace || workspace_bytes < pool_ws(g) || ((uintptr_t)workspace & 255u)))
    return BSA_ERR_WORKSPACE;
  return BSA_OK;
}

// A row order is applied to Q, K and V alike, so options that name rows by
// position (conditioning sinks, an anchor over part of the rows) are refused.
int check_reorder(const bsa_problem* p) {
  if (p->sink_rows != 0) return BSA_ERR_UNSUPPORTED;
  if (p->summary == BSA_SUMMARY_REWEIGHT && p->anchor_rows != 0 && p->anchor_rows != p->seq_len)
    return BSA_ERR_UNSUPPORTED;
  return BSA_OK;
}

template <bool REWEIGHT, bool GATHER>
void launch_pool_t(const Geometry& g, const int32_t* perm, const void* q, const void* k, const void* v,
                   float* q_pool, float* k_pool, void* sum_k, void* sum_v, float* sum_bias, void* k_out, void* v_out,
                   char* ws, hipStream_t s) {
  const dim3 grid((unsigned)g.nb, (unsigned)g.H, (unsigned)g.B);
  double* apart = REWEIGHT ? (double*)ws : nullptr;
  double* anc = REWEIGHT ? (double*)(ws + pool_anchor_off(g)) : nullptr;
  hipLaunchKernelGGL((pool_q_kernel<REWEIGHT, GATHER>), grid, dim3(256), 0, s, (const uint16_t*)q, perm, q_pool,
                     apart, (int)g.N, (int)g.nb, REWEIGHT ? g.anchor_rows : 0);
  if (REWEIGHT)
    hipLaunchKernelGGL(anchor_kernel, dim3((unsigned)g.H, (unsigned)g.B), dim3(8 * HD), 0, s,
                       (const double*)apart, anc, (int)g.nb, g.anchor_rows);
  hipLaunchKernelGGL((pool_kv_kernel<REWEIGHT, GATHER>), grid, dim3(256), 0, s, (const uint16_t*)k,
                     (const uint16_t*)v, perm, (uint16_t*)k_out, (uint16_t*)v_out, (const double*)anc, k_pool,
                     (uint16_t*)sum_k, (uint16_t*)sum_v, sum_bias, (int)g.N, (int)g.nb, g.scale);
}

int launch_pool(const Geometry& g, const int32_t* perm, const void* q, const void* k, const void* v,
                float* q_pool, float* k_pool, void* sum_k, void* sum_v, float* sum_bias, void* k_out, void* v_out,
                char* ws, hipStream_t s) {
  if (g.reweight) {
    if (perm)
      launch_pool_t<true, true>(g, perm, q, k, v, q_pool, k_pool, sum_k, sum_v, sum_bias, k_out, v_out, ws, s);
    else
      launch_pool_t<true, false>(g, perm, q, k, v, q_pool, k_pool, sum_k, sum_v, sum_bias, k_out, v_out, ws, s);
  } else {
    if (perm)
      launch_pool_t<false, true>(g, perm, q, k, v, q_pool, k_pool, sum_k, sum_v, sum_bias, k_out, v_out, ws, s);
    else
      launch_pool_t<false, false>(g, perm, q, k, v, q_pool, k_pool, sum_k, sum_v, sum_bias, k_out, v_out, ws, s);
  }
  return launch_status();
}

// Scratch of bsa_forward_noalloc: the visiting order (int32 per (b, h, query
// block)) in a file-scope device array instead of a workspace argument.  In
// host code `scratch` only names the symbol; its device address, one per GPU,
// comes from hipGetSymbolAddress on the first call on that device.
constexpr size_t NOALLOC_ORDER_MAX = (size_t)1 << 20;  // entries: 4 MiB
__device__ __align__(256) int32_t scratch[NOALLOC_ORDER_MAX];

constexpr int NOALLOC_MAX_DEVICES = 64;
std::mutex scratch_mutex;
int32_t* scratch_ptr[NOALLOC_MAX_DEVICES] = {};

// Device address of this GPU's scratch array (looked up once per device, with
// that device current), or nullptr on failure.
int32_t* device_scratch() {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    bsa_note_hip_error(e);
    return nullptr;
  }
  if (dev < 0 || dev >= NOALLOC_MAX_DEVICES) {
    bsa_note_hip_error(hipErrorInvalidDevice);
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(scratch_mutex);
  if (!scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) {
      bsa_note_hip_error(e != hipSuccess ? e : hipErrorInvalidSymbol);
      return nullptr;
    }
    scratch_ptr[dev] = (int32_t*)ptr;
  }
  return scratch_ptr[dev];
}

}  // namespace

extern "C" {

const char* bsa_status_str(int status) {
  switch (status) {
    case BSA_OK: return "ok";
    case BSA_ERR_INVALID: return "invalid argument";
    case BSA_ERR_UNSUPPORTED: return "unsupported problem (head_dim/block must be 128, nb <= 2048)";
    case BSA_ERR_WORKSPACE: return "workspace missing or too small";
    case BSA_ERR_HIP: return "HIP launch failed (bsa_hip_error_str names the runtime's error)";
    case BSA_ERR_SCRATCH:
      return "problem too large for the static scratch of bsa_forward_noalloc (B*H*nb > 1048576)";
    default: return "unknown status";
  }
}

const char* bsa_hip_error_str(void) {
  return last_hip_error == hipSuccess ? "none" : hipGetErrorName(last_hip_error);
}

int bsa_problem_blocks(const bsa_problem* p, int32_t* n_blocks, int32_t* k_eff) {
  Geometry g;
  const int st = make_geometry(p, &g);
  if (st != BSA_OK) return st;
  if (n_blocks) *n_blocks = (int32_t)g.nb;
  if (k_eff) *k_eff = (int32_t)g.k;
  return BSA_OK;
}

size_t bsa_workspace_bytes(const bsa_problem* p) {
  Geometry g;
  if (make_geometry(p, &g) != BSA_OK) return 0;
  return ws_total(g);
}

int bsa_pool(const bsa_problem* p, const void* q, const void* k, const void* v, float* q_pool,
             float* k_pool, void* sum_k, void* sum_v, float* sum_bias, void* workspace,
             size_t workspace_bytes, void* hip_stream) {
  Geometry g;
  int st = make_geometry(p, &g);
  if (st != BSA_OK) return st;
  if ((st = check_pool(g, q, k, v, q_pool, k_pool, sum_k, sum_v, sum_bias, workspace, workspace_bytes)) != BSA_OK)
    return st;
  drop_stale_error();
  return launch_pool(g, nullptr, q, k, v, q_pool, k_pool, sum_k, sum_v, sum_bias, nullptr, nullptr,
                     (char*)workspace, (hipStream_t)hip_stream);
}

int bsa_pool_reordered(const bsa_problem* p, const int32_t* perm, const void* q, const void* k, const void* v,
                       float* q_pool, float* k_pool, void* sum_k, void* sum_v, float* sum_bias, void* k_out,
                       void* v_out, void* workspace, size_t workspace_bytes, void* hip_stream) {
  Geometry g;
  int st = make_geometry(p, &g);
  if (st != BSA_OK) return st;
  if ((st = check_reorder(p)) != BSA_OK) return st;
  if (!perm || ((uintptr_t)perm & 3u) || !k_out || !v_out || !aligned16(k_out) || !aligned16(v_out))
    return BSA_ERR_INVALID;
  if (k_out == v_out || k_out == q || k_out == k || k_out == v || v_out == q || v_out == k || v_out == v)
    return BSA_ERR_INVALID;
  if ((st = check_pool(g, q, k, v, q_pool, k_pool, sum_k, sum_v, sum_bias, workspace, workspace_bytes)) != BSA_OK)
    return st;
  drop_stale_error();
  return launch_pool(g, perm, q, k, v, q_pool, k_pool, sum_k, sum_v, sum_bias, k_out, v_out, (char*)workspace,
                     (hipStream_t)hip_stream);
}

int bsa_select(const bsa_problem* p, const float* q_pool, const float* k_pool, int32_t* block_idx,
               void* hip_stream) {
  Geometry g;
  int st = make_geometry(p, &g);
  if (st != BSA_OK) return st;
  if (g.k == 0) return BSA_OK;
  if (!q_pool || !k_pool || !block_idx) return BSA_ERR_INVALID;
  if (!aligned16(q_pool) || !aligned16(k_pool) || ((uintptr_t)block_idx & 3u)) return BSA_ERR_INVALID;
  drop_stale_error();
  hipStream_t s = (hipStream_t)hip_stream;
  // key blocks per lane (top-k phase) sized to nb.  Scores on the float64
  // matrix cores while 16 score rows fit the LDS (nb <= 1200); past that the
  // row-split VALU score phase (four query rows in registers, whole-line key
  // loads).  Top-k keeps only the high halves of the keys in LDS (two
  // workgroups of 8 wavefronts a CU, one scoring while the other ranks).  The
  // threshold mode needs the float64 rows for its mean and deviation: up to
  // 512 blocks four workgroups of 4 wavefronts share a CU, past that one
  // workgroup of 16 wavefronts keeps the CU busy (2K 5s: 0.64 ms against
  // 0.92 with 4)
  if (!g.threshold) {
    if (g.nb <= 256) return launch_select_mfma_hi<4>(g, q_pool, k_pool, block_idx, s);
    if (g.nb <= 512) return launch_select_mfma_hi<8>(g, q_pool, k_pool, block_idx, s);
    if (g.nb <= 1024) return launch_select_mfma_hi<16>(g, q_pool, k_pool, block_idx, s);
    if (g.nb <= 1280) return launch_select_mfma_hi<20>(g, q_pool, k_pool, block_idx, s);
  }
  if (g.nb <= 256) return launch_select_mfma<4, 4>(g, q_pool, k_pool, block_idx, s);
  if (g.nb <= 512) return launch_select_mfma<8, 4>(g, q_pool, k_pool, block_idx, s);
  if (g.nb <= 1024) return launch_select_mfma<16, 16>(g, q_pool, k_pool, block_idx, s);
  if (g.nb <= 1200) return launch_select_mfma<19, 16>(g, q_pool, k_pool, block_idx, s);
  return launch_select<8, 4, true>(g, q_pool, k_pool, block_idx, s);
}

int bsa_forward(const bsa_problem* p, const void* q, const void* k, const void* v, const void* sum_k,
                const void* sum_v, const float* sum_bias, const int32_t* block_idx, void* out, void* workspace,
                size_t workspace_bytes, void* hip_stream) {
  Geometry g;
  int st = make_geometry(p, &g);
  if (st != BSA_OK) return st;
  if (g.E > 0) return BSA_ERR_INVALID;  // extra tokens go through bsa_forward_tokens
  if ((st = check_forward(g, q, k, v, sum_k, sum_v, sum_bias, block_idx, out, workspace, workspace_bytes)) !=
      BSA_OK)
    return st;
  drop_stale_error();
  return launch_attention(g, q, k, v, sum_k, sum_v, sum_bias, block_idx, nullptr, nullptr, out,
                          (int32_t*)workspace, (hipStream_t)hip_stream);
}

int bsa_forward_noalloc(const bsa_problem* p, const void* q, const void* k, const void* v, const void* sum_k,
                        const void* sum_v, const float* sum_bias, const int32_t* block_idx, void* out,
                        void* hip_stream) {
  Geometry g;
  int st = make_geometry(p, &g);
  if (st != BSA_OK) return st;
  if (g.E > 0) return BSA_ERR_INVALID;
  if ((st = check_forward(g, q, k, v, sum_k, sum_v, sum_bias, block_idx, out, nullptr, 0)) != BSA_OK) return st;
  if ((size_t)(g.B * g.H * g.nb) > NOALLOC_ORDER_MAX) return BSA_ERR_SCRATCH;
  drop_stale_error();
  int32_t* order = device_scratch();
  if (!order) return BSA_ERR_HIP;
  return launch_attention(g, q, k, v, sum_k, sum_v, sum_bias, block_idx, nullptr, nullptr, out, order,
                          (hipStream_t)hip_stream);
}

int bsa_select_tokens(const bsa_problem* p, const float* q_pool, const void* k,
                      const int32_t* block_idx, int32_t* token_idx, void* workspace,
                      size_t workspace_bytes, void* hip_stream) {
  Geometry g;
  const int st = make_geometry(p, &g);
  if (st != BSA_OK) return st;
  if (g.E == 0) return BSA_OK;
  if (!q_pool || !k || !token_idx || (g.k > 0 && !block_idx)) return BSA_ERR_INVALID;
  if (!aligned16(q_pool) || !aligned16(k) || ((uintptr_t)token_idx & 3u) || ((uintptr_t)block_idx & 3u))
    return BSA_ERR_INVALID;
  if (!workspace || workspace_bytes < tokens_ws(g) || ((uintptr_t)workspace & 255u)) return BSA_ERR_WORKSPACE;
  // sample size of the first phase: T_m lands near the 2E- to 3E-th score,
  // with a margin for samples that are not random (small E: no sample)
  auto sample_m = [&](double S) { return g.E >= 64 ? std::min(g.E, (int)ceil(g.E / S + 8.0 * sqrt(g.E / S))) : 0; };
  const int G = (int)(((g.nb + TS_ROWS - 1) / TS_ROWS) * g.H * g.B);
  int n_whole, parts;
  token_split(g, &n_whole, &parts);
  const int tail = G - n_whole;
  const size_t prow = (size_t)tail * parts * TS_ROWS;
  char* ws = (char*)workspace;
  uint64_t* pseg = (uint64_t*)(ws + tokens_seg_bytes(g));
  uint64_t* plist = (uint64_t*)((char*)pseg + align256(prow * TS_SEGS * SEG_CAP * sizeof(uint64_t)));
  int32_t* pcount = (int32_t*)((char*)plist + align256(prow * g.E * sizeof(uint64_t)));
  drop_stale_error();
  hipLaunchKernelGGL(token_select_kernel, dim3((unsigned)(n_whole + tail * parts)), dim3(TS_THREADS), 0,
                     (hipStream_t)hip_stream, q_pool, (const uint16_t*)k, g.k > 0 ? block_idx : nullptr, token_idx,
                     (uint64_t*)workspace, pseg, plist, pcount, (int)g.N, (int)g.nb, (int)g.k, g.E,
                     sample_m(TS_STRIDE), sample_m(TS_STRIDE_PART), (int)g.f0, (int)g.f1, n_whole, parts);
  if (parts > 1) {
    const int rows = tail * TS_ROWS;
    hipLaunchKernelGGL(token_merge_kernel, dim3((unsigned)((rows + 7) / 8)), dim3(512), 0, (hipStream_t)hip_stream,
                       plist, pcount, token_idx, (int)g.nb, g.E, n_whole, parts, rows);
  }
  return launch_status();
}

int bsa_forward_tokens(const bsa_problem* p, const void* q, const void* k, const void* v, const void* sum_k,
                       const void* sum_v, const float* sum_bias, const int32_t* block_idx,
                       const int32_t* token_idx, void* out, void* workspace, size_t workspace_bytes,
                       void* hip_stream) {
  Geometry g;
  int st = make_geometry(p, &g);
  if (st != BSA_OK) return st;
  if ((st = check_forward(g, q, k, v, sum_k, sum_v, sum_bias, block_idx, out, workspace, workspace_bytes)) !=
      BSA_OK)
    return st;
  if (g.E > 0 && (!token_idx || ((uintptr_t)token_idx & 3u))) return BSA_ERR_INVALID;
  drop_stale_error();
  return launch_attention(g, q, k, v, sum_k, sum_v, sum_bias, block_idx, g.E > 0 ? token_idx : nullptr, nullptr,
                          out, (int32_t*)workspace, (hipStream_t)hip_stream);
}

int bsa_forward_reordered(const bsa_problem* p, const int32_t* perm, const void* q, const void* k_r,
                          const void* v_r, const void* sum_k, const void* sum_v, const float* sum_bias,
                          const int32_t* block_idx, const int32_t* token_idx, void* out, void* workspace,
                          size_t workspace_bytes, void* hip_stream) {
  Geometry g;
  int st = make_geometry(p, &g);
  if (st != BSA_OK) return st;
  if ((st = check_reorder(p)) != BSA_OK) return st;
  if (!perm || ((uintptr_t)perm & 3u)) return BSA_ERR_INVALID;
  if ((st = check_forward(g, q, k_r, v_r, sum_k, sum_v, sum_bias, block_idx, out, workspace, workspace_bytes)) !=
      BSA_OK)
    return st;
  if (out == q || out == k_r || out == v_r) return BSA_ERR_INVALID;
  if (g.E > 0 && (!token_idx || ((uintptr_t)token_idx & 3u))) return BSA_ERR_INVALID;
  drop_stale_error();
  return launch_attention(g, q, k_r, v_r, sum_k, sum_v, sum_bias, block_idx, g.E > 0 ? token_idx : nullptr, perm,
                          out, nullptr, (hipStream_t)hip_stream);
}

}  // extern "C"
