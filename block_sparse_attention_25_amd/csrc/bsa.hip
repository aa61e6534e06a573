// Block-sparse self-attention with summary rows, written for gfx950 (MI355X).
//
// Kernels (all launched by the extern "C" entry points at the bottom):
//   pool_q_kernel     block means of Q (float64 sums -> float32); in reweight
//                     mode also per-block float64 partial sums of the anchor rows
//   anchor_kernel     reweight only: per-head anchor = mean of the anchor rows
//   pool_kv_kernel    block means of K (for scoring), summary key/value rows and
//                     bias (mean or Spark-Reweight), V of every block transposed
//                     into the workspace, summary values transposed likewise
//   select_kernel     float64 block scores and a wavefront top-k with
//                     lowest-index ties, ascending output
//   attn_fwd_kernel   fused gather attention: bf16 MFMA 32x32x16, K and V^T
//                     tiles staged in LDS, one online softmax over the selected
//                     blocks and the summary rows
//
// Sources: "h3-sparse-attn 0.1.0" (PyPI page), opening paragraph and "Use";
// "Spark-H3: Block Sparse Attention Speeds Up MiniMax-H3 in ComfyUI",
// "What Spark-Attn changes".
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "bsa.h"

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

// Column order of V^T inside each 16-key group.  The P operand of the PV
// product comes straight from the S^T accumulator, whose lane holds keys
// {8a + 4g + e : a in 0..1, e in 0..3} of every 16-key slice (g = lane / 32).
// Storing key j at position swap(bits 2, 3 of j) makes those 8 keys contiguous,
// so the V^T operand is one 16-byte LDS read.  The map is its own inverse.
__host__ __device__ __forceinline__ int vt_pos(int j) {
  return (j & ~12) | ((j & 4) << 1) | ((j & 8) >> 1);
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

template <bool REWEIGHT>
__global__ __launch_bounds__(256) void pool_q_kernel(const uint16_t* __restrict__ q,
                                                     float* __restrict__ q_pool,
                                                     double* __restrict__ anchor_part, int N,
                                                     int nb, int anchor_rows) {
  __shared__ double red[16][HD];
  const int c = blockIdx.x, tid = threadIdx.x;
  const size_t bh = (size_t)blockIdx.z * gridDim.y + blockIdx.y;
  const int s = c * BLK, n = min(BLK, N - s);
  const uint16_t* xb = q + (bh * N + s) * HD;
  const int cc = tid & 15, rp = tid >> 4;
  double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0}, acc_a[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = rp + 16 * i;
    if (row < n) {
      double vals[8];
      unpack8(*(const uint4*)(xb + row * HD + cc * 8), vals);
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

// anchor[b,h,:] = (sum over blocks of the partial sums, in block order) / rows
__global__ __launch_bounds__(128) void anchor_kernel(const double* __restrict__ anchor_part,
                                                     double* __restrict__ anchor, int nb,
                                                     int anchor_rows) {
  const size_t bh = (size_t)blockIdx.y * gridDim.x + blockIdx.x;
  const int d = threadIdx.x;
  const int nblk = (anchor_rows + BLK - 1) / BLK;
  double s = 0.0;
  for (int c = 0; c < nblk; ++c) s += anchor_part[(bh * nb + c) * HD + d];
  anchor[bh * HD + d] = s / (double)anchor_rows;
}

template <bool REWEIGHT>
__global__ __launch_bounds__(256) void pool_kv_kernel(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, const double* __restrict__ anchor,
    float* __restrict__ k_pool, uint16_t* __restrict__ sum_k, uint16_t* __restrict__ sum_v,
    float* __restrict__ sum_bias, uint16_t* __restrict__ vt, uint16_t* __restrict__ svt, int N,
    int nb, int nsb, double scale) {
  __shared__ double red[16][HD];
  __shared__ uint16_t vl[BLK][HD + 2];  // V block, rows padded against bank conflicts
  __shared__ double rowred[16][3];
  const int c = blockIdx.x, tid = threadIdx.x;
  const size_t bh = (size_t)blockIdx.z * gridDim.y + blockIdx.y;
  const int s = c * BLK, n = min(BLK, N - s);
  const uint16_t* kb = k + (bh * N + s) * HD;
  const uint16_t* vb = v + (bh * N + s) * HD;
  const int cc = tid & 15, rp = tid >> 4;

  uint4 kr[8], vr[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = rp + 16 * i;
    // load a valid row (clamped) and zero it afterwards: no pointer select
    const int rowc = min(row, n - 1);
    kr[i] = zero_unless(*(const uint4*)(kb + rowc * HD + cc * 8), row < n);
    vr[i] = zero_unless(*(const uint4*)(vb + rowc * HD + cc * 8), row < n);
    // stage V (zeros past the end of a short block) for the transpose below
    uint32_t* dst = (uint32_t*)&vl[row][cc * 8];
    dst[0] = vr[i].x; dst[1] = vr[i].y; dst[2] = vr[i].z; dst[3] = vr[i].w;
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
    if (cc == 0) rowred[rp][0] = lmax;
    __syncthreads();
    double m = rowred[0][0];
#pragma unroll
    for (int i = 1; i < 16; ++i) m = fmax(m, rowred[i][0]);
    __syncthreads();
    double w[8], zpart = 0.0, lsum = 0.0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const bool ok = rp + 16 * i < n;
      w[i] = ok ? exp(l[i] - m) : 0.0;
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
    const uint16_t svb = f2bf((float)sv_out);
    sum_v[(bh * nb + c) * HD + tid] = svb;
    // summary values transposed, groups of 128 blocks: svt[bh][c/128][d][pos]
    uint16_t* sg = svt + ((bh * nsb + c / BLK) * HD + tid) * BLK;
    sg[vt_pos(c % BLK)] = svb;
    if (c == nb - 1)
      for (int cp = nb; cp < nsb * BLK; ++cp) sg[vt_pos(cp % BLK) + 0] = 0;
  }
  if (tid == 0) sum_bias[bh * nb + c] = (float)bias_out;
  __syncthreads();

  // V^T of this block: vt[bh][c][d][vt_pos(j)] = V[s + j][d]; 16-byte stores,
  // 16 threads per 256-byte output row.
  uint16_t* vto = vt + (bh * nb + c) * (size_t)(BLK * HD);
#pragma unroll
  for (int it = 0; it < 8; ++it) {
    const int id = it * 256 + tid;
    const int d = id >> 4, pc = id & 15;
    uint32_t wv[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int j0 = vt_pos(pc * 8 + 2 * e), j1 = vt_pos(pc * 8 + 2 * e + 1);
      wv[e] = (uint32_t)vl[j0][d] | ((uint32_t)vl[j1][d] << 16);
    }
    *(uint4*)(vto + d * BLK + pc * 8) = make_uint4(wv[0], wv[1], wv[2], wv[3]);
  }
}

// ---------------------------------------------------------------- select ---
// One workgroup of 4 wavefronts per 4 query blocks of one (b, h).  Scores of
// the 4 rows against all nb key blocks go to LDS in float64; then each
// wavefront selects the top k of one row on order-preserving 64-bit keys with
// an MSB-first bitwise search for the k-th largest key, and writes the chosen
// indices in ascending order (ballot prefix counts).
constexpr int SEL_RB = 4;
constexpr int SEL_MAXPL = BSA_MAX_BLOCKS / 64;

__device__ __forceinline__ uint64_t order_key(double s) {
  if (s == 0.0) s = 0.0;  // -0 ties with +0
  const uint64_t u = (uint64_t)__double_as_longlong(s);
  return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}

__global__ __launch_bounds__(256) void select_kernel(const float* __restrict__ q_pool,
                                                     const float* __restrict__ k_pool,
                                                     int32_t* __restrict__ block_idx, int nb,
                                                     int ksel) {
  extern __shared__ double sc[];  // [SEL_RB][nb]
  __shared__ double qs[SEL_RB][HD];
  __shared__ float kT[HD][65];
  const int tid = threadIdx.x;
  const int r0 = blockIdx.x * SEL_RB;
  const size_t bh = (size_t)blockIdx.z * gridDim.y + blockIdx.y;
  const float* qpb = q_pool + bh * nb * HD;
  const float* kpb = k_pool + bh * nb * HD;
  for (int i = tid; i < SEL_RB * HD; i += 256) {
    const int r = i / HD, d = i % HD;
    qs[r][d] = (r0 + r < nb) ? (double)qpb[(size_t)(r0 + r) * HD + d] : 0.0;
  }
  for (int c0 = 0; c0 < nb; c0 += 64) {
    __syncthreads();
    for (int i = tid; i < 64 * 32; i += 256) {
      const int c = i >> 5, d4 = i & 31;
      float4 val = make_float4(0.f, 0.f, 0.f, 0.f);
      if (c0 + c < nb) val = *(const float4*)(kpb + (size_t)(c0 + c) * HD + 4 * d4);
      kT[4 * d4 + 0][c] = val.x;
      kT[4 * d4 + 1][c] = val.y;
      kT[4 * d4 + 2][c] = val.z;
      kT[4 * d4 + 3][c] = val.w;
    }
    __syncthreads();
    const int c = tid & 63, r = tid >> 6;
    double a0 = 0.0, a1 = 0.0, a2 = 0.0, a3 = 0.0;
#pragma unroll 8
    for (int d = 0; d < HD; d += 4) {
      a0 = fma(qs[r][d + 0], (double)kT[d + 0][c], a0);
      a1 = fma(qs[r][d + 1], (double)kT[d + 1][c], a1);
      a2 = fma(qs[r][d + 2], (double)kT[d + 2][c], a2);
      a3 = fma(qs[r][d + 3], (double)kT[d + 3][c], a3);
    }
    if (c0 + c < nb) sc[r * nb + c0 + c] = (a0 + a1) + (a2 + a3);
  }
  __syncthreads();

  const int w = tid >> 6, lane = tid & 63;
  const int r = r0 + w;
  if (r >= nb || ksel == 0) return;
  const double* srow = sc + w * nb;
  uint64_t key[SEL_MAXPL];
#pragma unroll
  for (int i = 0; i < SEL_MAXPL; ++i) {
    const int c = i * 64 + lane;
    key[i] = (c < nb) ? order_key(srow[c]) : 0ull;  // real keys are > 0
  }
  // T = largest value with #{key >= T} >= ksel, i.e. the ksel-th largest key
  uint64_t T = 0;
  for (int bit = 63; bit >= 0; --bit) {
    const uint64_t cand = T | (1ull << bit);
    int cnt = 0;
#pragma unroll
    for (int i = 0; i < SEL_MAXPL; ++i)
      if (i * 64 < nb) cnt += __popcll(__ballot(key[i] >= cand));
    if (cnt >= ksel) T = cand;
  }
  int gt = 0;
#pragma unroll
  for (int i = 0; i < SEL_MAXPL; ++i)
    if (i * 64 < nb) gt += __popcll(__ballot(key[i] > T));
  const int need_eq = ksel - gt;  // keys equal to T taken lowest index first
  const uint64_t lt = (1ull << lane) - 1ull;
  int eq_before = 0, sel_before = 0;
  int32_t* orow = block_idx + (bh * nb + r) * (size_t)ksel;
#pragma unroll
  for (int i = 0; i < SEL_MAXPL; ++i) {
    if (i * 64 >= nb) break;
    const bool is_eq = key[i] == T, is_gt = key[i] > T;
    const uint64_t em = __ballot(is_eq);
    const int erank = eq_before + __popcll(em & lt);
    const bool sel = is_gt || (is_eq && erank < need_eq);
    const uint64_t sm = __ballot(sel);
    if (sel) orow[sel_before + __popcll(sm & lt)] = i * 64 + lane;
    eq_before += __popcll(em);
    sel_before += __popcll(sm);
  }
}

// ------------------------------------------------------------- attention ---
// One workgroup (4 wavefronts) per (b, h, query block r), 128 query rows;
// wavefront w owns queries [32w, 32w + 32) of the block.  Per key tile (a
// selected block, or 128 summary rows) the workgroup stages K (rows) and V^T
// (feature rows) in LDS, XOR-swizzled by 16-byte chunk, then each wavefront
// computes S^T = K Q^T (4 x 8 MFMA 32x32x16), updates its online softmax in
// base 2, and accumulates O^T += V^T P^T (4 x 8 MFMA) with P taken directly
// from the S^T accumulator.  Lane l holds query 32w + l%32; lanes l and l^32
// hold the two halves of that query's keys.

__device__ __forceinline__ int swz(int row, int chunk) { return row * HD + ((chunk ^ (row & 15)) << 3); }

__device__ __forceinline__ bf16x8 ld_bf16x8(const uint16_t* p) { return *(const bf16x8*)p; }

__device__ __forceinline__ int xcd_remap(int hw, int total) {
  // workgroups are dealt to the 8 XCDs round-robin; give each XCD a contiguous
  // range of (head, query block) so neighbouring query blocks share its L2
  const int per = total / 8, rem = total % 8;
  const int x = hw & 7, j = hw >> 3;
  return (x < rem) ? x * (per + 1) + j : rem * (per + 1) + (x - rem) * per + j;
}

__global__ __launch_bounds__(256, 2) void attn_fwd_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ vt, const uint16_t* __restrict__ sum_k,
    const uint16_t* __restrict__ svt, const float* __restrict__ sum_bias,
    const int32_t* __restrict__ block_idx, uint16_t* __restrict__ out, int N, int nb, int ksel,
    int nsb, float scale_log2, int total_wg) {
  __shared__ __attribute__((aligned(16))) uint16_t ks[BLK * HD];
  __shared__ __attribute__((aligned(16))) uint16_t vs[HD * BLK];
  __shared__ float addv[BLK];
  __shared__ uint32_t selmask[BSA_MAX_BLOCKS / 32];

  const int logical = xcd_remap(blockIdx.x, total_wg);
  const int r = logical % nb;
  const size_t bh = (size_t)(logical / nb);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, ln = lane & 31;

  const uint16_t* kb = k + bh * (size_t)N * HD;
  const uint16_t* vtb = vt + bh * (size_t)nb * BLK * HD;
  const uint16_t* skb = sum_k ? sum_k + bh * (size_t)nb * HD : nullptr;
  const uint16_t* svtb = svt + bh * (size_t)nsb * BLK * HD;
  const float* biasb = sum_bias ? sum_bias + bh * (size_t)nb : nullptr;
  const int32_t* irow = block_idx + (bh * nb + r) * (size_t)ksel;

  // Q fragments (B operand of S^T = K Q^T): query qi, features 16kk + 8g + [0, 8)
  const int qi = r * BLK + 32 * wave + ln;
  bf16x8 qf[8];
  {
    const uint16_t* qrow = q + (bh * (size_t)N + (size_t)min(qi, N - 1)) * HD;
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
  for (int i = tid; i < ksel; i += 256) {
    const int c = irow[i];
    atomicOr(&selmask[c >> 5], 1u << (c & 31));
  }
  __syncthreads();

  f32x16 o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) o[db] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  const int ntiles = ksel + ((ksel < nb) ? nsb : 0);
  for (int t = 0; t < ntiles; ++t) {
    const bool summary = t >= ksel;
    const uint16_t* ksrc;
    const uint16_t* vsrc;
    int nvalid, st = 0;
    if (!summary) {
      const int c = irow[t];
      ksrc = kb + (size_t)c * BLK * HD;
      vsrc = vtb + (size_t)c * BLK * HD;
      nvalid = min(BLK, N - c * BLK);
    } else {
      st = t - ksel;
      nvalid = min(BLK, nb - st * BLK);
      int nsel = 0;
#pragma unroll
      for (int wd = 0; wd < 4; ++wd) {
        const int word = st * 4 + wd;
        if (word < nwords) nsel += __popc(selmask[word]);
      }
      if (nsel == nvalid) continue;  // every block of this group is exact
      ksrc = skb + (size_t)st * BLK * HD;
      vsrc = svtb + (size_t)st * BLK * HD;
    }
    const bool need_add = summary || nvalid < BLK;

    __syncthreads();  // previous tile fully consumed
    {
      uint4 kv[8], vv[8];
#pragma unroll
      for (int it = 0; it < 8; ++it) {
        const int id = it * 256 + tid;
        const int row = id >> 4, ch = id & 15;
        kv[it] = zero_unless(*(const uint4*)(ksrc + min(row, nvalid - 1) * HD + ch * 8), row < nvalid);
        vv[it] = *(const uint4*)(vsrc + row * BLK + ch * 8);
      }
#pragma unroll
      for (int it = 0; it < 8; ++it) {
        const int id = it * 256 + tid;
        const int row = id >> 4, ch = id & 15;
        *(uint4*)(ks + swz(row, ch)) = kv[it];
        *(uint4*)(vs + swz(row, ch)) = vv[it];
      }
      if (need_add && tid < BLK) {
        float a;
        if (!summary) {
          a = tid < nvalid ? 0.f : -INFINITY;
        } else {
          const int c = st * BLK + tid;
          const bool skipped = c < nb && !((selmask[c >> 5] >> (c & 31)) & 1u);
          a = skipped ? biasb[c] * LOG2E : -INFINITY;
        }
        addv[tid] = a;
      }
    }
    __syncthreads();

    // S^T = K Q^T : s[mb] holds keys 32mb + 8(i/4) + 4g + i%4, query ln
    f32x16 s[4];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      s[mb] = f32x16{};
      const int row = 32 * mb + ln;
#pragma unroll
      for (int kk = 0; kk < 8; ++kk)
        s[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ld_bf16x8(ks + swz(row, 2 * kk + g)),
                                                         qf[kk], s[mb], 0, 0, 0);
    }

    // online softmax (base 2)
    float mx = -INFINITY;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float x = s[mb][i] * scale_log2;
        if (need_add) x += addv[32 * mb + 8 * (i >> 2) + 4 * g + (i & 3)];
        s[mb][i] = x;
        mx = fmaxf(mx, x);
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    float psum = 0.f;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = __builtin_amdgcn_exp2f(s[mb][i] - m_use);
        s[mb][i] = p;
        psum += p;
      }
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int db = 0; db < 4; ++db) o[db] *= alpha;

    // O^T += V^T P^T
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const f32x16& sv = s[kk >> 1];
      const int base = 8 * (kk & 1);
      f32x8 pf = {sv[base + 0], sv[base + 1], sv[base + 2], sv[base + 3],
                  sv[base + 4], sv[base + 5], sv[base + 6], sv[base + 7]};
      const bf16x8 pb = __builtin_convertvector(pf, bf16x8);
#pragma unroll
      for (int db = 0; db < 4; ++db)
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ld_bf16x8(vs + swz(32 * db + ln, 2 * kk + g)),
                                                         pb, o[db], 0, 0, 0);
    }
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = 1.f / l_tot;
  if (qi < N) {
    uint16_t* orow = out + (bh * (size_t)N + qi) * HD;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d0 = 32 * db + 8 * r4 + 4 * g;
        const uint32_t w0 = (uint32_t)f2bf(o[db][4 * r4 + 0] * inv) |
                            ((uint32_t)f2bf(o[db][4 * r4 + 1] * inv) << 16);
        const uint32_t w1 = (uint32_t)f2bf(o[db][4 * r4 + 2] * inv) |
                            ((uint32_t)f2bf(o[db][4 * r4 + 3] * inv) << 16);
        *(uint2*)(orow + d0) = make_uint2(w0, w1);
      }
    }
  }
}

// ------------------------------------------------------------------ host ---
struct Geometry {
  int64_t B, H, N, nb, nsb, k;
  bool reweight;
  int anchor_rows;
  double scale;
};

struct WsLayout {
  size_t vt, svt, apart, anchor, total;
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

int make_geometry(const bsa_problem* p, Geometry* g) {
  if (!p) return BSA_ERR_INVALID;
  if (p->head_dim != BSA_HEAD_DIM || p->block_size != BSA_BLOCK) return BSA_ERR_UNSUPPORTED;
  if (p->batch < 1 || p->heads < 1 || p->seq_len < 1 || p->top_k < 0) return BSA_ERR_INVALID;
  if (p->batch > 65535 || p->heads > 65535) return BSA_ERR_INVALID;
  if (p->summary != BSA_SUMMARY_MEAN && p->summary != BSA_SUMMARY_REWEIGHT) return BSA_ERR_INVALID;
  if (p->anchor_rows < 0 || p->anchor_rows > p->seq_len) return BSA_ERR_INVALID;
  if (!(p->scale >= 0.f) || !isfinite(p->scale)) return BSA_ERR_INVALID;
  g->B = p->batch;
  g->H = p->heads;
  g->N = p->seq_len;
  g->nb = (g->N + BLK - 1) / BLK;
  if (g->nb > BSA_MAX_BLOCKS) return BSA_ERR_UNSUPPORTED;
  g->nsb = (g->nb + BLK - 1) / BLK;
  g->k = p->top_k < g->nb ? p->top_k : g->nb;
  g->reweight = p->summary == BSA_SUMMARY_REWEIGHT;
  g->anchor_rows = p->anchor_rows == 0 ? p->seq_len : p->anchor_rows;
  g->scale = p->scale == 0.f ? 1.0 / sqrt((double)HD) : (double)p->scale;
  // the attention launch is a 1-D grid of 256-thread workgroups, and a grid
  // dimension counts work-items in 32 bits
  if (g->B * g->H * g->nb * 256 >= (1ll << 32)) return BSA_ERR_UNSUPPORTED;
  return BSA_OK;
}

WsLayout ws_layout(const Geometry& g) {
  WsLayout w{};
  const size_t bh = (size_t)(g.B * g.H);
  w.vt = 0;
  size_t off = align256(bh * g.nb * BLK * HD * 2);
  w.svt = off;
  off = align256(off + bh * g.nsb * BLK * HD * 2);
  if (g.reweight) {
    w.apart = off;
    off = align256(off + bh * g.nb * HD * sizeof(double));
    w.anchor = off;
    off = align256(off + bh * HD * sizeof(double));
  }
  w.total = off;
  return w;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int launch_status() { return hipGetLastError() == hipSuccess ? BSA_OK : BSA_ERR_HIP; }

}  // namespace

extern "C" {

const char* bsa_status_str(int status) {
  switch (status) {
    case BSA_OK: return "ok";
    case BSA_ERR_INVALID: return "invalid argument";
    case BSA_ERR_UNSUPPORTED: return "unsupported problem (head_dim/block must be 128, nb <= 2048)";
    case BSA_ERR_WORKSPACE: return "workspace missing or too small";
    case BSA_ERR_HIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

int bsa_problem_blocks(const bsa_problem* p, int32_t* n_blocks, int32_t* k_eff) {
  Geometry g;
  const int st = make_geometry(p, &g);
  if (st != BSA_OK) return st;
  if (n_blocks) *n_blocks = (int32_t)g.nb;
  if (k_eff) *k_eff = (int32_t)g.k;
  return BSA_OK;
}

int bsa_workspace_bytes(const bsa_problem* p, size_t* bytes) {
  Geometry g;
  const int st = make_geometry(p, &g);
  if (st != BSA_OK) return st;
  if (!bytes) return BSA_ERR_INVALID;
  *bytes = ws_layout(g).total;
  return BSA_OK;
}

int bsa_pool(const bsa_problem* p, const void* q, const void* k, const void* v, float* q_pool,
             float* k_pool, void* sum_k, void* sum_v, float* sum_bias, void* workspace,
             size_t workspace_bytes, void* hip_stream) {
  Geometry g;
  int st = make_geometry(p, &g);
  if (st != BSA_OK) return st;
  if (!q || !k || !v || !q_pool || !k_pool || !sum_k || !sum_v || !sum_bias) return BSA_ERR_INVALID;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(q_pool) || !aligned16(k_pool) ||
      !aligned16(sum_k) || !aligned16(sum_v))
    return BSA_ERR_INVALID;
  const WsLayout w = ws_layout(g);
  if (!workspace || workspace_bytes < w.total || ((uintptr_t)workspace & 255u)) return BSA_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)hip_stream;
  char* ws = (char*)workspace;
  const dim3 grid((unsigned)g.nb, (unsigned)g.H, (unsigned)g.B);
  double* apart = g.reweight ? (double*)(ws + w.apart) : nullptr;
  double* anc = g.reweight ? (double*)(ws + w.anchor) : nullptr;
  if (g.reweight) {
    hipLaunchKernelGGL(pool_q_kernel<true>, grid, dim3(256), 0, s, (const uint16_t*)q, q_pool, apart,
                       (int)g.N, (int)g.nb, g.anchor_rows);
    if ((st = launch_status()) != BSA_OK) return st;
    hipLaunchKernelGGL(anchor_kernel, dim3((unsigned)g.H, (unsigned)g.B), dim3(HD), 0, s,
                       (const double*)apart, anc, (int)g.nb, g.anchor_rows);
    if ((st = launch_status()) != BSA_OK) return st;
    hipLaunchKernelGGL(pool_kv_kernel<true>, grid, dim3(256), 0, s, (const uint16_t*)k,
                       (const uint16_t*)v, (const double*)anc, k_pool, (uint16_t*)sum_k,
                       (uint16_t*)sum_v, sum_bias, (uint16_t*)(ws + w.vt), (uint16_t*)(ws + w.svt),
                       (int)g.N, (int)g.nb, (int)g.nsb, g.scale);
  } else {
    hipLaunchKernelGGL(pool_q_kernel<false>, grid, dim3(256), 0, s, (const uint16_t*)q, q_pool,
                       (double*)nullptr, (int)g.N, (int)g.nb, 0);
    if ((st = launch_status()) != BSA_OK) return st;
    hipLaunchKernelGGL(pool_kv_kernel<false>, grid, dim3(256), 0, s, (const uint16_t*)k,
                       (const uint16_t*)v, (const double*)nullptr, k_pool, (uint16_t*)sum_k,
                       (uint16_t*)sum_v, sum_bias, (uint16_t*)(ws + w.vt), (uint16_t*)(ws + w.svt),
                       (int)g.N, (int)g.nb, (int)g.nsb, g.scale);
  }
  return launch_status();
}

int bsa_select(const bsa_problem* p, const float* q_pool, const float* k_pool, int32_t* block_idx,
               void* hip_stream) {
  Geometry g;
  int st = make_geometry(p, &g);
  if (st != BSA_OK) return st;
  if (g.k == 0) return BSA_OK;
  if (!q_pool || !k_pool || !block_idx) return BSA_ERR_INVALID;
  if (!aligned16(q_pool) || !aligned16(k_pool)) return BSA_ERR_INVALID;
  const dim3 grid((unsigned)((g.nb + SEL_RB - 1) / SEL_RB), (unsigned)g.H, (unsigned)g.B);
  const size_t lds = (size_t)SEL_RB * g.nb * sizeof(double);
  if (lds > 48 * 1024) {
    // allow the score rows of large sequences beyond the default dynamic LDS cap
    if (hipFuncSetAttribute((const void*)select_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)lds) != hipSuccess)
      return BSA_ERR_HIP;
  }
  hipLaunchKernelGGL(select_kernel, grid, dim3(256), lds, (hipStream_t)hip_stream, q_pool, k_pool,
                     block_idx, (int)g.nb, (int)g.k);
  return launch_status();
}

int bsa_forward(const bsa_problem* p, const void* q, const void* k, const void* sum_k,
                const float* sum_bias, const int32_t* block_idx, const void* workspace,
                size_t workspace_bytes, void* out, void* hip_stream) {
  Geometry g;
  int st = make_geometry(p, &g);
  if (st != BSA_OK) return st;
  if (!q || !k || !out) return BSA_ERR_INVALID;
  if (g.k > 0 && !block_idx) return BSA_ERR_INVALID;
  if (g.k < g.nb && (!sum_k || !sum_bias)) return BSA_ERR_INVALID;
  if (!aligned16(q) || !aligned16(k) || !aligned16(out) || (sum_k && !aligned16(sum_k)))
    return BSA_ERR_INVALID;
  const WsLayout w = ws_layout(g);
  if (!workspace || workspace_bytes < w.total || ((uintptr_t)workspace & 255u)) return BSA_ERR_WORKSPACE;
  const char* ws = (const char*)workspace;
  const int total = (int)(g.B * g.H * g.nb);
  const float scale_log2 = (float)(g.scale * 1.4426950408889634);
  hipLaunchKernelGGL(attn_fwd_kernel, dim3((unsigned)total), dim3(256), 0, (hipStream_t)hip_stream,
                     (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)(ws + w.vt),
                     (const uint16_t*)sum_k, (const uint16_t*)(ws + w.svt), sum_bias, block_idx,
                     (uint16_t*)out, (int)g.N, (int)g.nb, (int)g.k, (int)g.nsb, scale_log2, total);
  return launch_status();
}

}  // extern "C"
