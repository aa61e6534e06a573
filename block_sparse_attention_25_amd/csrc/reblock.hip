// Spark-Reblock for gfx950 (MI355X): an adaptive 128-row block layout per
// (batch, head), applied to Q, K and V alike before the block-sparse path and
// undone on its output.
//
// Sources: "Spark-H3: Block Sparse Attention Speeds Up MiniMax-H3 in
// ComfyUI", section "What Spark-Attn changes" (queries are grouped by the
// similarity of their score patterns over the keys, a cosine distance in the
// metric of the keys' second moment; a hierarchical partitioner splits groups
// until every leaf holds one block, in O(N log N)) and section "Workflows"
// (reblock_layout=q_reuse_k: keys and values reuse the query layout).
//
// What is computed, per (batch, head):
//   M = (1/N) sum_j k_j k_j^T, L L^T = M + 1e-6 (trace(M) / 128) I + 1e-30 I,
//   z_i = L^T q_i / |L^T q_i|, so that z_i . z_j is the cosine of q_i and q_j
//   in the metric M.  A group of n rows (m = ceil(n / 128) blocks, m >= 2)
//   splits on the coordinate of z with the largest variance over the group
//   (lowest coordinate on ties): its 128 ceil(m / 2) rows with the smallest
//   value of that coordinate (ties to the lower row) go left, the rest right,
//   each in ascending row order.  The leaves, left to right, are the new
//   order: perm[p] is the row placed at position p.
//
// Kernels:
//   rb_moment_kernel    K^T K over 2048-row chunks on the matrix cores (bf16
//                       products are exact; float32 sums within a chunk)
//   rb_factor_kernel    the chunks summed in float64 (fixed order), the ridge,
//                       Cholesky in LDS (float64), L split into three bf16
//                       terms whose sum is the float32 value of each entry
//   rb_embed_kernel     z = Q L on the matrix cores (three terms), each row
//                       normalised (float32); the identity order
//   rb_level_kernel     one level of the bisection, one workgroup per group:
//                       float64 coordinate variances, a radix select of the
//                       split value, a stable partition of the group's rows
//   rb_permute_kernel   rows of Q, K, V gathered into the new order
//   rb_unpermute_kernel output rows put back in their original places
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "bsa.h"

namespace {

constexpr int RB_BLK = 128;    // rows per leaf
constexpr int RB_HD = 128;     // head_dim
constexpr int RB_CHUNK = 2048; // key rows per partial second moment
constexpr double RB_EPS = 1e-6;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ float rb_bf2f(uint32_t h) { return __uint_as_float(h << 16); }

// float -> bfloat16 bits, round to nearest even (finite inputs)
__device__ __forceinline__ uint16_t rb_f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// order-preserving key of a float (-0 and +0 equal)
__device__ __forceinline__ uint32_t rb_key(float x) {
  const uint32_t u = x == 0.f ? 0u : __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ------------------------------------------------------------ moment ---
// One workgroup of 4 wavefronts per (chunk of 2048 key rows, batch x head).
// Each 64-row step is staged in LDS transposed (feature-major), so that both
// MFMA operands of K^T K read 8 consecutive rows of one feature in 16 bytes.
// Wavefront w owns the 32 x 128 output stripe of features 32 w + [0, 32).
constexpr int MT_STRIDE = 64 + 8;  // LDS row stride (elements) of the transposed step

__global__ __launch_bounds__(256) void rb_moment_kernel(const uint16_t* __restrict__ k,
                                                        float* __restrict__ part, int N, int nchunk) {
  __shared__ __attribute__((aligned(16))) uint16_t kt[RB_HD * MT_STRIDE];
  const int chunk = blockIdx.x % nchunk;
  const size_t bh = blockIdx.x / nchunk;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, ln = lane & 31;
  const uint16_t* kb = k + bh * (size_t)N * RB_HD;
  const int r0 = chunk * RB_CHUNK, r1 = min(N, r0 + RB_CHUNK);
  f32x16 acc[4] = {f32x16{}, f32x16{}, f32x16{}, f32x16{}};
  for (int t0 = r0; t0 < r1; t0 += 64) {
    // 64 rows x 128 features = 1024 pieces of 8 features, four per thread
    uint4 piece[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int x = tid + 256 * u, row = x >> 4, c8 = x & 15;
      piece[u] = t0 + row < r1 ? *(const uint4*)(kb + (size_t)(t0 + row) * RB_HD + 8 * c8)
                               : make_uint4(0u, 0u, 0u, 0u);
    }
    __syncthreads();  // the previous step's operand reads are done
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int x = tid + 256 * u, row = x >> 4, c8 = x & 15;
      const uint32_t w[4] = {piece[u].x, piece[u].y, piece[u].z, piece[u].w};
#pragma unroll
      for (int e = 0; e < 8; ++e)
        kt[(8 * c8 + e) * MT_STRIDE + row] = (uint16_t)((e & 1) ? (w[e >> 1] >> 16) : (w[e >> 1] & 0xFFFFu));
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const bf16x8 a = *(const bf16x8*)&kt[(32 * wave + ln) * MT_STRIDE + 16 * s + 8 * g];
#pragma unroll
      for (int tj = 0; tj < 4; ++tj) {
        const bf16x8 b = *(const bf16x8*)&kt[(32 * tj + ln) * MT_STRIDE + 16 * s + 8 * g];
        acc[tj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[tj], 0, 0, 0);
      }
    }
  }
  // accumulator element a of tile (wave, tj): feature pair (32 wave + m, 32 tj + ln)
  // with m = 8 (a / 4) + 4 g + a % 4
  float* pb = part + (bh * nchunk + chunk) * (size_t)RB_HD * RB_HD;
#pragma unroll
  for (int tj = 0; tj < 4; ++tj)
#pragma unroll
    for (int a = 0; a < 16; ++a) {
      const int m = 8 * (a >> 2) + 4 * g + (a & 3);
      pb[(32 * wave + m) * RB_HD + 32 * tj + ln] = acc[tj][a];
    }
}

// ------------------------------------------------------------ factor ---
// One workgroup of 1024 threads per (batch, head): M in LDS (float64), the
// ridge, a right-looking Cholesky on the lower triangle, then L^T written as
// three bfloat16 terms per entry (rows d = output coordinate, columns e =
// query feature), the B operand of z = q L.
__global__ __launch_bounds__(1024) void rb_factor_kernel(const float* __restrict__ part,
                                                         uint16_t* __restrict__ ltw, int N, int nchunk) {
  __shared__ double A[RB_HD][RB_HD + 1];
  __shared__ double ridge_s;
  const size_t bh = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63;
  const float* pb = part + bh * (size_t)nchunk * RB_HD * RB_HD;
  for (int x = tid; x < RB_HD * RB_HD; x += 1024) {
    double s = 0.0;
    for (int c = 0; c < nchunk; ++c) s += (double)pb[(size_t)c * RB_HD * RB_HD + x];
    A[x / RB_HD][x % RB_HD] = s / (double)N;
  }
  __syncthreads();
  if (tid < 64) {
    double t = A[lane][lane] + A[lane + 64][lane + 64];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) t += __shfl_xor(t, off, 64);
    if (lane == 0) ridge_s = RB_EPS * (t / RB_HD) + 1e-30;
  }
  __syncthreads();
  const double ridge = ridge_s;
  if (tid < RB_HD) A[tid][tid] += ridge;
  __syncthreads();
  for (int j = 0; j < RB_HD; ++j) {
    // a pivot that float32 rounding of M pushed below the ridge is held at it
    if (tid == 0) A[j][j] = sqrt(fmax(A[j][j], ridge));
    __syncthreads();
    const double piv = A[j][j];
    if (tid > j && tid < RB_HD) A[tid][j] /= piv;
    __syncthreads();
    const int nr = RB_HD - 1 - j;
    for (int x = tid; x < nr * nr; x += 1024) {
      const int i = j + 1 + x / nr, c = j + 1 + x % nr;
      if (c <= i) A[i][c] -= A[i][j] * A[c][j];
    }
    __syncthreads();
  }
  uint16_t* lb = ltw + bh * 3 * (size_t)RB_HD * RB_HD;
  for (int x = tid; x < RB_HD * RB_HD; x += 1024) {
    const int d = x / RB_HD, e = x % RB_HD;
    const float f = e >= d ? (float)A[e][d] : 0.f;
    const uint16_t hi = rb_f2bf(f);
    const float r1 = f - rb_bf2f(hi);  // exact
    const uint16_t mid = rb_f2bf(r1);
    const float r2 = r1 - rb_bf2f(mid);  // exact, at most 8 significant bits
    lb[x] = hi;
    lb[RB_HD * RB_HD + x] = mid;
    lb[2 * RB_HD * RB_HD + x] = rb_f2bf(r2);
  }
}

// ------------------------------------------------------------- embed ---
// One workgroup of 4 wavefronts per (256 rows, batch x head); wavefront w
// takes rows 64 w + [0, 64) as two 32-row tiles against the four 32-column
// tiles of z.  The three terms of L^T sit in LDS with the 16-byte piece c of
// row d stored at piece c ^ (d mod 16), so that the 32 rows a B-operand read
// touches fall into different banks.
__global__ __launch_bounds__(256) void rb_embed_kernel(const uint16_t* __restrict__ q,
                                                       const uint16_t* __restrict__ ltw,
                                                       float* __restrict__ zh, int32_t* __restrict__ order0,
                                                       int N, int ntile) {
  __shared__ __attribute__((aligned(16))) uint16_t lb[3 * RB_HD * RB_HD];
  const int tile = blockIdx.x % ntile;
  const size_t bh = blockIdx.x / ntile;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, ln = lane & 31;
  const int row0 = tile * 256;
  {
    const uint4* src = (const uint4*)(ltw + bh * 3 * (size_t)RB_HD * RB_HD);
    for (int x = tid; x < 3 * RB_HD * 16; x += 256) {
      const int t = x / (RB_HD * 16), d = (x >> 4) % RB_HD, c = x & 15;
      *(uint4*)&lb[(t * RB_HD + d) * RB_HD + 8 * (c ^ (d & 15))] = src[x];
    }
  }
  if (row0 + tid < N) order0[bh * N + row0 + tid] = row0 + tid;
  __syncthreads();
  f32x16 acc[2][4];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int tj = 0; tj < 4; ++tj) acc[rt][tj] = f32x16{};
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    const int qi = row0 + 64 * wave + 32 * rt + ln;
    const uint16_t* qrow = q + (bh * (size_t)N + (size_t)min(qi, N - 1)) * RB_HD;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      uint4 u = *(const uint4*)(qrow + 16 * s + 8 * g);
      if (qi >= N) u = make_uint4(0u, 0u, 0u, 0u);
      const bf16x8 a = __builtin_bit_cast(bf16x8, u);
#pragma unroll
      for (int term = 2; term >= 0; --term)
#pragma unroll
        for (int tj = 0; tj < 4; ++tj) {
          const int d = 32 * tj + ln;
          const bf16x8 b = *(const bf16x8*)&lb[(term * RB_HD + d) * RB_HD + 8 * ((2 * s + g) ^ (d & 15))];
          acc[rt][tj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[rt][tj], 0, 0, 0);
        }
    }
  }
  // element a of tile (rt, tj): row 8 (a / 4) + 4 g + a % 4 of the row tile,
  // coordinate 32 tj + ln; a row's 128 coordinates live in the 32 lanes of
  // one half-wave
  float* zb = zh + bh * (size_t)N * RB_HD;
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int a = 0; a < 16; ++a) {
      float ss = 0.f;
#pragma unroll
      for (int tj = 0; tj < 4; ++tj) ss += acc[rt][tj][a] * acc[rt][tj][a];
#pragma unroll
      for (int off = 16; off > 0; off >>= 1) ss += __shfl_xor(ss, off, 64);
      const float inv = ss > 0.f ? 1.0f / sqrtf(ss) : 0.f;
      const int row = row0 + 64 * wave + 32 * rt + 8 * (a >> 2) + 4 * g + (a & 3);
      if (row < N) {
#pragma unroll
        for (int tj = 0; tj < 4; ++tj) zb[(size_t)row * RB_HD + 32 * tj + ln] = acc[rt][tj][a] * inv;
      }
    }
}

// ------------------------------------------------------------- level ---
constexpr int LV_THREADS = 1024;
constexpr int LV_WAVES = LV_THREADS / 64;

// exclusive prefix over the workgroup of two counters (x, y) per thread
__device__ __forceinline__ void block_scan2(int& x, int& y, int (*wt)[2], int lane, int wave) {
  int ix = x, iy = y;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int ox = __shfl_up(ix, off, 64), oy = __shfl_up(iy, off, 64);
    if (lane >= off) {
      ix += ox;
      iy += oy;
    }
  }
  if (lane == 63) {
    wt[wave][0] = ix;
    wt[wave][1] = iy;
  }
  __syncthreads();
  int bx = 0, by = 0;
  for (int w = 0; w < wave; ++w) {
    bx += wt[w][0];
    by += wt[w][1];
  }
  x = bx + ix - x;
  y = by + iy - y;
}

// One level of the bisection.  Workgroup (bh, g) follows the bits of g from
// the root to its group [s, s + n) of the current order; a path that enters a
// finished leaf with a 1 bit is empty, one with 0 bits carries the leaf over.
__global__ __launch_bounds__(LV_THREADS) void rb_level_kernel(const float* __restrict__ zh,
                                                              const int32_t* __restrict__ pin,
                                                              int32_t* __restrict__ pout,
                                                              uint32_t* __restrict__ keys, int N, int level) {
  __shared__ double red[2][LV_WAVES][RB_HD];
  __shared__ uint32_t hist[256];
  __shared__ int wt[LV_WAVES][2];
  __shared__ int sh_d, sh_digit, sh_want;
  const int ng = 1 << level;
  const int gi = blockIdx.x % ng;
  const size_t bh = blockIdx.x / ng;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  int s = 0, n = N;
  for (int t = level - 1; t >= 0; --t) {
    const int m = (n + RB_BLK - 1) / RB_BLK;
    const int bit = (gi >> t) & 1;
    if (m <= 1) {
      if (bit) return;
      continue;
    }
    const int nl = RB_BLK * ((m + 1) / 2);
    if (bit) {
      s += nl;
      n -= nl;
    } else {
      n = nl;
    }
  }
  const int32_t* pi = pin + bh * N + s;
  int32_t* po = pout + bh * N + s;
  const int m = (n + RB_BLK - 1) / RB_BLK;
  if (m <= 1) {
    for (int j = tid; j < n; j += LV_THREADS) po[j] = pi[j];
    return;
  }
  const int nl = RB_BLK * ((m + 1) / 2);
  const float* zb = zh + bh * (size_t)N * RB_HD;
  uint32_t* kb = keys + bh * N + s;

  // (1) sums of z and z^2 per coordinate (float64): wavefront w takes rows
  // w, w + 16, ...; lane l coordinates 2 l and 2 l + 1
  {
    double s1x = 0.0, s1y = 0.0, s2x = 0.0, s2y = 0.0;
    for (int j = wave; j < n; j += 4 * LV_WAVES) {
      int r[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) r[u] = j + u * LV_WAVES < n ? pi[j + u * LV_WAVES] : -1;
      float2 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u)
        v[u] = r[u] >= 0 ? *(const float2*)(zb + (size_t)r[u] * RB_HD + 2 * lane) : make_float2(0.f, 0.f);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        s1x += (double)v[u].x;
        s1y += (double)v[u].y;
        s2x += (double)v[u].x * (double)v[u].x;
        s2y += (double)v[u].y * (double)v[u].y;
      }
    }
    red[0][wave][2 * lane] = s1x;
    red[0][wave][2 * lane + 1] = s1y;
    red[1][wave][2 * lane] = s2x;
    red[1][wave][2 * lane + 1] = s2y;
  }
  __syncthreads();
  if (wave == 0) {
    double best = -1.0;
    int bd = 0;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int d = lane + 64 * h;
      double a = 0.0, b = 0.0;
      for (int w = 0; w < LV_WAVES; ++w) {
        a += red[0][w][d];
        b += red[1][w][d];
      }
      const double mu = a / n;
      const double var = b / n - mu * mu;
      if (var > best) {
        best = var;
        bd = d;
      }
    }
    // largest variance, the lowest coordinate on ties
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      const double ob = __shfl_xor(best, off, 64);
      const int od = __shfl_xor(bd, off, 64);
      if (ob > best || (ob == best && od < bd)) {
        best = ob;
        bd = od;
      }
    }
    if (lane == 0) sh_d = bd;
  }
  __syncthreads();
  const int dstar = sh_d;

  // (2) keys of the split coordinate, in group order
  for (int j = tid; j < n; j += LV_THREADS) kb[j] = rb_key(zb[(size_t)pi[j] * RB_HD + dstar]);
  __syncthreads();

  // (3) the key of rank nl - 1: MSB-first radix select, 8 bits a pass
  uint32_t prefix = 0u, pmask = 0u;
  int want = nl - 1;
  for (int shift = 24; shift >= 0; shift -= 8) {
    if (tid < 256) hist[tid] = 0u;
    __syncthreads();
    for (int j = tid; j < n; j += LV_THREADS) {
      const uint32_t key = kb[j];
      if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (wave == 0) {
      const uint32_t h0 = hist[4 * lane], h1 = hist[4 * lane + 1], h2 = hist[4 * lane + 2],
                     h3 = hist[4 * lane + 3];
      const int c = (int)(h0 + h1 + h2 + h3);
      int incl = c;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int o = __shfl_up(incl, off, 64);
        if (lane >= off) incl += o;
      }
      int before = incl - c;
      if (before <= want && want < incl) {
        const uint32_t hh[4] = {h0, h1, h2, h3};
        int dg = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (dg == e && before + (int)hh[e] <= want) {
            before += (int)hh[e];
            dg = e + 1;
          }
        }
        sh_digit = 4 * lane + dg;
        sh_want = want - before;
      }
    }
    __syncthreads();
    prefix |= (uint32_t)sh_digit << shift;
    pmask |= 255u << shift;
    want = sh_want;
  }
  const uint32_t T = prefix;
  const int need = want + 1;  // keys equal to T that go left, the first in order

  // (4) stable partition: thread t takes positions [t C, t C + C)
  const int C = (n + LV_THREADS - 1) / LV_THREADS;
  const int j0 = min(n, tid * C), j1 = min(n, j0 + C);
  int lt = 0, eq = 0;
  for (int j = j0; j < j1; ++j) {
    const uint32_t key = kb[j];
    lt += key < T;
    eq += key == T;
  }
  block_scan2(lt, eq, wt, lane, wave);
  for (int j = j0; j < j1; ++j) {
    const uint32_t key = kb[j];
    const int before_left = lt + min(eq, need);
    const bool left = key < T || (key == T && eq < need);
    // the counts place every row inside [0, n); the clamp only keeps a
    // miscount from writing outside the group
    po[min(left ? before_left : nl + (j - before_left), n - 1)] = pi[j];
    lt += key < T;
    eq += key == T;
  }
}

// ----------------------------------------------------------- permute ---
// 16 rows of 256 bytes per workgroup, 16 bytes a thread, for each tensor.
__global__ __launch_bounds__(256) void rb_permute_kernel(const uint16_t* __restrict__ q,
                                                         const uint16_t* __restrict__ k,
                                                         const uint16_t* __restrict__ v,
                                                         const int32_t* __restrict__ perm,
                                                         uint16_t* __restrict__ qp, uint16_t* __restrict__ kp,
                                                         uint16_t* __restrict__ vp, int N, int ntile) {
  const int tile = blockIdx.x % ntile;
  const size_t bh = blockIdx.x / ntile;
  const int p = tile * 16 + (threadIdx.x >> 4), c = threadIdx.x & 15;
  if (p >= N) return;
  const size_t src = (bh * N + (size_t)perm[bh * N + p]) * RB_HD + 8 * c;
  const size_t dst = (bh * N + (size_t)p) * RB_HD + 8 * c;
  const uint4 a = *(const uint4*)(q + src), b = *(const uint4*)(k + src), d = *(const uint4*)(v + src);
  *(uint4*)(qp + dst) = a;
  *(uint4*)(kp + dst) = b;
  *(uint4*)(vp + dst) = d;
}

__global__ __launch_bounds__(256) void rb_unpermute_kernel(const uint16_t* __restrict__ x,
                                                           const int32_t* __restrict__ perm,
                                                           uint16_t* __restrict__ y, int N, int ntile) {
  const int tile = blockIdx.x % ntile;
  const size_t bh = blockIdx.x / ntile;
  const int p = tile * 16 + (threadIdx.x >> 4), c = threadIdx.x & 15;
  if (p >= N) return;
  const size_t src = (bh * N + (size_t)p) * RB_HD + 8 * c;
  const size_t dst = (bh * N + (size_t)perm[bh * N + p]) * RB_HD + 8 * c;
  *(uint4*)(y + dst) = *(const uint4*)(x + src);
}

// ---------------------------------------------------------------- host ---
struct RbGeom {
  int64_t BH, N, nb;
  int levels, nchunk;
};

struct RbLayout {
  size_t part, ltw, zh, keys, perm, total;
};

size_t rb_align(size_t x) { return (x + 255) & ~(size_t)255; }

int rb_geometry(const bsa_problem* p, RbGeom* g) {
  if (!p) return BSA_ERR_INVALID;
  if (p->head_dim != BSA_HEAD_DIM || p->block_size != BSA_BLOCK) return BSA_ERR_UNSUPPORTED;
  if (p->batch < 1 || p->heads < 1 || p->seq_len < 1) return BSA_ERR_INVALID;
  if (p->batch > 65535 || p->heads > 65535) return BSA_ERR_INVALID;
  // the later stages address rows by position: a conditioning row range, or
  // an anchor over part of the rows, would no longer name the same rows
  if (p->sink_rows != 0) return BSA_ERR_UNSUPPORTED;
  if (p->summary == BSA_SUMMARY_REWEIGHT && p->anchor_rows != 0 && p->anchor_rows != p->seq_len)
    return BSA_ERR_UNSUPPORTED;
  g->BH = (int64_t)p->batch * p->heads;
  g->N = p->seq_len;
  g->nb = (g->N + RB_BLK - 1) / RB_BLK;
  g->levels = 0;
  while ((int64_t(1) << g->levels) < g->nb) ++g->levels;
  g->nchunk = (int)((g->N + RB_CHUNK - 1) / RB_CHUNK);
  // 1-D grids: work-items per launch must fit 32 bits
  const int64_t lv_wg = g->levels > 0 ? (int64_t(1) << (g->levels - 1)) : 1;
  if (g->BH * lv_wg * LV_THREADS >= (int64_t(1) << 32)) return BSA_ERR_UNSUPPORTED;
  if (g->BH * ((g->N + 15) / 16) * 256 >= (int64_t(1) << 32)) return BSA_ERR_UNSUPPORTED;
  return BSA_OK;
}

RbLayout rb_layout(const RbGeom& g) {
  RbLayout w{};
  size_t off = 0;
  w.part = off;
  off = rb_align(off + (size_t)g.BH * g.nchunk * RB_HD * RB_HD * sizeof(float));
  w.ltw = off;
  off = rb_align(off + (size_t)g.BH * 3 * RB_HD * RB_HD * sizeof(uint16_t));
  w.zh = off;
  off = rb_align(off + (size_t)g.BH * g.N * RB_HD * sizeof(float));
  w.keys = off;
  off = rb_align(off + (size_t)g.BH * g.N * sizeof(uint32_t));
  w.perm = off;
  off = rb_align(off + (size_t)g.BH * g.N * sizeof(int32_t));
  w.total = off;
  return w;
}

bool rb_aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int rb_status() { return hipGetLastError() == hipSuccess ? BSA_OK : BSA_ERR_HIP; }

}  // namespace

extern "C" {

int bsa_reblock_workspace_bytes(const bsa_problem* p, size_t* bytes) {
  RbGeom g;
  const int st = rb_geometry(p, &g);
  if (st != BSA_OK) return st;
  if (!bytes) return BSA_ERR_INVALID;
  *bytes = rb_layout(g).total;
  return BSA_OK;
}

int bsa_reblock(const bsa_problem* p, const void* q, const void* k, int32_t* perm, void* workspace,
                size_t workspace_bytes, void* stream) {
  RbGeom g;
  const int st = rb_geometry(p, &g);
  if (st != BSA_OK) return st;
  if (!q || !k || !perm) return BSA_ERR_INVALID;
  if (!rb_aligned16(q) || !rb_aligned16(k) || ((uintptr_t)perm & 3u)) return BSA_ERR_INVALID;
  const RbLayout w = rb_layout(g);
  if (!workspace || workspace_bytes < w.total || ((uintptr_t)workspace & 255u)) return BSA_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  char* ws = (char*)workspace;
  float* part = (float*)(ws + w.part);
  uint16_t* ltw = (uint16_t*)(ws + w.ltw);
  float* zh = (float*)(ws + w.zh);
  uint32_t* keys = (uint32_t*)(ws + w.keys);
  int32_t* tmp = (int32_t*)(ws + w.perm);
  // level l reads buf[l % 2] and writes buf[(l + 1) % 2]; the last level
  // writes the caller's array
  int32_t* buf[2] = {(g.levels % 2 == 0) ? perm : tmp, (g.levels % 2 == 0) ? tmp : perm};
  const int N = (int)g.N;
  hipLaunchKernelGGL(rb_moment_kernel, dim3((unsigned)(g.BH * g.nchunk)), dim3(256), 0, s,
                     (const uint16_t*)k, part, N, g.nchunk);
  hipLaunchKernelGGL(rb_factor_kernel, dim3((unsigned)g.BH), dim3(1024), 0, s, (const float*)part, ltw, N,
                     g.nchunk);
  const int ntile = (N + 255) / 256;
  hipLaunchKernelGGL(rb_embed_kernel, dim3((unsigned)(g.BH * ntile)), dim3(256), 0, s, (const uint16_t*)q,
                     (const uint16_t*)ltw, zh, buf[0], N, ntile);
  for (int l = 0; l < g.levels; ++l)
    hipLaunchKernelGGL(rb_level_kernel, dim3((unsigned)(g.BH << l)), dim3(LV_THREADS), 0, s, (const float*)zh,
                       (const int32_t*)buf[l & 1], buf[(l + 1) & 1], keys, N, l);
  return rb_status();
}

int bsa_permute_rows(const bsa_problem* p, const int32_t* perm, const void* q, const void* k, const void* v,
                     void* q_out, void* k_out, void* v_out, void* stream) {
  RbGeom g;
  const int st = rb_geometry(p, &g);
  if (st != BSA_OK) return st;
  if (!perm || !q || !k || !v || !q_out || !k_out || !v_out) return BSA_ERR_INVALID;
  if (!rb_aligned16(q) || !rb_aligned16(k) || !rb_aligned16(v) || !rb_aligned16(q_out) ||
      !rb_aligned16(k_out) || !rb_aligned16(v_out))
    return BSA_ERR_INVALID;
  const int ntile = (int)((g.N + 15) / 16);
  hipLaunchKernelGGL(rb_permute_kernel, dim3((unsigned)(g.BH * ntile)), dim3(256), 0, (hipStream_t)stream,
                     (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, perm, (uint16_t*)q_out,
                     (uint16_t*)k_out, (uint16_t*)v_out, (int)g.N, ntile);
  return rb_status();
}

int bsa_unpermute_rows(const bsa_problem* p, const int32_t* perm, const void* x, void* out, void* stream) {
  RbGeom g;
  const int st = rb_geometry(p, &g);
  if (st != BSA_OK) return st;
  if (!perm || !x || !out) return BSA_ERR_INVALID;
  if (!rb_aligned16(x) || !rb_aligned16(out)) return BSA_ERR_INVALID;
  const int ntile = (int)((g.N + 15) / 16);
  hipLaunchKernelGGL(rb_unpermute_kernel, dim3((unsigned)(g.BH * ntile)), dim3(256), 0, (hipStream_t)stream,
                     (const uint16_t*)x, perm, (uint16_t*)out, (int)g.N, ntile);
  return rb_status();
}

}  // extern "C"
