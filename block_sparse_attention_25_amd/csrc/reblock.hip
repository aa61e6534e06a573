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
//   splits by two pivots: a, its row farthest from the centroid of its z
//   rows, and b, its row farthest from a (lowest row on ties); its 128
//   ceil(m / 2) rows with the smallest z_i . (z_b - z_a) (ties to the lower
//   row) go left, the rest right, each in ascending row order.  The leaves,
//   left to right, are the new order: perm[p] is the row placed at position
//   p.  Only distances between z rows enter, so the order depends on the
//   metric cosines alone, not on the basis of the head features.
//
// Kernels:
//   rb_moment_kernel    K^T K over 2048-row chunks on the matrix cores (bf16
//                       products are exact; float32 sums within a chunk)
//   rb_msum_kernel      the chunks summed in float64 (fixed order)
//   rb_factor_kernel    the ridge, Cholesky in LDS (float64), L split into
//                       three bf16 terms whose sum is the float32 value of
//                       each entry
//   rb_embed_kernel     z = Q L on the matrix cores (three terms), each row
//                       normalised (float32, and a float16 copy); the
//                       identity order
//   per level of the bisection:
//   rb_stats_kernel     float64 sums of z per coordinate over 128-position
//                       slices of the root and of left children (a right
//                       child's sums are its parent's less its left sibling's)
//   rb_center_kernel    per group: its totals and centroid
//   rb_far16_kernel     per slice: each row's distance from the group's
//                       centroid (then from its first pivot) from the float16
//                       copy of z, and the slice's largest
//   rb_pivot_kernel     per group: the rows within the float16 error bound of
//                       the largest, their float64 distances from the float32
//                       z, the farthest (lowest row on ties)
//   rb_keys_kernel      per slice: each row's split key z_i . (z_b - z_a)
//   rb_split_*_kernel   per group: the split value of the keys (a radix
//                       select, or a bitwise search for small groups), a
//                       stable partition of the group's rows (one wavefront
//                       per group up to 1024 rows, else one workgroup)
//   rb_permute_kernel   rows of Q, K, V gathered into the new order
//   rb_unpermute_kernel output rows put back in their original places
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "bsa.h"

// keeps the runtime error behind a failed launch for bsa_hip_error_str (bsa.hip)
void bsa_note_hip_error(hipError_t e);

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

// two floats -> float16 bits (round to nearest even), the first in the low half
__device__ __forceinline__ uint32_t rb_half2(float a, float b) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)a) |
         ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)b) << 16);
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
// Thread t loads 8 features (piece t mod 16) of rows 4 (t / 16) + [0, 4) and
// writes each feature's 4 values in one 8-byte store; the next step's rows
// are loaded while this step's MFMAs run.  Wavefront w owns the 32 x 128
// output stripe of features 32 w + [0, 32).
constexpr int MT_STRIDE = 64 + 8;  // LDS row stride (elements) of the transposed step

__global__ __launch_bounds__(256) void rb_moment_kernel(const uint16_t* __restrict__ k,
                                                        float* __restrict__ part, int N, int nchunk) {
  __shared__ __attribute__((aligned(16))) uint16_t kt[RB_HD * MT_STRIDE];
  const int chunk = blockIdx.x % nchunk;
  const size_t bh = blockIdx.x / nchunk;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, ln = lane & 31;
  const int c8 = tid & 15, tq = tid >> 4;
  const uint16_t* kb = k + bh * (size_t)N * RB_HD;
  const int r0 = chunk * RB_CHUNK, r1 = min(N, r0 + RB_CHUNK);
  // rows past the chunk read its last row and are zeroed when staged
  auto load = [&](int t0, uint4* pc) {
#pragma unroll
    for (int u = 0; u < 4; ++u)
      pc[u] = *(const uint4*)(kb + (size_t)min(t0 + 4 * tq + u, r1 - 1) * RB_HD + 8 * c8);
  };
  f32x16 acc[4] = {f32x16{}, f32x16{}, f32x16{}, f32x16{}};
  uint4 pc[4];
  load(r0, pc);
  for (int t0 = r0; t0 < r1; t0 += 64) {
    __syncthreads();  // the previous step's operand reads are done
    uint32_t w[4][4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const bool ok = t0 + 4 * tq + u < r1;
      w[u][0] = ok ? pc[u].x : 0u;
      w[u][1] = ok ? pc[u].y : 0u;
      w[u][2] = ok ? pc[u].z : 0u;
      w[u][3] = ok ? pc[u].w : 0u;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      uint32_t h[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) h[u] = (e & 1) ? (w[u][e >> 1] >> 16) : (w[u][e >> 1] & 0xFFFFu);
      *(uint2*)&kt[(8 * c8 + e) * MT_STRIDE + 4 * tq] = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
    }
    __syncthreads();
    load(t0 + 64, pc);
    // keep the next step's loads ahead of this step's MFMAs (left to itself
    // the scheduler sinks them past the MFMAs, next to their first use)
    __builtin_amdgcn_sched_barrier(0);
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

// M = (1/N) times the sum of the chunk partials, float64, added in chunk
// order; one thread per entry, 64 workgroups per (batch, head).
__global__ __launch_bounds__(256) void rb_msum_kernel(const float* __restrict__ part, double* __restrict__ msum,
                                                      int N, int nchunk) {
  const int x = (blockIdx.x & 63) * 256 + threadIdx.x;
  const size_t bh = blockIdx.x >> 6;
  const float* pb = part + bh * (size_t)nchunk * RB_HD * RB_HD + x;
  double s = 0.0;
  int c = 0;
  for (; c + 4 <= nchunk; c += 4) {
    float v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = pb[(size_t)(c + u) * RB_HD * RB_HD];
#pragma unroll
    for (int u = 0; u < 4; ++u) s += (double)v[u];
  }
  for (; c < nchunk; ++c) s += (double)pb[(size_t)c * RB_HD * RB_HD];
  msum[bh * RB_HD * RB_HD + x] = s / (double)N;
}

// ------------------------------------------------------------ factor ---
// One workgroup of 1024 threads per (batch, head): M in LDS (float64), the
// ridge, a right-looking Cholesky on the lower triangle, then L^T written as
// three bfloat16 terms per entry (rows d = output coordinate, columns e =
// query feature), the B operand of z = q L.
__global__ __launch_bounds__(1024) void rb_factor_kernel(const double* __restrict__ msum,
                                                         uint16_t* __restrict__ ltw) {
  __shared__ double A[RB_HD][RB_HD + 1];
  __shared__ double piv[RB_HD];
  __shared__ double ridge_s;
  const size_t bh = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63;
  const double* mb = msum + bh * RB_HD * RB_HD;
#pragma unroll
  for (int u = 0; u < RB_HD * RB_HD / 1024; ++u) {
    const int x = tid + 1024 * u;
    A[x / RB_HD][x % RB_HD] = mb[x];
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
  // Right-looking elimination on the unscaled Schur complements, one barrier
  // a step: step j subtracts A[i][j] A[c][j] / d_j from every entry (i, c),
  // j < c <= i, with d_j = A[j][j] (held at the ridge when float32 rounding
  // of M pushed it below); L[j][j] = sqrt(d_j), L[i][j] = A[i][j] / sqrt(d_j).
  // Thread t keeps the entries x = t + 1024 u of the lower triangle (x = i
  // (i + 1) / 2 + c, c <= i) in registers; column j + 1, once step j has
  // updated it, goes through LDS (two buffers by step parity), which is all
  // that step j + 1 reads.
  constexpr int NTRI = RB_HD * (RB_HD + 1) / 2, PER = (NTRI + 1023) / 1024;
  __shared__ double col[2][RB_HD];
  double a[PER];
  int ei[PER], ec[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int x = tid + 1024 * u;
    int i = 0, c = 0;
    if (x < NTRI) {
      i = (int)((sqrtf(8.0f * (float)x + 1.0f) - 1.0f) * 0.5f);
      if ((i + 1) * (i + 2) / 2 <= x) ++i;
      if (i * (i + 1) / 2 > x) --i;
      c = x - i * (i + 1) / 2;
    }
    ei[u] = x < NTRI ? i : -1;  // -1: no entry
    ec[u] = c;
    a[u] = x < NTRI ? A[i][c] : 0.0;
    if (x < NTRI && c == 0) col[0][i] = a[u];
  }
  __syncthreads();
  for (int j = 0; j < RB_HD; ++j) {
    const double* cj = col[j & 1];
    double* cn = col[(j + 1) & 1];
    const double dj = fmax(cj[j], ridge);
    if (tid == 0) piv[j] = dj;
    const double inv = 1.0 / dj;
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int i = ei[u], c = ec[u];
      if (c > j) {  // and so i >= c > j (entries without one have i = -1, c = 0)
        a[u] -= cj[i] * cj[c] * inv;
        if (c == j + 1) cn[i] = a[u];
      }
    }
    __syncthreads();
  }
  // the final values back to LDS for the output
#pragma unroll
  for (int u = 0; u < PER; ++u)
    if (ei[u] >= 0) A[ei[u]][ec[u]] = a[u];
  __syncthreads();
  if (tid < RB_HD) piv[tid] = sqrt(piv[tid]);
  __syncthreads();
  uint16_t* lb = ltw + bh * 3 * (size_t)RB_HD * RB_HD;
  for (int x = tid; x < RB_HD * RB_HD; x += 1024) {
    const int d = x / RB_HD, e = x % RB_HD;
    const float f = e > d ? (float)(A[e][d] / piv[d]) : e == d ? (float)piv[d] : 0.f;
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
// One workgroup of 8 wavefronts per (1024 rows, batch x head).  The product
// is taken transposed, z^T = L^T Q^T, so that lane l of a wavefront's 32-row
// tile holds 64 of the 128 coordinates of row l (the other 64 in lane l ^ 32):
// a row's squared norm is a local sum and one exchange.  The A operands (the
// three terms of L^T) come from LDS, with the 16-byte piece c of row d stored
// at piece c ^ (d mod 16); the B operands are the tile's Q rows, the next
// tile's loaded during this tile's 96 MFMAs (four independent chains).
constexpr int EM_ROWS = 1024;
constexpr int EM_WAVES = 8;

__global__ __launch_bounds__(64 * EM_WAVES) void rb_embed_kernel(const uint16_t* __restrict__ q,
                                                                 const uint16_t* __restrict__ ltw,
                                                                 float* __restrict__ zh,
                                                                 uint16_t* __restrict__ zl,
                                                                 int32_t* __restrict__ order0, int N,
                                                                 int ntile) {
  __shared__ __attribute__((aligned(16))) uint16_t lb[3 * RB_HD * RB_HD];
  // each wavefront's output, 32 rows x 32 coordinates at a time, so that the
  // stores write whole 128-byte pieces of rows (16-byte chunk c of row r at
  // chunk c ^ (r & 7))
  __shared__ __attribute__((aligned(16))) float4 stage[EM_WAVES][32 * 8];
  const int tile = blockIdx.x % ntile;
  const size_t bh = blockIdx.x / ntile;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, ln = lane & 31;
  const int row0 = tile * EM_ROWS;
  {
    const uint4* src = (const uint4*)(ltw + bh * 3 * (size_t)RB_HD * RB_HD);
    for (int x = tid; x < 3 * RB_HD * 16; x += 64 * EM_WAVES) {
      const int t = x / (RB_HD * 16), d = (x >> 4) % RB_HD, c = x & 15;
      *(uint4*)&lb[(t * RB_HD + d) * RB_HD + 8 * (c ^ (d & 15))] = src[x];
    }
  }
  for (int i = tid; i < EM_ROWS; i += 64 * EM_WAVES)
    if (row0 + i < N) order0[bh * N + row0 + i] = row0 + i;
  __syncthreads();
  const int nrows = min(EM_ROWS, N - row0);
  const int ntl = (nrows + 31) / 32;  // 32-row tiles; wavefront w takes w, w + 8, ...
  // rows past N read row N - 1; nothing is stored for them
  auto load_b = [&](int t, uint4* dst) {
    const int qi = min(row0 + 32 * t + ln, N - 1);
    const uint16_t* qr = q + (bh * (size_t)N + (size_t)qi) * RB_HD;
#pragma unroll
    for (int s = 0; s < 8; ++s) dst[s] = *(const uint4*)(qr + 16 * s + 8 * g);
  };
  float* zb = zh + bh * (size_t)N * RB_HD;
  uint16_t* zlb = zl + bh * (size_t)N * RB_HD;
  uint4 bq[8], bn[8];
  int t = wave;
  if (t < ntl) load_b(t, bq);
  for (; t < ntl; t += EM_WAVES) {
    load_b(min(t + EM_WAVES, ntl - 1), bn);
    f32x16 acc[4] = {f32x16{}, f32x16{}, f32x16{}, f32x16{}};
#pragma unroll
    for (int s = 0; s < 8; ++s) {
#pragma unroll
      for (int term = 2; term >= 0; --term)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          const int d = 32 * mt + ln;
          const bf16x8 av = *(const bf16x8*)&lb[(term * RB_HD + d) * RB_HD + 8 * ((2 * s + g) ^ (d & 15))];
          acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, __builtin_bit_cast(bf16x8, bq[s]), acc[mt], 0, 0, 0);
        }
      // keep each k-step's twelve operand reads next to its MFMAs (hoisting
      // all of them would not fit the registers)
      __builtin_amdgcn_sched_barrier(0);
    }
    // element e of tile mt: coordinate 32 mt + 8 (e / 4) + 4 g + e % 4 of row ln
    float ss = 0.f;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int e = 0; e < 16; ++e) ss += acc[mt][e] * acc[mt][e];
    ss += __shfl_xor(ss, 32, 64);
    const float inv = ss > 0.f ? 1.0f / sqrtf(ss) : 0.f;
    // coordinates 32 mt + [0, 32) of the tile's rows through the wavefront's
    // stage: lane (ln, g) puts its chunks 2 j + g of row ln, then lane l
    // takes chunk l % 8 of rows 8 k + l / 8 and stores it (float32 and float16)
    float4* st = stage[wave];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        st[ln * 8 + ((2 * j + g) ^ (ln & 7))] = make_float4(acc[mt][4 * j] * inv, acc[mt][4 * j + 1] * inv,
                                                          acc[mt][4 * j + 2] * inv, acc[mt][4 * j + 3] * inv);
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int r = 8 * k + (lane >> 3), c = lane & 7;
        const float4 f = st[r * 8 + (c ^ (r & 7))];
        const int row = row0 + 32 * t + r;
        if (row < N) {
          *(float4*)(zb + (size_t)row * RB_HD + 32 * mt + 4 * c) = f;
          *(uint2*)(zlb + (size_t)row * RB_HD + 32 * mt + 4 * c) = make_uint2(rb_half2(f.x, f.y), rb_half2(f.z, f.w));
        }
      }
      __builtin_amdgcn_wave_barrier();
    }
#pragma unroll
    for (int s = 0; s < 8; ++s) bq[s] = bn[s];
  }
}

// ------------------------------------------------------------- level ---
// One level of the bisection.  rb_stats_kernel sums z per coordinate over
// each 128-position slice of the current order (groups start on multiples of
// 128, so a slice lies in one group), for the root and the left children
// only; rb_center_kernel adds a group's slices in slice order (a right child:
// its parent's totals, kept from the level before, less its left sibling's
// slices) into its totals and centroid.  Reading only the left children's
// rows halves the sums' traffic.  Then the two pivots (rb_far16_kernel and
// rb_pivot_kernel, twice), the keys (rb_keys_kernel) and the split
// (rb_split_*_kernel).

// the group [s, s + n) that holds position pos after `level` splits (the
// tree's shape depends on N only); a finished leaf keeps its range.  right:
// the last split sent the group right.
__device__ __forceinline__ void rb_group_of(int N, int level, int pos, int& s, int& n, bool& right) {
  s = 0;
  n = N;
  right = false;
  for (int t = 0; t < level; ++t) {
    const int m = (n + RB_BLK - 1) / RB_BLK;
    if (m <= 1) break;
    const int nl = RB_BLK * ((m + 1) / 2);
    right = pos >= s + nl;
    if (right) {
      s += nl;
      n -= nl;
    } else {
      n = nl;
    }
  }
}

// One workgroup of 4 wavefronts per (slice, batch x head); wavefront w sums
// rows w + 4 i of the slice, lane l coordinates 2 l and 2 l + 1, with eight
// row loads in flight.  stats[bh][slice][d]: sum of z_d.
__global__ __launch_bounds__(256) void rb_stats_kernel(const float* __restrict__ zh,
                                                       const int32_t* __restrict__ pin,
                                                       double* __restrict__ stats, int N, int nb, int level) {
  __shared__ double red[4][RB_HD];
  const int c = blockIdx.x % nb;
  const size_t bh = blockIdx.x / nb;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int s, n;
  bool right;
  rb_group_of(N, level, c * RB_BLK, s, n, right);
  if (n <= RB_BLK || right) return;  // a leaf, or sums the centre kernel derives
  const int p0 = c * RB_BLK, cnt = min(RB_BLK, N - p0);
  const float* zb = zh + bh * (size_t)N * RB_HD;
  // lane i < 32 holds the row of slice position wave + 4 i; positions past
  // the end of a short last slice read its last row and are weighted out, so
  // every load is unconditional and all eight are in flight together
  const int myrow = pin[bh * N + p0 + min(wave + 4 * (lane & 31), cnt - 1)];
  double s1x = 0.0, s1y = 0.0;
#pragma unroll
  for (int i0 = 0; i0 < 32; i0 += 8) {
    float2 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int r = __builtin_amdgcn_readlane(myrow, i0 + u);
      v[u] = *(const float2*)(zb + (size_t)r * RB_HD + 2 * lane);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const double w = wave + 4 * (i0 + u) < cnt ? 1.0 : 0.0;
      s1x += w * (double)v[u].x;
      s1y += w * (double)v[u].y;
    }
  }
  red[wave][2 * lane] = s1x;
  red[wave][2 * lane + 1] = s1y;
  __syncthreads();
  if (tid < RB_HD) stats[(bh * nb + c) * RB_HD + tid] = red[0][tid] + red[1][tid] + red[2][tid] + red[3][tid];
}

// exclusive prefix over the workgroup of two counters (x, y) per thread
template <int W>
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

// The group [s, s + n) of workgroup-or-wavefront g at `level`, following the
// bits of g from the root: a path that enters a finished leaf with a 1 bit is
// empty (returns false); one with 0 bits carries the leaf over.  sp: the start
// of the group's parent when the last split sent it right (its left sibling
// is [sp, s)), else s.
__device__ __forceinline__ bool rb_locate(int N, int level, int gi, int& s, int& n, int& sp) {
  s = 0;
  n = N;
  sp = 0;
  for (int t = level - 1; t >= 0; --t) {
    const int m = (n + RB_BLK - 1) / RB_BLK;
    const int bit = (gi >> t) & 1;
    if (m <= 1) {
      if (bit) return false;
      continue;
    }
    const int nl = RB_BLK * ((m + 1) / 2);
    sp = s;
    if (bit) {
      s += nl;
      n -= nl;
    } else {
      n = nl;
    }
  }
  return true;
}

// sum of z_d over the slices [c0, c0 + cnt), added in slice order with eight
// loads in flight
__device__ __forceinline__ double rb_slice_sum(const double* stats_bh, int c0, int cnt, int d) {
  const double* sp = stats_bh + (size_t)c0 * RB_HD + d;
  double a = 0.0;
  for (int base = 0; base < cnt; base += 8) {
    double va[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) va[c] = sp[(size_t)min(base + c, cnt - 1) * RB_HD];
#pragma unroll
    for (int c = 0; c < 8; ++c) a += base + c < cnt ? va[c] : 0.0;
  }
  return a;
}

// One workgroup of 128 threads (one per coordinate) per group slot of the
// level: the group's totals (its slices' sums, or for a right child its
// parent's totals less its left sibling's slices), kept in tcur for its
// children, and its centroid.  Per-group arrays are indexed by the group's
// first slice.
__global__ __launch_bounds__(RB_HD) void rb_center_kernel(const double* __restrict__ stats,
                                                          const double* __restrict__ tprev,
                                                          double* __restrict__ tcur, double* __restrict__ cen,
                                                          int N, int nb, int level) {
  const int ng = 1 << level;
  const int gi = blockIdx.x % ng;
  const size_t bh = blockIdx.x / ng;
  const int d = threadIdx.x;
  int s, n, sp;
  if (!rb_locate(N, level, gi, s, n, sp)) return;
  if (n <= RB_BLK) return;
  const double* st = stats + bh * (size_t)nb * RB_HD;
  double tot;
  if (sp == s) {
    tot = rb_slice_sum(st, s / RB_BLK, (n + RB_BLK - 1) / RB_BLK, d);
  } else {
    tot = tprev[(bh * nb + sp / RB_BLK) * RB_HD + d] - rb_slice_sum(st, sp / RB_BLK, (s - sp) / RB_BLK, d);
  }
  tcur[(bh * nb + s / RB_BLK) * RB_HD + d] = tot;
  cen[(bh * nb + s / RB_BLK) * RB_HD + d] = tot / (double)n;
}

// (t, row) pairs: the larger distance wins, the lower row on ties
__device__ __forceinline__ bool rb_better(double t, int r, double bt, int br) {
  return t > bt || (t == bt && r < br);
}

// Sums over the wavefront of eight per-lane values x[u] at once: lane l ends
// with the sum of x[u], u = (l >> 3) & 7 (its bits 5, 4, 3).  Each sum pairs
// lanes as a plain butterfly does (lane ^ 32 first, then ^ 16, ..., ^ 1),
// so it has the same bits, with 10 exchanges instead of 48: at the first
// three steps a lane keeps the half of its values its bit selects and adds
// the partner's copy of that half.
template <typename T>
__device__ __forceinline__ T rb_wave_sum8(const T (&x)[8], int lane) {
  const bool b5 = lane & 32, b4 = lane & 16, b3 = lane & 8;
  T a[4], b[2];
#pragma unroll
  for (int k = 0; k < 4; ++k) a[k] = (b5 ? x[4 + k] : x[k]) + __shfl_xor(b5 ? x[k] : x[4 + k], 32, 64);
#pragma unroll
  for (int k = 0; k < 2; ++k) b[k] = (b4 ? a[2 + k] : a[k]) + __shfl_xor(b4 ? a[k] : a[2 + k], 16, 64);
  T c = (b3 ? b[1] : b[0]) + __shfl_xor(b3 ? b[0] : b[1], 8, 64);
#pragma unroll
  for (int off = 4; off > 0; off >>= 1) c += __shfl_xor(c, off, 64);
  return c;
}

// Pivot search, two stages.  The farthest row is first looked for in the
// float16 copy of z: with RNE rounding each coordinate moves by at most 2^-11
// of itself (2^-25 below the normal range), so a unit row moves by at most
// 4.9e-4, and as every row and the reference (the centroid, or the first
// pivot's row) lie within distance 2 of each other, a squared distance moves
// by at most 2 * 2 * 4.9e-4 + 3e-7 plus the float32 sum's rounding (below
// 1e-5): under 2.1e-3.  RB_FAR_EPS takes twice that.  The farthest row by the
// float64 distance from the float32 z, which defines the pivot, is then among
// the rows within 2 RB_FAR_EPS of the largest float16 distance; only those
// rows are measured again exactly (on the 768p inputs one to nine per group).
constexpr float RB_FAR_EPS = 4.2e-3f;
constexpr int RB_CAND = 2048;  // more rows in the band: every row of the group is measured exactly

// Stage one, one workgroup of 4 wavefronts per (slice, batch x head): the
// squared distance, in float32 from the float16 copy of z, of each row of the
// slice from the group's centroid (FROM_PIVOT false) or from its first pivot's
// z row (FROM_PIVOT true), at the row's position in dt, and the slice's
// largest in best_t.  Wavefront w takes positions w + 4 i, lane l coordinates
// 2 l and 2 l + 1, eight rows per exchange sequence.
template <bool FROM_PIVOT>
__global__ __launch_bounds__(256) void rb_far16_kernel(const uint16_t* __restrict__ zl,
                                                       const float* __restrict__ zh,
                                                       const int32_t* __restrict__ pin,
                                                       const double* __restrict__ cen,
                                                       const int32_t* __restrict__ piv, float* __restrict__ dt,
                                                       double* __restrict__ best_t, int N, int nb, int level) {
  __shared__ float wm[4];
  const int c = blockIdx.x % nb;
  const size_t bh = blockIdx.x / nb;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int s, n;
  bool right;
  rb_group_of(N, level, c * RB_BLK, s, n, right);
  if (n <= RB_BLK) return;  // a leaf
  const size_t g0 = bh * nb + s / RB_BLK;
  const uint16_t* zlb = zl + bh * (size_t)N * RB_HD;
  float v0, v1;
  if (FROM_PIVOT) {
    const float2 pz = *(const float2*)(zh + (bh * (size_t)N + piv[2 * g0]) * RB_HD + 2 * lane);
    v0 = pz.x;
    v1 = pz.y;
  } else {
    v0 = (float)cen[g0 * RB_HD + 2 * lane];
    v1 = (float)cen[g0 * RB_HD + 2 * lane + 1];
  }
  const int p0 = c * RB_BLK, cnt = min(RB_BLK, N - p0);
  const int myrow = pin[bh * N + p0 + min(wave + 4 * (lane & 31), cnt - 1)];
  const int mu = (lane >> 3) & 7;  // the row of each group of 8 rows whose sum this lane ends with
  float mx = -1.f;
#pragma unroll
  for (int i0 = 0; i0 < 32; i0 += 8) {
    uint32_t hv[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int r = __builtin_amdgcn_readlane(myrow, i0 + u);
      hv[u] = *(const uint32_t*)(zlb + (size_t)r * RB_HD + 2 * lane);
    }
    float d[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const float x0 = (float)__builtin_bit_cast(_Float16, (uint16_t)(hv[u] & 0xFFFFu));
      const float x1 = (float)__builtin_bit_cast(_Float16, (uint16_t)(hv[u] >> 16));
      const float dx = x0 - v0, dy = x1 - v1;
      d[u] = dx * dx + dy * dy;
    }
    const float t = rb_wave_sum8(d, lane);
    const int pos = wave + 4 * (i0 + mu);
    if (pos < cnt) {
      if ((lane & 7) == 0) dt[bh * N + p0 + pos] = t;
      mx = fmaxf(mx, t);
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
  if (lane == 0) wm[wave] = mx;
  __syncthreads();
  if (tid == 0) best_t[bh * nb + c] = fmaxf(fmaxf(wm[0], wm[1]), fmaxf(wm[2], wm[3]));
}

// Stage two, one workgroup of 4 wavefronts per group slot: the group's
// largest float16 distance over its slices, the positions whose float16
// distance is within 2 RB_FAR_EPS of it, and for those rows the float64
// squared distance from the float32 z (lane l coordinates 2 l and 2 l + 1,
// summed over the wavefront lane ^ 32 first, then ^ 16, ..., ^ 1, eight rows
// per exchange sequence with their loads in flight together); the farthest,
// lowest row on ties, is pivot WHICH (0: a, from the centroid; 1: b, from a)
// of the group.  At 2K 5s the band holds about 250 rows at the root (its
// 1,024 random conditioning rows lie at nearly one distance), a few below.
template <int WHICH>
__global__ __launch_bounds__(256) void rb_pivot_kernel(const float* __restrict__ zh, const int32_t* __restrict__ pin,
                                                       const double* __restrict__ cen, const float* __restrict__ dt,
                                                       const double* __restrict__ best_t, int32_t* __restrict__ piv,
                                                       int N, int nb, int level) {
  __shared__ int cand[RB_CAND];
  __shared__ int ncand;
  __shared__ float wm[4];
  __shared__ double wt[4];
  __shared__ int wr[4];
  const int ng = 1 << level;
  const int gi = blockIdx.x % ng;
  const size_t bh = blockIdx.x / ng;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int s, n, sp;
  if (!rb_locate(N, level, gi, s, n, sp)) return;
  if (n <= RB_BLK) return;
  const int c0 = s / RB_BLK, m = (n + RB_BLK - 1) / RB_BLK;
  const size_t g0 = bh * nb + c0;
  if (tid == 0) ncand = 0;
  float mx = -1.f;
  for (int j = tid; j < m; j += 256) mx = fmaxf(mx, (float)best_t[g0 + j]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
  if (lane == 0) wm[wave] = mx;
  __syncthreads();
  const float thr = fmaxf(fmaxf(wm[0], wm[1]), fmaxf(wm[2], wm[3])) - 2.f * RB_FAR_EPS;
  // eight loads in flight per thread; a position is listed once
  const float* dg = dt + bh * N + s;
  for (int j0 = tid; j0 < n; j0 += 8 * 256) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = dg[min(j0 + 256 * u, n - 1)];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (j0 + 256 * u < n && v[u] >= thr) {
        const int x = atomicAdd(&ncand, 1);
        if (x < RB_CAND) cand[x] = j0 + 256 * u;
      }
  }
  __syncthreads();
  const int nc = ncand;
  const float* zb = zh + bh * (size_t)N * RB_HD;
  double v0, v1;
  if (WHICH == 1) {
    const float2 pz = *(const float2*)(zb + (size_t)piv[2 * g0] * RB_HD + 2 * lane);
    v0 = pz.x;
    v1 = pz.y;
  } else {
    v0 = cen[g0 * RB_HD + 2 * lane];
    v1 = cen[g0 * RB_HD + 2 * lane + 1];
  }
  double bt = -1.0;
  int br = 0x7fffffff;
  const int mu = (lane >> 3) & 7;  // the row of each batch of 8 whose sum this lane ends with
  // rows x0 .. x0 + 7 of the list (the candidates, or every position of the
  // group when there are too many): lane u < 8 fetches the row of item x0 + u
  const bool all = nc > RB_CAND;
  const int items = all ? n : nc;
  for (int x0 = 8 * wave; x0 < items; x0 += 32) {
    const int xi = min(x0 + (lane & 7), items - 1);
    const int myrow = pin[bh * N + s + (all ? xi : cand[xi])];
    int r[8];
    float2 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      r[u] = __builtin_amdgcn_readlane(myrow, u);
      v[u] = *(const float2*)(zb + (size_t)r[u] * RB_HD + 2 * lane);
    }
    double d[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const double dx = (double)v[u].x - v0, dy = (double)v[u].y - v1;
      d[u] = dx * dx + dy * dy;
    }
    const double t = rb_wave_sum8(d, lane);
    int rm = r[0];
#pragma unroll
    for (int u = 1; u < 8; ++u) rm = mu == u ? r[u] : rm;
    if (x0 + mu < items && rb_better(t, rm, bt, br)) {
      bt = t;
      br = rm;
    }
  }
  // the wavefront's farthest: a total order, so any pairing gives it
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const double ot = __shfl_xor(bt, off, 64);
    const int orr = __shfl_xor(br, off, 64);
    if (rb_better(ot, orr, bt, br)) {
      bt = ot;
      br = orr;
    }
  }
  if (lane == 0) {
    wt[wave] = bt;
    wr[wave] = br;
  }
  __syncthreads();
  if (tid == 0) {
    for (int w = 1; w < 4; ++w)
      if (rb_better(wt[w], wr[w], bt, br)) {
        bt = wt[w];
        br = wr[w];
      }
    // a row of the head even if no distance compared as a number (non-finite
    // inputs), so that later reads stay inside z
    piv[2 * g0 + WHICH] = min(max(br, 0), N - 1);
  }
}

// One workgroup of 4 wavefronts per (slice, batch x head): the split key of
// each row of the slice, z_i . (z_b - z_a) in float64 rounded to float32,
// as an order-preserving 32-bit key at the row's position.
__global__ __launch_bounds__(256) void rb_keys_kernel(const float* __restrict__ zh, const int32_t* __restrict__ pin,
                                                      const int32_t* __restrict__ piv, uint32_t* __restrict__ keys,
                                                      int N, int nb, int level) {
  const int c = blockIdx.x % nb;
  const size_t bh = blockIdx.x / nb;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int s, n;
  bool right;
  rb_group_of(N, level, c * RB_BLK, s, n, right);
  if (n <= RB_BLK) return;
  const size_t g0 = bh * nb + s / RB_BLK;
  const float* zb = zh + bh * (size_t)N * RB_HD;
  const float2 za = *(const float2*)(zb + (size_t)piv[2 * g0] * RB_HD + 2 * lane);
  const float2 zbb = *(const float2*)(zb + (size_t)piv[2 * g0 + 1] * RB_HD + 2 * lane);
  const double w0 = (double)zbb.x - (double)za.x, w1 = (double)zbb.y - (double)za.y;
  const int p0 = c * RB_BLK, cnt = min(RB_BLK, N - p0);
  const int myrow = pin[bh * N + p0 + min(wave + 4 * (lane & 31), cnt - 1)];
  const int mu = (lane >> 3) & 7;  // the row of each group of 8 rows whose sum this lane ends with
#pragma unroll
  for (int i0 = 0; i0 < 32; i0 += 8) {
    float2 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int r = __builtin_amdgcn_readlane(myrow, i0 + u);
      v[u] = *(const float2*)(zb + (size_t)r * RB_HD + 2 * lane);
    }
    double x[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) x[u] = (double)v[u].x * w0 + (double)v[u].y * w1;
    const double key = rb_wave_sum8(x, lane);
    const int pos = wave + 4 * (i0 + mu);
    if ((lane & 7) == 0 && pos < cnt) keys[bh * N + p0 + pos] = rb_key((float)key);
  }
}

// Groups of at most 1024 rows: one wavefront per group, four per workgroup,
// no workgroup barriers.  Lane l owns positions [l C, l C + C), C <= 16, keys
// and rows in registers; the split value is found bit by bit from the top
// (the smallest key with at least n_left keys at or below it).
constexpr int WS_KPT = 16;

__global__ __launch_bounds__(256) void rb_split_wave_kernel(const uint32_t* __restrict__ keys,
                                                            const int32_t* __restrict__ pin,
                                                            int32_t* __restrict__ pout, int N, int level,
                                                            int total) {
  const int lane = threadIdx.x & 63;
  const int G = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (G >= total) return;
  const int gi = G & ((1 << level) - 1);
  const size_t bh = (size_t)(G >> level);
  int s, n, sp;
  if (!rb_locate(N, level, gi, s, n, sp)) return;
  const int32_t* pi = pin + bh * N + s;
  int32_t* po = pout + bh * N + s;
  const int m = (n + RB_BLK - 1) / RB_BLK;
  if (m <= 1) {
    for (int j = lane; j < n; j += 64) po[j] = pi[j];
    return;
  }
  const int nl = RB_BLK * ((m + 1) / 2);
  const uint32_t* kb = keys + bh * N + s;
  const int C = (n + 63) / 64;
  const int j0 = lane * C;
  int32_t pr[WS_KPT];
  uint32_t kr[WS_KPT];
#pragma unroll
  for (int u = 0; u < WS_KPT; ++u) pr[u] = pi[min(j0 + u, n - 1)];
#pragma unroll
  for (int u = 0; u < WS_KPT; ++u) kr[u] = kb[min(j0 + u, n - 1)];
  auto valid = [&](int u) { return u < C && j0 + u < n; };
  // counts by ballot: no cross-lane data movement
  auto count_le = [&](uint32_t cand) {
    int c = 0;
#pragma unroll
    for (int u = 0; u < WS_KPT; ++u) c += __popcll(__ballot(valid(u) && kr[u] <= cand));
    return c;
  };
  uint32_t Tk = 0u;
  for (int bit = 31; bit >= 0; --bit)
    if (count_le(Tk | ((1u << bit) - 1u)) < nl) Tk |= 1u << bit;
  int lt = 0, eq = 0;
#pragma unroll
  for (int u = 0; u < WS_KPT; ++u) {
    lt += (valid(u) && kr[u] < Tk) ? 1 : 0;
    eq += (valid(u) && kr[u] == Tk) ? 1 : 0;
  }
  const int need = nl - (Tk ? count_le(Tk - 1u) : 0);  // keys equal to Tk that go left, the first in order
  int ilt = lt, ieq = eq;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int ox = __shfl_up(ilt, off, 64), oy = __shfl_up(ieq, off, 64);
    if (lane >= off) {
      ilt += ox;
      ieq += oy;
    }
  }
  lt = ilt - lt;
  eq = ieq - eq;
#pragma unroll
  for (int u = 0; u < WS_KPT; ++u) {
    if (valid(u)) {
      const uint32_t key = kr[u];
      const int before_left = lt + min(eq, need);
      const bool left = key < Tk || (key == Tk && eq < need);
      po[min(left ? before_left : nl + (j0 + u - before_left), n - 1)] = pr[u];
      lt += key < Tk;
      eq += key == Tk;
    }
  }
}

// Larger groups: one workgroup of 1024 threads per group, thread t owning
// positions [t C, t C + C), C <= KPT, keys and rows in registers; the split
// value by an MSB-first radix select, 8 bits a pass.
template <int KPT>
__global__ __launch_bounds__(1024) void rb_split_reg_kernel(const uint32_t* __restrict__ keys,
                                                            const int32_t* __restrict__ pin,
                                                            int32_t* __restrict__ pout, int N, int level) {
  constexpr int T = 1024, W = T / 64;
  __shared__ uint32_t hist[256];
  __shared__ int wt[W][2];
  __shared__ int sh_digit, sh_want;
  const int ng = 1 << level;
  const int gi = blockIdx.x % ng;
  const size_t bh = blockIdx.x / ng;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int s, n, sp;
  if (!rb_locate(N, level, gi, s, n, sp)) return;
  const int32_t* pi = pin + bh * N + s;
  int32_t* po = pout + bh * N + s;
  const int m = (n + RB_BLK - 1) / RB_BLK;
  if (m <= 1) {
    for (int j = tid; j < n; j += T) po[j] = pi[j];
    return;
  }
  const int nl = RB_BLK * ((m + 1) / 2);
  const uint32_t* kbg = keys + bh * N + s;
  const int C = (n + T - 1) / T;
  const int j0 = min(n, tid * C);
  uint32_t kr[KPT];
#pragma unroll
  for (int u = 0; u < KPT; ++u) kr[u] = kbg[(uint32_t)min(j0 + u, n - 1)];
  auto valid = [&](int u) { return u < C && j0 + u < n; };

  uint32_t prefix = 0u, pmask = 0u;
  int want = nl - 1;
  for (int shift = 24; shift >= 0; shift -= 8) {
    if (tid < 256) hist[tid] = 0u;
    __syncthreads();
#pragma unroll
    for (int u = 0; u < KPT; ++u)
      if (valid(u) && (kr[u] & pmask) == prefix) atomicAdd(&hist[(kr[u] >> shift) & 255u], 1u);
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
  const uint32_t Tk = prefix;
  const int need = want + 1;
  int lt = 0, eq = 0;
#pragma unroll
  for (int u = 0; u < KPT; ++u) {
    lt += (valid(u) && kr[u] < Tk) ? 1 : 0;
    eq += (valid(u) && kr[u] == Tk) ? 1 : 0;
  }
  block_scan2<W>(lt, eq, wt, lane, wave);
  // the rows again (all loads in flight together), rather than held in
  // registers through the select
  int32_t pr[KPT];
#pragma unroll
  for (int u = 0; u < KPT; ++u) pr[u] = pi[(uint32_t)min(j0 + u, n - 1)];
#pragma unroll
  for (int u = 0; u < KPT; ++u) {
    if (valid(u)) {
      const uint32_t key = kr[u];
      const int before_left = lt + min(eq, need);
      const bool left = key < Tk || (key == Tk && eq < need);
      po[min(left ? before_left : nl + (j0 + u - before_left), n - 1)] = pr[u];
      lt += key < Tk;
      eq += key == Tk;
    }
  }
}

// The largest groups (more than 20 rows per thread of 1024): one workgroup
// per group, keys in the global key buffer (read from L2 in every pass, eight
// loads in flight), the split value by an MSB-first radix select.
__global__ __launch_bounds__(1024) void rb_split_big_kernel(const uint32_t* __restrict__ keys,
                                                            const int32_t* __restrict__ pin,
                                                            int32_t* __restrict__ pout, int N, int level) {
  constexpr int T = 1024, W = T / 64, U = 8;
  __shared__ uint32_t hist[256];
  __shared__ int wt[W][2];
  __shared__ int sh_digit, sh_want;
  const int ng = 1 << level;
  const int gi = blockIdx.x % ng;
  const size_t bh = blockIdx.x / ng;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int s, n, sp;
  if (!rb_locate(N, level, gi, s, n, sp)) return;
  const int32_t* pi = pin + bh * N + s;
  int32_t* po = pout + bh * N + s;
  const int m = (n + RB_BLK - 1) / RB_BLK;
  if (m <= 1) {
    for (int j = tid; j < n; j += T) po[j] = pi[j];
    return;
  }
  const int nl = RB_BLK * ((m + 1) / 2);
  const uint32_t* kb = keys + bh * N + s;

  uint32_t prefix = 0u, pmask = 0u;
  int want = nl - 1;
  for (int shift = 24; shift >= 0; shift -= 8) {
    if (tid < 256) hist[tid] = 0u;
    __syncthreads();
    for (int j0 = tid; j0 < n; j0 += U * T) {
      uint32_t k8[U];
#pragma unroll
      for (int u = 0; u < U; ++u) k8[u] = kb[(uint32_t)min(j0 + u * T, n - 1)];
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (j0 + u * T < n && (k8[u] & pmask) == prefix) atomicAdd(&hist[(k8[u] >> shift) & 255u], 1u);
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
  const uint32_t Tk = prefix;
  const int need = want + 1;  // keys equal to Tk that go left, the first in order

  // stable partition: thread t takes positions [t C, t C + C), read in
  // batches of eight
  const int C = (n + T - 1) / T;
  const int j0 = min(n, tid * C), j1 = min(n, j0 + C);
  int lt = 0, eq = 0;
  for (int j = j0; j < j1; j += U) {
    uint32_t k8[U];
#pragma unroll
    for (int u = 0; u < U; ++u) k8[u] = kb[(uint32_t)min(j + u, j1 - 1)];
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (j + u < j1) {
        lt += k8[u] < Tk;
        eq += k8[u] == Tk;
      }
  }
  block_scan2<W>(lt, eq, wt, lane, wave);
  for (int j = j0; j < j1; j += U) {
    uint32_t k8[U];
    int32_t r8[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      k8[u] = kb[(uint32_t)min(j + u, j1 - 1)];
      r8[u] = pi[(uint32_t)min(j + u, j1 - 1)];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (j + u < j1) {
        const uint32_t key = k8[u];
        const int before_left = lt + min(eq, need);
        const bool left = key < Tk || (key == Tk && eq < need);
        // the counts place every row inside [0, n); the clamp only keeps a
        // miscount from writing outside the group
        po[min(left ? before_left : nl + (j + u - before_left), n - 1)] = r8[u];
        lt += key < Tk;
        eq += key == Tk;
      }
    }
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
  size_t part, msum, ltw, zh, zl, dt, keys, perm, stats, tot, cen, best_t, piv, total;
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
  if (g->BH * lv_wg * 1024 >= (int64_t(1) << 32)) return BSA_ERR_UNSUPPORTED;
  if (g->BH * g->nb * 256 >= (int64_t(1) << 32)) return BSA_ERR_UNSUPPORTED;
  if (g->BH * ((g->N + 15) / 16) * 256 >= (int64_t(1) << 32)) return BSA_ERR_UNSUPPORTED;
  return BSA_OK;
}

RbLayout rb_layout(const RbGeom& g) {
  RbLayout w{};
  size_t off = 0;
  w.part = off;
  off = rb_align(off + (size_t)g.BH * g.nchunk * RB_HD * RB_HD * sizeof(float));
  w.msum = off;
  off = rb_align(off + (size_t)g.BH * RB_HD * RB_HD * sizeof(double));
  w.ltw = off;
  off = rb_align(off + (size_t)g.BH * 3 * RB_HD * RB_HD * sizeof(uint16_t));
  w.zh = off;
  off = rb_align(off + (size_t)g.BH * g.N * RB_HD * sizeof(float));
  w.zl = off;  // z as float16
  off = rb_align(off + (size_t)g.BH * g.N * RB_HD * sizeof(uint16_t));
  w.dt = off;  // each position's float16 distance from the current reference
  off = rb_align(off + (size_t)g.BH * g.N * sizeof(float));
  w.keys = off;
  off = rb_align(off + (size_t)g.BH * g.N * sizeof(uint32_t));
  w.perm = off;
  off = rb_align(off + (size_t)g.BH * g.N * sizeof(int32_t));
  w.stats = off;  // slice sums of z
  off = rb_align(off + (size_t)g.BH * g.nb * RB_HD * sizeof(double));
  w.tot = off;  // group totals, two levels (by level parity)
  off = rb_align(off + 2 * (size_t)g.BH * g.nb * RB_HD * sizeof(double));
  w.cen = off;  // group centroids
  off = rb_align(off + (size_t)g.BH * g.nb * RB_HD * sizeof(double));
  w.best_t = off;  // each slice's largest float16 distance
  off = rb_align(off + (size_t)g.BH * g.nb * sizeof(double));
  w.piv = off;  // each group's two pivot rows
  off = rb_align(off + (size_t)g.BH * g.nb * 2 * sizeof(int32_t));
  w.total = off;
  return w;
}

bool rb_aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int rb_status() {
  const hipError_t e = hipGetLastError();
  if (e == hipSuccess) return BSA_OK;
  bsa_note_hip_error(e);
  return BSA_ERR_HIP;
}

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
  (void)hipGetLastError();  // an error earlier code left pending is not this call's
  hipStream_t s = (hipStream_t)stream;
  char* ws = (char*)workspace;
  float* part = (float*)(ws + w.part);
  uint16_t* ltw = (uint16_t*)(ws + w.ltw);
  float* zh = (float*)(ws + w.zh);
  uint16_t* zl = (uint16_t*)(ws + w.zl);
  float* dt = (float*)(ws + w.dt);
  uint32_t* keys = (uint32_t*)(ws + w.keys);
  int32_t* tmp = (int32_t*)(ws + w.perm);
  // level l reads buf[l % 2] and writes buf[(l + 1) % 2]; the last level
  // writes the caller's array
  int32_t* buf[2] = {(g.levels % 2 == 0) ? perm : tmp, (g.levels % 2 == 0) ? tmp : perm};
  const int N = (int)g.N;
  hipLaunchKernelGGL(rb_moment_kernel, dim3((unsigned)(g.BH * g.nchunk)), dim3(256), 0, s,
                     (const uint16_t*)k, part, N, g.nchunk);
  double* msum = (double*)(ws + w.msum);
  hipLaunchKernelGGL(rb_msum_kernel, dim3((unsigned)(g.BH * 64)), dim3(256), 0, s, (const float*)part, msum, N,
                     g.nchunk);
  hipLaunchKernelGGL(rb_factor_kernel, dim3((unsigned)g.BH), dim3(1024), 0, s, (const double*)msum, ltw);
  const int ntile = (N + EM_ROWS - 1) / EM_ROWS;
  hipLaunchKernelGGL(rb_embed_kernel, dim3((unsigned)(g.BH * ntile)), dim3(64 * EM_WAVES), 0, s, (const uint16_t*)q,
                     (const uint16_t*)ltw, zh, zl, buf[0], N, ntile);
  double* stats = (double*)(ws + w.stats);
  // level l writes its groups' totals to tot[l % 2] and reads its parents'
  // from tot[(l + 1) % 2]
  double* tot[2] = {(double*)(ws + w.tot), (double*)(ws + w.tot) + (size_t)g.BH * g.nb * RB_HD};
  double* cen = (double*)(ws + w.cen);
  double* best_t = (double*)(ws + w.best_t);
  int32_t* piv = (int32_t*)(ws + w.piv);
  const int nb = (int)g.nb;
  const dim3 slices((unsigned)(g.BH * nb));
  for (int l = 0; l < g.levels; ++l) {
    const int32_t* pin = buf[l & 1];
    int32_t* pout = buf[(l + 1) & 1];
    const dim3 groups((unsigned)(g.BH << l));
    hipLaunchKernelGGL(rb_stats_kernel, slices, dim3(256), 0, s, (const float*)zh, pin, stats, N, nb, l);
    hipLaunchKernelGGL(rb_center_kernel, groups, dim3(RB_HD), 0, s, (const double*)stats,
                       (const double*)tot[(l + 1) & 1], tot[l & 1], cen, N, nb, l);
    hipLaunchKernelGGL(rb_far16_kernel<false>, slices, dim3(256), 0, s, (const uint16_t*)zl, (const float*)zh, pin,
                       (const double*)cen, (const int32_t*)piv, dt, best_t, N, nb, l);
    hipLaunchKernelGGL(rb_pivot_kernel<0>, groups, dim3(256), 0, s, (const float*)zh, pin, (const double*)cen,
                       (const float*)dt, (const double*)best_t, piv, N, nb, l);
    hipLaunchKernelGGL(rb_far16_kernel<true>, slices, dim3(256), 0, s, (const uint16_t*)zl, (const float*)zh, pin,
                       (const double*)cen, (const int32_t*)piv, dt, best_t, N, nb, l);
    hipLaunchKernelGGL(rb_pivot_kernel<1>, groups, dim3(256), 0, s, (const float*)zh, pin, (const double*)cen,
                       (const float*)dt, (const double*)best_t, piv, N, nb, l);
    hipLaunchKernelGGL(rb_keys_kernel, slices, dim3(256), 0, s, (const float*)zh, pin, (const int32_t*)piv, keys, N,
                       nb, l);
    // largest group at this level: 128 ceil(nb / 2^l) rows
    const int64_t largest = (int64_t)RB_BLK * ((g.nb + (int64_t(1) << l) - 1) >> l);
    const int64_t per = (largest + 1023) / 1024;  // rows per thread of a 1024-thread workgroup
    const uint32_t* kc = keys;
    if (largest <= 64 * WS_KPT) {
      const int total = (int)(g.BH << l);
      hipLaunchKernelGGL(rb_split_wave_kernel, dim3((unsigned)((total + 3) / 4)), dim3(256), 0, s, kc, pin, pout, N,
                         l, total);
    } else if (per <= 4) {
      hipLaunchKernelGGL((rb_split_reg_kernel<4>), groups, dim3(1024), 0, s, kc, pin, pout, N, l);
    } else if (per <= 12) {
      hipLaunchKernelGGL((rb_split_reg_kernel<12>), groups, dim3(1024), 0, s, kc, pin, pout, N, l);
    } else if (per <= 20) {
      hipLaunchKernelGGL((rb_split_reg_kernel<20>), groups, dim3(1024), 0, s, kc, pin, pout, N, l);
    } else {
      hipLaunchKernelGGL(rb_split_big_kernel, groups, dim3(1024), 0, s, kc, pin, pout, N, l);
    }
  }
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
  (void)hipGetLastError();  // an error earlier code left pending is not this call's
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
  (void)hipGetLastError();  // an error earlier code left pending is not this call's
  hipLaunchKernelGGL(rb_unpermute_kernel, dim3((unsigned)(g.BH * ntile)), dim3(256), 0, (hipStream_t)stream,
                     (const uint16_t*)x, perm, (uint16_t*)out, (int)g.N, ntile);
  return rb_status();
}

}  // extern "C"
