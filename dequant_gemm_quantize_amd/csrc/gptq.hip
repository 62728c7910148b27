// GPTQ-style second-order INT4 quantization ("Build a GPTQ INT4 Quantization
// Engine in Python/NumPy", Step 3), producing the library's packed format.
//
// Three stages, each an entry point:
//  1. Hessian  H = X^T X / T + 1e-4 * mean(diag(X^T X / T)) * I  from float32
//     calibration rows X [T, K]; products and sums in float64.
//  2. U, the upper-triangular Cholesky factor of H^-1 (U^T U = H^-1), in
//     float64.  No explicit inverse is formed.  With J the reversal of the
//     index order, J H J = L L^T (lower Cholesky) gives H = R R^T with
//     R = J L J upper triangular, so H^-1 = R^-T R^-1 and U = R^-1 =
//     J L^-1 J.  The kernels therefore run a blocked lower Cholesky and a
//     blocked lower-triangular inverse on the reversed view of H, and write
//     L^-1 straight into U at reversed positions.  The view is padded to a
//     multiple of 64 with the identity, which leaves both factors unchanged.
//  3. The column sweep: columns left to right, each quantized with its
//     group's parameters (taken when the sweep reaches the group, from the
//     current values), its error e = (w - w_hat) / U[i, i] propagated into
//     the later columns as w_j -= e * U[i, j].  Columns go in blocks of 128
//     (the lazy-batch form of the method): one kernel runs the sequential
//     part inside a block, one lane per weight row, with U's diagonal block
//     in LDS; a float32 MFMA kernel then applies the block's errors to every
//     later column at once, W[:, b1:] -= E[:, b0:b1] U[b0:b1, b1:].
//
// Integer decisions (codes, zero-points, scales) use the same float32 steps
// as the round-to-nearest quantizer; contraction into FMA is switched off in
// this file, and FMAs are written out where they are meant.
#include <cmath>

#include "w4_common.h"
#include "w4_internal.h"

#pragma clang fp contract(off)

namespace w4 {
namespace {

constexpr int NB = 64;        // factorization tile
constexpr int LDP = NB + 1;   // padded LDS row (float64 elements)
constexpr int CB = 128;       // column block of the sweep

// Element (a, b) of the reversed view of a k x k row-major matrix.
__device__ __forceinline__ int64_t rev(int k, int a, int b) {
  return (int64_t)(k - 1 - a) * k + (k - 1 - b);
}

// ---------------------------------------------------------------------------
// 1. Hessian
// ---------------------------------------------------------------------------
constexpr int HT = 64;   // output tile
constexpr int HS = 32;   // calibration rows per LDS stage

// One 64 x 64 tile of X^T X / T per workgroup, upper tiles only; each is
// also written transposed.  Thread (ty, tx) owns rows ty + 16a, columns
// tx + 16b.  Products of float32 values are exact in float64.
__global__ __launch_bounds__(256) void k_gptq_hessian(const float* __restrict__ x, int64_t t, int k,
                                                      double* __restrict__ h) {
  const int ti = blockIdx.y, tj = blockIdx.x;
  if (ti > tj) return;
  __shared__ float xi[HS][HT];
  __shared__ float xj[HS][HT];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int i0 = ti * HT, j0 = tj * HT;
  double acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = 0.0;
  for (int64_t s0 = 0; s0 < t; s0 += HS) {
    float va[(HS * HT) / 256], vb[(HS * HT) / 256];
#pragma unroll
    for (int r = 0; r < (HS * HT) / 256; ++r) {
      const int e = tid + 256 * r, s = e >> 6, c = e & 63;
      const int64_t ts = s0 + s;
      va[r] = (ts < t && i0 + c < k) ? x[ts * k + i0 + c] : 0.f;
      vb[r] = (ts < t && j0 + c < k) ? x[ts * k + j0 + c] : 0.f;
    }
#pragma unroll
    for (int r = 0; r < (HS * HT) / 256; ++r) {
      const int e = tid + 256 * r, s = e >> 6, c = e & 63;
      xi[s][c] = va[r];
      xj[s][c] = vb[r];
    }
    __syncthreads();
#pragma unroll 4
    for (int s = 0; s < HS; ++s) {
      double av[4], bv[4];
#pragma unroll
      for (int a = 0; a < 4; ++a) av[a] = (double)xi[s][ty + 16 * a];
#pragma unroll
      for (int b = 0; b < 4; ++b) bv[b] = (double)xj[s][tx + 16 * b];
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = fma(av[a], bv[b], acc[a][b]);
    }
    __syncthreads();
  }
  const double td = (double)t;
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int i = i0 + ty + 16 * a, j = j0 + tx + 16 * b;
      if (i < k && j < k) {
        const double v = acc[a][b] / td;
        h[(int64_t)i * k + j] = v;
        if (ti != tj) h[(int64_t)j * k + i] = v;
      }
    }
}

// diag += 1e-4 * mean(diag), one workgroup, fixed summation order.
__global__ __launch_bounds__(1024) void k_gptq_damp(double* __restrict__ h, int k) {
  __shared__ double part[1024];
  const int tid = threadIdx.x;
  double s = 0.0;
  for (int i = tid; i < k; i += 1024) s += h[(int64_t)i * k + i];
  part[tid] = s;
  __syncthreads();
  for (int o = 512; o > 0; o >>= 1) {
    if (tid < o) part[tid] += part[tid + o];
    __syncthreads();
  }
  const double damp = 1e-4 * (part[0] / (double)k);
  for (int i = tid; i < k; i += 1024) h[(int64_t)i * k + i] += damp;
}

// ---------------------------------------------------------------------------
// 2. Blocked Cholesky of the reversed view (in place, lower triangle of the
//    view = upper triangle of h), then the blocked inverse of the factor,
//    written into u at reversed positions.
// ---------------------------------------------------------------------------
__device__ __forceinline__ double view_lower(const double* h, int k, int a, int b) {
  if (a < k && b < k) return h[rev(k, a, b)];
  return a == b ? 1.0 : 0.0;
}

// Factor diagonal tile kb in wave 0 of the calling workgroup (left-looking):
// lane i keeps row i of the tile (given in T, lower part) in registers; at
// step j it forms s_i = A[i][j] - sum_{m<j} L[i][m] L[j][m] with row j of L
// read from Lr (a broadcast), and the pivot is sqrt(s_j).  Every thread of
// the workgroup must call this (it holds the workgroup's barriers).  info
// receives 1 + the original column index of the first pivot that is not
// positive.
__device__ __forceinline__ void diag_factor(double* __restrict__ h, int k, int kb, int* __restrict__ info,
                                            const double (*T)[LDP], double (*Lr)[LDP]) {
  const int i = threadIdx.x & 63, o = kb * NB;
  const bool w0 = threadIdx.x < 64;
  double a[NB];
#pragma unroll
  for (int c = 0; c < NB; ++c) a[c] = (w0 && c <= i) ? T[i][c] : 0.0;
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    if (w0) {
      double s0 = a[j], s1 = 0.0, s2 = 0.0, s3 = 0.0;
#pragma unroll
      for (int m = 0; m < j; ++m) {
        const double l = Lr[j][m];
        if ((m & 3) == 0) s0 = fma(-a[m], l, s0);
        else if ((m & 3) == 1) s1 = fma(-a[m], l, s1);
        else if ((m & 3) == 2) s2 = fma(-a[m], l, s2);
        else s3 = fma(-a[m], l, s3);
      }
      const double s = (s0 + s1) + (s2 + s3);
      const double d = __shfl(s, j, kWave);
      if (i == 0 && !(d > 0.0) && o + j < k && *info == 0) *info = k - (o + j);
      const double r = rsqrt(d);            // pivot sqrt(d) = d r, column scale 1/pivot = r
      if (i == j) a[j] = d * r;
      else if (i > j) a[j] = s * r;
      Lr[i][j] = a[j];
    }
    __syncthreads();
  }
  if (w0 && o + i < k)
#pragma unroll
    for (int c = 0; c < NB; ++c)
      if (c <= i) h[rev(k, o + i, o + c)] = a[c];
}

// The first diagonal tile (later ones are factored by k_chol_update).
__global__ __launch_bounds__(64) void k_chol_diag(double* __restrict__ h, int k, int kb,
                                                  int* __restrict__ info) {
  __shared__ double T[NB][LDP];
  __shared__ double Lr[NB][LDP];
  const int t = threadIdx.x, o = kb * NB;
  if (kb == 0 && t == 0) *info = 0;
#pragma unroll
  for (int r_ = 0; r_ < NB * NB / 64; ++r_) {
    const int e = t + 64 * r_;
    const int r = e / NB, c = e % NB;
    T[r][c] = c <= r ? view_lower(h, k, o + r, o + c) : 0.0;
  }
  __syncthreads();
  diag_factor(h, k, kb, info, T, Lr);
}

// Panel: the tiles below diagonal tile kb, X L_kk^T = A, one tile row per
// workgroup.  Each row is solved by four lanes of one wave; lane `sub` keeps
// the row's columns sub, sub + 4, ... in registers, so every inner product
// is split by m mod 4 and its parts combined with two butterflies.
__global__ __launch_bounds__(256) void k_chol_panel(double* __restrict__ h, int k, int kb) {
  __shared__ double L[NB][LDP];
  __shared__ double rd[NB];
  const int tid = threadIdx.x, r = tid >> 2, sub = tid & 3;
  const int o = kb * NB, ob = (kb + 1 + (int)blockIdx.x) * NB;
  #pragma unroll
  for (int r_ = 0; r_ < NB * NB / 256; ++r_) {
    const int e = tid + 256 * r_;
    const int rr = e / NB, c = e % NB;
    L[rr][c] = c <= rr ? view_lower(h, k, o + rr, o + c) : 0.0;
  }
  __syncthreads();
  if (tid < NB) rd[tid] = 1.0 / L[tid][tid];
  const bool live = ob + r < k;
  double x[NB / 4];
#pragma unroll
  for (int t = 0; t < NB / 4; ++t) {
    const int c = sub + 4 * t;
    x[t] = (live && o + c < k) ? h[rev(k, ob + r, o + c)] : 0.0;
  }
  __syncthreads();
#pragma unroll
  for (int c = 0; c < NB; ++c) {
    double p = 0.0;
#pragma unroll
    for (int t = 0; t < NB / 4; ++t)
      if (4 * t < c) {                       // m = sub + 4t < c, decided per lane below
        const double v = sub + 4 * t < c ? x[t] : 0.0;
        p = fma(v, L[c][sub + 4 * t], p);
      }
    p += __shfl_xor(p, 1, kWave);
    p += __shfl_xor(p, 2, kWave);
    if (sub == (c & 3)) x[c >> 2] = (x[c >> 2] - p) * rd[c];
  }
  if (live)
#pragma unroll
    for (int t = 0; t < NB / 4; ++t) {
      const int c = sub + 4 * t;
      if (o + c < k) h[rev(k, ob + r, o + c)] = x[t];
    }
}

// Trailing update: tile (ib, jb), kb < jb <= ib, minus L_ib,kb L_jb,kb^T.
// The workgroup of tile (kb+1, kb+1) then factors that tile at once (the
// next step's diagonal), while the others are still updating theirs.
__global__ __launch_bounds__(256) void k_chol_update(double* __restrict__ h, int k, int kb,
                                                     int* __restrict__ info) {
  const int ib = kb + 1 + (int)blockIdx.y, jb = kb + 1 + (int)blockIdx.x;
  if (jb > ib) return;
  __shared__ double Li[NB][LDP];
  __shared__ double Lj[NB][LDP];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int o = kb * NB, oi = ib * NB, oj = jb * NB;
  #pragma unroll
  for (int r_ = 0; r_ < NB * NB / 256; ++r_) {
    const int e = tid + 256 * r_;
    const int rr = e / NB, c = e % NB;
    const bool cin = o + c < k;
    Li[rr][c] = (cin && oi + rr < k) ? h[rev(k, oi + rr, o + c)] : 0.0;
    Lj[rr][c] = (cin && oj + rr < k) ? h[rev(k, oj + rr, o + c)] : 0.0;
  }
  __syncthreads();
  double acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = 0.0;
#pragma unroll 4
  for (int c = 0; c < NB; ++c) {
    double av[4], bv[4];
#pragma unroll
    for (int a = 0; a < 4; ++a) av[a] = Li[ty + 16 * a][c];
#pragma unroll
    for (int b = 0; b < 4; ++b) bv[b] = Lj[tx + 16 * b][c];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b) acc[a][b] = fma(av[a], bv[b], acc[a][b]);
  }
  const bool next_diag = ib == kb + 1 && jb == kb + 1;
  if (next_diag) __syncthreads();           // Li is reused for the updated tile
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int r = ty + 16 * a, q = tx + 16 * b;
      if (next_diag) {
        if (q <= r) Li[r][q] = view_lower(h, k, oi + r, oi + q) - acc[a][b];
      } else if (oi + r < k && oj + q < k && (ib != jb || q <= r)) {
        const int64_t p = rev(k, oi + r, oj + q);
        h[p] = h[p] - acc[a][b];
      }
    }
  if (next_diag) {
    __syncthreads();
    diag_factor(h, k, ib, info, Li, Lj);
  }
}

// u = 0: the strictly lower part of U, and the accumulators of the inverse.
__global__ __launch_bounds__(256) void k_zero(double* __restrict__ u, int64_t total) {
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (int64_t)gridDim.x * 256)
    u[e] = 0.0;
}

// Inverse of each diagonal tile of L; thread t solves column t.
__global__ __launch_bounds__(64) void k_trinv_diag(const double* __restrict__ h, double* __restrict__ u,
                                                   int k) {
  __shared__ double L[NB][LDP];
  __shared__ double X[NB][LDP];
  __shared__ double rd[NB];
  const int t = threadIdx.x, o = (int)blockIdx.x * NB;
  #pragma unroll
  for (int r_ = 0; r_ < NB * NB / 64; ++r_) {
    const int e = t + 64 * r_;
    const int rr = e / NB, c = e % NB;
    L[rr][c] = c <= rr ? view_lower(h, k, o + rr, o + c) : 0.0;
  }
  __syncthreads();
  rd[t] = 1.0 / L[t][t];
  __syncthreads();
  for (int r = 0; r < NB; ++r) {
    if (r < t) {
      X[r][t] = 0.0;
      continue;
    }
    double s0 = r == t ? 1.0 : 0.0, s1 = 0.0, s2 = 0.0, s3 = 0.0;
    int m = t;
    for (; m + 4 <= r; m += 4) {
      s0 = fma(-L[r][m], X[m][t], s0);
      s1 = fma(-L[r][m + 1], X[m + 1][t], s1);
      s2 = fma(-L[r][m + 2], X[m + 2][t], s2);
      s3 = fma(-L[r][m + 3], X[m + 3][t], s3);
    }
    for (; m < r; ++m) s0 = fma(-L[r][m], X[m][t], s0);
    X[r][t] = ((s0 + s1) + (s2 + s3)) * rd[r];
  }
  if (o + t < k)
    for (int r = 0; r < NB && o + r < k; ++r) u[rev(k, o + r, o + t)] = X[r][t];
}

// Right-looking inverse: tile (i, j), j < i, of X = L^-1 is
// X_ij = -X_ii B_ij with B_ij = sum_{m=j}^{i-1} L_im X_mj.  B accumulates in
// u at X's place: when block row m is final, every later block row ib gets
// L_ib,m X_m,j added for all j <= m (k_trinv_update, many tiles at once),
// and block row m + 1, now complete, is finished in the same launch.
__device__ __forceinline__ void tile_mma(const double (*A)[LDP], const double (*B)[LDP], int tx, int ty,
                                         double acc[4][4]) {
#pragma unroll 4
  for (int c = 0; c < NB; ++c) {
    double av[4], bv[4];
#pragma unroll
    for (int a = 0; a < 4; ++a) av[a] = A[ty + 16 * a][c];
#pragma unroll
    for (int b = 0; b < 4; ++b) bv[b] = B[c][tx + 16 * b];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b) acc[a][b] = fma(av[a], bv[b], acc[a][b]);
  }
}

// B_ib,j += L_ib,m X_m,j for ib = m+1+blockIdx.y, j = blockIdx.x <= m.  The
// workgroups of block row m+1, whose sums are then complete, finish their
// tile in place: X_m+1,j = -X_m+1,m+1 B_m+1,j.
__global__ __launch_bounds__(256) void k_trinv_update(const double* __restrict__ h, double* __restrict__ u,
                                                      int k, int m) {
  __shared__ double A[NB][LDP];
  __shared__ double B[NB][LDP];
  const int jb = blockIdx.x, ib = m + 1 + (int)blockIdx.y;
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int oi = ib * NB, oj = jb * NB, om = m * NB;
  #pragma unroll
  for (int r_ = 0; r_ < NB * NB / 256; ++r_) {
    const int e = tid + 256 * r_;
    const int rr = e / NB, c = e % NB;
    A[rr][c] = (oi + rr < k && om + c < k) ? h[rev(k, oi + rr, om + c)] : 0.0;
    B[rr][c] = (om + rr < k && oj + c < k) ? u[rev(k, om + rr, oj + c)] : 0.0;
  }
  __syncthreads();
  double acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = 0.0;
  tile_mma(A, B, tx, ty, acc);
  if (ib != m + 1) {
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int r = ty + 16 * a, q = tx + 16 * b;
        if (oi + r < k && oj + q < k) {
          const int64_t p = rev(k, oi + r, oj + q);
          u[p] = u[p] + acc[a][b];
        }
      }
    return;
  }
  __syncthreads();                          // A and B are reused
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int r = ty + 16 * a, q = tx + 16 * b;
      B[r][q] = (oi + r < k && oj + q < k) ? u[rev(k, oi + r, oj + q)] + acc[a][b] : 0.0;
    }
  #pragma unroll
  for (int r_ = 0; r_ < NB * NB / 256; ++r_) {
    const int e = tid + 256 * r_;
    const int rr = e / NB, c = e % NB;
    A[rr][c] = (c <= rr && oi + rr < k && oi + c < k) ? u[rev(k, oi + rr, oi + c)] : 0.0;
  }
  __syncthreads();
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = 0.0;
  tile_mma(A, B, tx, ty, acc);
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int r = ty + 16 * a, q = tx + 16 * b;
      if (oi + r < k && oj + q < k) u[rev(k, oi + r, oj + q)] = -acc[a][b];
    }
}

// ---------------------------------------------------------------------------
// 3. Column sweep
// ---------------------------------------------------------------------------
template <typename TS> __device__ __forceinline__ float stored(float v);
template <> __device__ __forceinline__ float stored<float>(float v) { return v; }
template <> __device__ __forceinline__ float stored<_Float16>(float v) { return (float)(_Float16)v; }

constexpr int SB = 16;   // sub-block of the sweep (columns)
constexpr int SWEEP_THREADS = 256;  // rows per sweep workgroup (one per lane)
constexpr int ULD = CB + 4;  // LDS row of the U tile (floats; 16-byte multiple)

// One column's decision with the group's scale s and zero-point zp: the
// stored code and the dequantized value, in the same float32 steps as the
// round-to-nearest quantizer.
template <bool SYM>
__device__ __forceinline__ float decide(float v, float s, float zp, float& dq) {
  if (SYM) {
    const float q = fminf(fmaxf(rintf(v / s), -8.f), 7.f);
    dq = q * s;
    return q + 8.f;
  }
  const float q = fminf(fmaxf(rintf(v / s + zp), 0.f), 15.f);
  dq = (q - zp) * s;
  return q;
}

// dst = w[b0 + c .. + SB) of this row minus the updates from the block's
// columns [b0, b0 + upto), whose errors e were stored in w already.
__device__ __forceinline__ void load_updated(float (&dst)[SB], const float* wr, int b0, int c, int upto,
                                             const float (*Us)[ULD]) {
#pragma unroll
  for (int q = 0; q < SB / 4; ++q) {
    const f32x4 t = *(const f32x4*)(wr + b0 + c + 4 * q);
#pragma unroll
    for (int j = 0; j < 4; ++j) dst[4 * q + j] = t[j];
  }
  for (int i = 0; i < upto; i += 4) {
    const f32x4 e4 = *(const f32x4*)(wr + b0 + i);
#pragma unroll
    for (int ii = 0; ii < 4; ++ii)
#pragma unroll
      for (int j = 0; j < SB; ++j) dst[j] = fmaf(-e4[ii], Us[i + ii][c + j], dst[j]);
  }
}

// Columns [b0, b0 + bw) of 256 rows per workgroup, one lane per row, U's
// diagonal block in LDS (float32).  The block is walked in sub-blocks of 16
// columns: a sub-block's values are loaded and brought up to date with the
// errors of the block's earlier sub-blocks (read back from w, where they
// were stored), then its columns are quantized one at a time with the
// updates inside the sub-block applied in registers.  The errors replace the
// values in w (the update kernel consumes them), the codes are packed and
// stored per sub-block.
template <bool SYM, typename TS>
__global__ __launch_bounds__(SWEEP_THREADS) void k_gptq_sweep(float* __restrict__ w, const double* __restrict__ u,
                                                   int64_t n, int k, int g, int b0, int bw,
                                                   uint8_t* __restrict__ packed, TS* __restrict__ scales,
                                                   TS* __restrict__ zeros) {
  __shared__ __align__(16) float Us[CB][ULD];
  __shared__ float rdiag[CB];
  const int tid = threadIdx.x;
  constexpr int kPer = CB * CB / 2 / SWEEP_THREADS;   // double2 loads per thread
  static_assert(kPer % 16 == 0, "staging batches");
#pragma unroll
  for (int bt = 0; bt < kPer; bt += 16) {
    double2 d[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int e = tid + SWEEP_THREADS * (bt + r), i = e / (CB / 2), j = 2 * (e % (CB / 2));
      d[r] = (i < bw && j < bw) ? *(const double2*)(u + (int64_t)(b0 + i) * k + b0 + j) : double2{0.0, 0.0};
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int e = tid + SWEEP_THREADS * (bt + r), i = e / (CB / 2), j = 2 * (e % (CB / 2));
      Us[i][j] = (float)d[r].x;
      Us[i][j + 1] = (float)d[r].y;
    }
  }
  __syncthreads();
  for (int i = tid; i < CB; i += SWEEP_THREADS) rdiag[i] = i < bw ? 1.f / Us[i][i] : 0.f;
  __syncthreads();
  const int64_t row = (int64_t)blockIdx.x * SWEEP_THREADS + tid;
  if (row >= n) return;
  float* wr = w + row * k;
  const int ng = k / g;
  float s = 1.f, zp = SYM ? 8.f : 0.f;
  if (b0 % g != 0) {  // a group of more than one block continues here
    s = (float)scales[row * ng + b0 / g];
    zp = (float)zeros[row * ng + b0 / g];
  }
  for (int c0 = 0; c0 < bw; c0 += SB) {
    float v[SB];
    load_updated(v, wr, b0, c0, c0, Us);
    if ((b0 + c0) % g == 0) {
      float hi = v[0], lo = v[0];
#pragma unroll
      for (int j = 1; j < SB; ++j) {
        hi = fmaxf(hi, v[j]);
        lo = fminf(lo, v[j]);
      }
      for (int c2 = c0 + SB; c2 < c0 + g; c2 += SB) {
        float t[SB];
        load_updated(t, wr, b0, c2, c2 < bw ? c0 : 0, Us);
#pragma unroll
        for (int j = 0; j < SB; ++j) {
          hi = fmaxf(hi, t[j]);
          lo = fminf(lo, t[j]);
        }
      }
      float s_st;
      if (SYM) {
        s_st = stored<TS>(fmaxf(hi, -lo) / 7.f);
        if (s_st == 0.f) s_st = 1.f;
        zp = 8.f;
      } else {
        s_st = stored<TS>((hi - lo) / 15.f);
        if (s_st == 0.f) s_st = 1.f;
        zp = fminf(fmaxf(rintf(-lo / s_st), 0.f), 15.f);
      }
      s = s_st;
      scales[row * ng + (b0 + c0) / g] = (TS)s_st;
      zeros[row * ng + (b0 + c0) / g] = (TS)zp;
    }
    uint32_t cw[2] = {0u, 0u};
#pragma unroll
    for (int jj = 0; jj < SB; ++jj) {
      float dq;
      const float q = decide<SYM>(v[jj], s, zp, dq);
      const float e = (v[jj] - dq) * rdiag[c0 + jj];
#pragma unroll
      for (int j2 = jj + 1; j2 < SB; ++j2) v[j2] = fmaf(-e, Us[c0 + jj][c0 + j2], v[j2]);
      v[jj] = e;
      cw[jj >> 3] |= (uint32_t)q << (4 * (jj & 7));
    }
#pragma unroll
    for (int q = 0; q < SB / 4; ++q)
      *(f32x4*)(wr + b0 + c0 + 4 * q) = f32x4{v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]};
    *(u32x2*)(packed + row * (k / 2) + (b0 + c0) / 2) = u32x2{cw[0], cw[1]};
  }
}

// W[:, b1:] -= E[:, b0:b1] * U[b0:b1, b1:] with b1 = b0 + bw, float32 MFMA.
// Workgroup tile 128 rows x 128 columns, four waves of 64 x 64 (2 x 2
// v_mfma_f32_32x32x2f32 tiles), K = bw in LDS stages of 32; the next stage's
// global loads are issued before the current stage's MFMAs, and the output
// tile's current values are loaded up front.
__global__ __launch_bounds__(256) void k_gptq_update(float* __restrict__ w, const double* __restrict__ u,
                                                     int64_t n, int k, int b0, int bw) {
  __shared__ float Es[128][33];
  __shared__ float Ub[32][160];
  const int b1 = b0 + bw;
  const int64_t r0 = (int64_t)blockIdx.x * 128;
  const int c0 = b1 + (int)blockIdx.y * 128;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, wr = wv >> 1, wc = wv & 1;
  const int l32 = lane & 31, lk = lane >> 5;
  // stage loads: E as 4 float4 per thread (row tid/8 + 32j, columns 4 (tid%8)),
  // U as 8 double2 per thread (row tid/64 + 4j, columns 2 (tid%64))
  const int er = tid >> 3, ec = 4 * (tid & 7);
  const int ur = tid >> 6, uc = 2 * (tid & 63);
  f32x4 ev[4];
  double ua[8], ub[8];
  auto load_stage = [&](int kk) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t row = r0 + er + 32 * j;
      ev[j] = row < n ? *(const f32x4*)(w + row * k + b0 + kk + ec) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int col = c0 + uc;
      const double* src = u + (int64_t)(b0 + kk + ur + 4 * j) * k + col;
      if (col < k) {
        const double2 d = *(const double2*)src;
        ua[j] = d.x;
        ub[j] = d.y;
      } else {
        ua[j] = 0.0;
        ub[j] = 0.0;
      }
    }
  };
  f32x16 acc[2][2], wold[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  load_stage(0);
  // the output tile's current values, read while the stages are multiplied
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = r0 + wr * 64 + 32 * i + 8 * (r >> 2) + 4 * lk + (r & 3);
        const int col = c0 + wc * 64 + 32 * j + l32;
        wold[i][j][r] = (row < n && col < k) ? w[row * k + col] : 0.f;
      }
  for (int kk = 0; kk < bw; kk += 32) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int c = 0; c < 4; ++c) Es[er + 32 * j][ec + c] = ev[j][c];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      Ub[ur + 4 * j][uc] = (float)ua[j];
      Ub[ur + 4 * j][uc + 1] = (float)ub[j];
    }
    __syncthreads();
    if (kk + 32 < bw) load_stage(kk + 32);
#pragma unroll
    for (int q = 0; q < 32; q += 2) {
      const float a0 = Es[wr * 64 + l32][q + lk];
      const float a1 = Es[wr * 64 + 32 + l32][q + lk];
      const float bb0 = Ub[q + lk][wc * 64 + l32];
      const float bb1 = Ub[q + lk][wc * 64 + 32 + l32];
      acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a0, bb0, acc[0][0], 0, 0, 0);
      acc[0][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(a0, bb1, acc[0][1], 0, 0, 0);
      acc[1][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a1, bb0, acc[1][0], 0, 0, 0);
      acc[1][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(a1, bb1, acc[1][1], 0, 0, 0);
    }
    __syncthreads();
  }
  // lane holds rows 8(r/4) + 4(lane/32) + r%4, column lane%32 of each 32 x 32 tile
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = r0 + wr * 64 + 32 * i + 8 * (r >> 2) + 4 * lk + (r & 3);
        const int col = c0 + wc * 64 + 32 * j + l32;
        if (row < n && col < k) w[row * k + col] = wold[i][j][r] - acc[i][j][r];
      }
}

template <bool SYM, typename TS>
hipError_t sweep_blocks(float* w, const double* u, int64_t n, int k, int g, uint8_t* packed, void* scales,
                        void* zeros, hipStream_t st) {
  const unsigned rows_wg = (unsigned)((n + SWEEP_THREADS - 1) / SWEEP_THREADS);
  for (int b0 = 0; b0 < k; b0 += CB) {
    const int bw = k - b0 < CB ? k - b0 : CB;
    k_gptq_sweep<SYM, TS><<<rows_wg, SWEEP_THREADS, 0, st>>>(w, u, n, k, g, b0, bw, packed, (TS*)scales, (TS*)zeros);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int rest = k - b0 - bw;
    if (rest > 0) {
      dim3 grid((unsigned)((n + 127) / 128), (unsigned)((rest + 127) / 128));
      k_gptq_update<<<grid, 256, 0, st>>>(w, u, n, k, b0, bw);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

}  // namespace

bool gptq_group_ok(int g) { return g % 32 == 0 && g > 0 && (g <= CB ? CB % g == 0 : g % CB == 0); }

hipError_t launch_gptq_hessian(const float* x, int64_t t, int k, double* h, hipStream_t st) {
  const unsigned nt = (unsigned)((k + HT - 1) / HT);
  k_gptq_hessian<<<dim3(nt, nt), 256, 0, st>>>(x, t, k, h);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  k_gptq_damp<<<1, 1024, 0, st>>>(h, k);
  return hipGetLastError();
}

hipError_t launch_gptq_inverse_cholesky(double* h, int k, double* u, int* info, hipStream_t st) {
  const int nt = (k + NB - 1) / NB;
  hipError_t e;
  k_chol_diag<<<1, 64, 0, st>>>(h, k, 0, info);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  for (int kb = 0; kb + 1 < nt; ++kb) {   // the update of step kb factors diagonal tile kb + 1
    const int rest = nt - kb - 1;
    k_chol_panel<<<rest, 256, 0, st>>>(h, k, kb);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    k_chol_update<<<dim3(rest, rest), 256, 0, st>>>(h, k, kb, info);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  const int64_t total = (int64_t)k * k;
  const int64_t blocks = (total + 255) / 256;
  k_zero<<<(unsigned)(blocks < 8192 ? blocks : 8192), 256, 0, st>>>(u, total);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  k_trinv_diag<<<nt, 64, 0, st>>>(h, u, k);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  for (int m = 0; m + 1 < nt; ++m) {       // step m also finishes block row m + 1
    k_trinv_update<<<dim3(m + 1, nt - m - 1), 256, 0, st>>>(h, u, k, m);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_gptq_quantize_pack(float* w, const double* u, int64_t n, int k, int g, bool symmetric,
                                     uint8_t* packed, void* scales, void* zeros, int sz_dtype,
                                     hipStream_t st) {
  if (symmetric)
    return sz_dtype == W4_F16 ? sweep_blocks<true, _Float16>(w, u, n, k, g, packed, scales, zeros, st)
                              : sweep_blocks<true, float>(w, u, n, k, g, packed, scales, zeros, st);
  return sz_dtype == W4_F16 ? sweep_blocks<false, _Float16>(w, u, n, k, g, packed, scales, zeros, st)
                            : sweep_blocks<false, float>(w, u, n, k, g, packed, scales, zeros, st);
}

}  // namespace w4
