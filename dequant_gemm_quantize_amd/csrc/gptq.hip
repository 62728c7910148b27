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
//     part inside a block, one wave per weight row with the block's 128
//     values in registers and U's diagonal block in LDS; a float32 MFMA
//     kernel then applies the block's errors to every later column at once,
//     W[:, b1:] -= E[:, b0:b1] U[b0:b1, b1:].
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
#pragma unroll
    for (int r = 0; r < (HS * HT) / 256; ++r) {
      const int e = tid + 256 * r, s = e >> 6, c = e & 63;
      const int64_t ts = s0 + s;
      float va = 0.f, vb = 0.f;
      if (ts < t) {
        if (i0 + c < k) va = x[ts * k + i0 + c];
        if (j0 + c < k) vb = x[ts * k + j0 + c];
      }
      xi[s][c] = va;
      xj[s][c] = vb;
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

// Factor the diagonal tile kb (unblocked, in LDS).  info receives 1 + the
// original column index of the first pivot that is not positive.
__global__ __launch_bounds__(256) void k_chol_diag(double* __restrict__ h, int k, int kb,
                                                   int* __restrict__ info) {
  __shared__ double A[NB][LDP];
  const int tid = threadIdx.x, o = kb * NB;
  if (kb == 0 && tid == 0) *info = 0;
  for (int e = tid; e < NB * NB; e += 256) {
    const int r = e / NB, c = e % NB;
    A[r][c] = c <= r ? view_lower(h, k, o + r, o + c) : 0.0;
  }
  __syncthreads();
  for (int j = 0; j < NB; ++j) {
    if (tid == 0) {
      const double d = A[j][j];
      if (!(d > 0.0) && o + j < k && *info == 0) *info = k - (o + j);
      A[j][j] = sqrt(d);
    }
    __syncthreads();
    const double piv = A[j][j];
    if (tid > j && tid < NB) A[tid][j] = A[tid][j] / piv;
    __syncthreads();
    for (int e = tid; e < NB * NB; e += 256) {
      const int r = e / NB, c = e % NB;
      if (c > j && c <= r) A[r][c] = fma(-A[r][j], A[c][j], A[r][c]);
    }
    __syncthreads();
  }
  for (int e = tid; e < NB * NB; e += 256) {
    const int r = e / NB, c = e % NB;
    if (c <= r && o + r < k) h[rev(k, o + r, o + c)] = A[r][c];
  }
}

// Panel: the tiles below diagonal tile kb, X L_kk^T = A, one tile row per
// workgroup, one row of it per thread.
__global__ __launch_bounds__(64) void k_chol_panel(double* __restrict__ h, int k, int kb) {
  __shared__ double L[NB][LDP];
  __shared__ double X[NB][LDP];
  const int r = threadIdx.x, o = kb * NB, ob = (kb + 1 + (int)blockIdx.x) * NB;
  for (int e = r; e < NB * NB; e += 64) {
    const int rr = e / NB, c = e % NB;
    L[rr][c] = c <= rr ? view_lower(h, k, o + rr, o + c) : 0.0;
    X[rr][c] = (ob + rr < k && o + c < k) ? h[rev(k, ob + rr, o + c)] : 0.0;
  }
  __syncthreads();
  for (int c = 0; c < NB; ++c) {
    double s0 = X[r][c], s1 = 0.0, s2 = 0.0, s3 = 0.0;
    int m = 0;
    for (; m + 4 <= c; m += 4) {
      s0 = fma(-X[r][m], L[c][m], s0);
      s1 = fma(-X[r][m + 1], L[c][m + 1], s1);
      s2 = fma(-X[r][m + 2], L[c][m + 2], s2);
      s3 = fma(-X[r][m + 3], L[c][m + 3], s3);
    }
    for (; m < c; ++m) s0 = fma(-X[r][m], L[c][m], s0);
    X[r][c] = ((s0 + s1) + (s2 + s3)) / L[c][c];
  }
  if (ob + r < k)
    for (int c = 0; c < NB && o + c < k; ++c) h[rev(k, ob + r, o + c)] = X[r][c];
}

// Trailing update: tile (ib, jb), kb < jb <= ib, minus L_ib,kb L_jb,kb^T.
__global__ __launch_bounds__(256) void k_chol_update(double* __restrict__ h, int k, int kb) {
  const int ib = kb + 1 + (int)blockIdx.y, jb = kb + 1 + (int)blockIdx.x;
  if (jb > ib) return;
  __shared__ double Li[NB][LDP];
  __shared__ double Lj[NB][LDP];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int o = kb * NB, oi = ib * NB, oj = jb * NB;
  for (int e = tid; e < NB * NB; e += 256) {
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
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int r = ty + 16 * a, q = tx + 16 * b;
      if (oi + r < k && oj + q < k && (ib != jb || q <= r)) {
        const int64_t p = rev(k, oi + r, oj + q);
        h[p] = h[p] - acc[a][b];
      }
    }
}

// Strictly lower part of U (never written by the inverse kernels) = 0.
__global__ __launch_bounds__(256) void k_zero_lower(double* __restrict__ u, int k) {
  const int64_t total = (int64_t)k * k;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (int64_t)gridDim.x * 256) {
    const int64_t i = e / k, j = e - i * k;
    if (i > j) u[e] = 0.0;
  }
}

// Inverse of each diagonal tile of L; thread t solves column t.
__global__ __launch_bounds__(64) void k_trinv_diag(const double* __restrict__ h, double* __restrict__ u,
                                                   int k) {
  __shared__ double L[NB][LDP];
  __shared__ double X[NB][LDP];
  const int t = threadIdx.x, o = (int)blockIdx.x * NB;
  for (int e = t; e < NB * NB; e += 64) {
    const int rr = e / NB, c = e % NB;
    L[rr][c] = c <= rr ? view_lower(h, k, o + rr, o + c) : 0.0;
  }
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
    X[r][t] = ((s0 + s1) + (s2 + s3)) / L[r][r];
  }
  if (o + t < k)
    for (int r = 0; r < NB && o + r < k; ++r) u[rev(k, o + r, o + t)] = X[r][t];
}

// Tile (ib, jb), jb < ib, of L^-1:  X_ij = -X_ii * sum_{m=jb}^{ib-1} L_im X_mj.
__global__ __launch_bounds__(256) void k_trinv_row(const double* __restrict__ h, double* __restrict__ u,
                                                   int k, int ib) {
  __shared__ double A[NB][LDP];
  __shared__ double B[NB][LDP];
  const int jb = blockIdx.x;
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int oi = ib * NB, oj = jb * NB;
  double acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = 0.0;
  for (int mb = jb; mb < ib; ++mb) {
    const int om = mb * NB;
    for (int e = tid; e < NB * NB; e += 256) {
      const int rr = e / NB, c = e % NB;
      A[rr][c] = (oi + rr < k && om + c < k) ? h[rev(k, oi + rr, om + c)] : 0.0;
      B[rr][c] = (om + rr < k && oj + c < k) ? u[rev(k, om + rr, oj + c)] : 0.0;
    }
    __syncthreads();
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
    __syncthreads();
  }
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) A[ty + 16 * a][tx + 16 * b] = acc[a][b];
  for (int e = tid; e < NB * NB; e += 256) {
    const int rr = e / NB, c = e % NB;
    B[rr][c] = (c <= rr && oi + rr < k && oi + c < k) ? u[rev(k, oi + rr, oi + c)] : 0.0;
  }
  __syncthreads();
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = 0.0;
#pragma unroll 4
  for (int c = 0; c < NB; ++c) {
    double av[4], bv[4];
#pragma unroll
    for (int a = 0; a < 4; ++a) av[a] = B[ty + 16 * a][c];
#pragma unroll
    for (int b = 0; b < 4; ++b) bv[b] = A[c][tx + 16 * b];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b) acc[a][b] = fma(av[a], bv[b], acc[a][b]);
  }
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

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}
__device__ __forceinline__ float wave_min(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fminf(v, __shfl_xor(v, o, kWave));
  return v;
}

// Columns [b0, b0 + bw) of every row: one wave per row, lane l holding
// columns b0 + l and b0 + 64 + l.  On exit the block's columns of w hold the
// scaled errors e, which the update kernel consumes.
template <bool SYM, typename TS>
__global__ __launch_bounds__(1024) void k_gptq_sweep(float* __restrict__ w, const double* __restrict__ u,
                                                     int64_t n, int k, int g, int b0, int bw,
                                                     uint8_t* __restrict__ packed, TS* __restrict__ scales,
                                                     TS* __restrict__ zeros) {
  __shared__ float Us[CB][CB];
  const int tid = threadIdx.x;
  for (int e = tid; e < CB * CB; e += 1024) {
    const int i = e / CB, j = e % CB;
    Us[i][j] = (i < bw && j < bw) ? (float)u[(int64_t)(b0 + i) * k + b0 + j] : 0.f;
  }
  __syncthreads();
  const int lane = tid & 63;
  const int64_t row = (int64_t)blockIdx.x * 16 + (tid >> 6);
  if (row >= n) return;
  float* wr = w + row * k;
  const int ng = k / g;
  float v0 = lane < bw ? wr[b0 + lane] : 0.f;
  float v1 = 64 + lane < bw ? wr[b0 + 64 + lane] : 0.f;
  int c0 = 0, c1 = 0;
  float s = 1.f, zp = SYM ? 8.f : 0.f;
  if (b0 % g != 0) {  // a group of more than one block continues here
    s = (float)scales[row * ng + b0 / g];
    zp = (float)zeros[row * ng + b0 / g];
  }
  for (int i = 0; i < bw; ++i) {
    if ((b0 + i) % g == 0) {
      const bool in0 = lane >= i && lane < i + g;
      const bool in1 = 64 + lane >= i && 64 + lane < i + g;
      float hi = -INFINITY, lo = INFINITY;
      if (in0) { hi = v0; lo = v0; }
      if (in1) { hi = fmaxf(hi, v1); lo = fminf(lo, v1); }
      for (int c = b0 + bw + lane; c < b0 + g; c += 64) {
        const float v = wr[c];
        hi = fmaxf(hi, v);
        lo = fminf(lo, v);
      }
      hi = wave_max(hi);
      lo = wave_min(lo);
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
      if (lane == 0) {
        scales[row * ng + (b0 + i) / g] = (TS)s_st;
        zeros[row * ng + (b0 + i) / g] = (TS)zp;
      }
    }
    const float src = i < 64 ? v0 : v1;
    const float v = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(src), i & 63));
    float q, dq;
    if (SYM) {
      q = fminf(fmaxf(rintf(v / s), -8.f), 7.f);
      dq = q * s;
      q = q + 8.f;
    } else {
      q = fminf(fmaxf(rintf(v / s + zp), 0.f), 15.f);
      dq = (q - zp) * s;
    }
    const float e = (v - dq) / Us[i][i];
    v0 = fmaf(-e, Us[i][lane], v0);
    v1 = fmaf(-e, Us[i][64 + lane], v1);
    if (lane == (i & 63)) {
      if (i < 64) {
        v0 = e;
        c0 = (int)q;
      } else {
        v1 = e;
        c1 = (int)q;
      }
    }
  }
  if (lane < bw) wr[b0 + lane] = v0;
  if (64 + lane < bw) wr[b0 + 64 + lane] = v1;
  const int h0 = __shfl_down(c0, 1, kWave), h1 = __shfl_down(c1, 1, kWave);
  uint8_t* pr = packed + row * (k / 2);
  if ((lane & 1) == 0) {
    if (lane < bw) pr[(b0 + lane) / 2] = (uint8_t)(c0 | (h0 << 4));
    if (64 + lane < bw) pr[(b0 + 64 + lane) / 2] = (uint8_t)(c1 | (h1 << 4));
  }
}

// W[:, b1:] -= E[:, b0:b1] * U[b0:b1, b1:] with b1 = b0 + bw, float32 MFMA.
// Workgroup tile 128 rows x 128 columns, four waves of 64 x 64 (2 x 2
// v_mfma_f32_32x32x2f32 tiles), K = bw in LDS stages of 32.
__global__ __launch_bounds__(256) void k_gptq_update(float* __restrict__ w, const double* __restrict__ u,
                                                     int64_t n, int k, int b0, int bw) {
  __shared__ float Es[128][33];
  __shared__ float Ub[32][160];
  const int b1 = b0 + bw;
  const int64_t r0 = (int64_t)blockIdx.x * 128;
  const int c0 = b1 + (int)blockIdx.y * 128;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, wr = wv >> 1, wc = wv & 1;
  const int l32 = lane & 31, lk = lane >> 5;
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  for (int kk = 0; kk < bw; kk += 32) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int e = tid + 256 * r, rr = e >> 5, c = e & 31;
      const int64_t row = r0 + rr;
      Es[rr][c] = row < n ? w[row * k + b0 + kk + c] : 0.f;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int e = tid + 256 * r, rr = e >> 7, c = e & 127;
      const int col = c0 + c;
      Ub[rr][c] = col < k ? (float)u[(int64_t)(b0 + kk + rr) * k + col] : 0.f;
    }
    __syncthreads();
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
        if (row < n && col < k) w[row * k + col] -= acc[i][j][r];
      }
}

template <bool SYM, typename TS>
hipError_t sweep_blocks(float* w, const double* u, int64_t n, int k, int g, uint8_t* packed, void* scales,
                        void* zeros, hipStream_t st) {
  const unsigned rows_wg = (unsigned)((n + 15) / 16);
  for (int b0 = 0; b0 < k; b0 += CB) {
    const int bw = k - b0 < CB ? k - b0 : CB;
    k_gptq_sweep<SYM, TS><<<rows_wg, 1024, 0, st>>>(w, u, n, k, g, b0, bw, packed, (TS*)scales, (TS*)zeros);
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
  for (int kb = 0; kb < nt; ++kb) {
    k_chol_diag<<<1, 256, 0, st>>>(h, k, kb, info);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const int rest = nt - kb - 1;
    if (rest > 0) {
      k_chol_panel<<<rest, 64, 0, st>>>(h, k, kb);
      if ((e = hipGetLastError()) != hipSuccess) return e;
      k_chol_update<<<dim3(rest, rest), 256, 0, st>>>(h, k, kb);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
  }
  const int64_t total = (int64_t)k * k;
  const int64_t blocks = (total + 255) / 256;
  k_zero_lower<<<(unsigned)(blocks < 4096 ? blocks : 4096), 256, 0, st>>>(u, k);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  k_trinv_diag<<<nt, 64, 0, st>>>(h, u, k);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  for (int ib = 1; ib < nt; ++ib) {
    k_trinv_row<<<ib, 256, 0, st>>>(h, u, k, ib);
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
