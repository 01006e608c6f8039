// Offline weight preparation of svdq_w4a4 (int4, nvfp4) and awq_w4a16 layers on the
// GPU: the step before
// the layer runs (infolabhq tutorial, section on quantizing your own model; Diffusers
// docs "Nunchaku Lite" introduction: calibrate, SVDQuant, package).  The pages give
// no formulas; the readings, as in the CPU reference of this repository:
//
//   m_k   = bf16(fl32(1 / sqrt(max(amax_k(X_cal), 1e-5))))      smoothing, per channel
//   What  = W / m  (float64, per input row k)
//   What ~ L1 L2, L1 = U_r S_r [K, r], L2 = V_r^T [r, N]: a top-r factorization, each
//          column of L1 signed so its largest-magnitude entry is positive, then bf16
//   R     = What - L1_bf16 L2_bf16  (float64, stored as float32)
//   R quantized per output column in groups of 64 along K: s = bf16(fl32(amax / 7)),
//   q = round-half-even(R / s) in [-8, 7]; or NVFP4: g_w = fl32(amax|R| / 2688), E4M3
//   block scales and E2M1 codes per 16 (the activation quantizer's rule), and the
//   static activation scale g_x = fl32(amax|bf16(x_cal m)| / 2688);
//   AWQ (no smoothing, no factorization): asymmetric uint4 per column and group of 64.
//
// The factorization is a randomized subspace iteration (Halko, Martinsson and Tropp,
// "Finding structure with randomness", 2011: the randomized range finder with power
// iterations, Algorithms 4.3/4.4, and the direct SVD of the projected matrix,
// Algorithm 5.1), all in float64:
//   Y = What Omega (Omega [N, l] Gaussian, an input), Q = orth(Y);
//   repeat p times: Q = orth(What orth(What^T Q));
//   B = Q^T What [l, N];  B B^T = Ub diag(S^2) Ub^T (Jacobi, one workgroup);
//   L1 = Q Ub_r diag(S_r),  L2 = diag(1 / S_r) Ub_r^T B.
// orth() is CholeskyQR2: G = Y^T Y = R^T R (Cholesky, one workgroup), Y = Y R^-1,
// twice.  It is not the exact SVD: L1 L2 is the projection of What on an l-dimensional
// subspace found by p power iterations, whose residual approaches the optimal one
// (Eckart-Young) as p grows.
#include <algorithm>
#include <cmath>

#include "common.h"
#include "kernels.h"
#include "nvfp4_device.h"

namespace svdq {

namespace {

constexpr int kMaxL = 64;  // l = rank + oversampling

// Channel amax of the calibration activations over the rows [z rc, (z + 1) rc) of chunk
// z = blockIdx.y: two channels per thread (32-bit loads, coalesced over k), written to
// part[z][K].  K is even.
__global__ void __launch_bounds__(256)
k_prep_amax_part(const uint16_t* __restrict__ xc, int64_t Mc, int K, int64_t rc,
                 float* __restrict__ part) {
  const int k = 2 * (blockIdx.x * 256 + threadIdx.x);
  if (k >= K) return;
  const int64_t r0 = blockIdx.y * rc, r1 = min(Mc, r0 + rc);
  float a0 = 0.f, a1 = 0.f;
  for (int64_t i = r0; i < r1; ++i) {
    const uint32_t v = *reinterpret_cast<const uint32_t*>(xc + i * K + k);
    a0 = fmaxf(a0, fabsf(bf16_to_f32(v & 0xFFFFu)));
    a1 = fmaxf(a1, fabsf(bf16_to_f32(v >> 16)));
  }
  part[(int64_t)blockIdx.y * K + k] = a0;
  part[(int64_t)blockIdx.y * K + k + 1] = a1;
}

// m_k = bf16(1 / sqrt(max(amax_k, 1e-5))) from the nz chunk maxima (a maximum does not
// depend on the order it is taken in).
__global__ void __launch_bounds__(256)
k_prep_smooth(const float* __restrict__ part, int nz, int K, uint16_t* __restrict__ m) {
  const int k = blockIdx.x * 256 + threadIdx.x;
  if (k >= K) return;
  float a = 0.f;
  for (int z = 0; z < nz; ++z) a = fmaxf(a, part[(int64_t)z * K + k]);
  const double lam = sqrt(fmax((double)a, 1e-5));
  m[k] = (uint16_t)f32_to_bf16_rne((float)(1.0 / lam));
}

// What[k][n] = W[k][n] / m_k in float64.
__global__ void __launch_bounds__(256)
k_prep_what(const float* __restrict__ w, const uint16_t* __restrict__ m, double* __restrict__ wh,
            int K, int N) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)K * N) return;
  wh[i] = (double)w[i] / (double)bf16_to_f32(m[i / N]);
}

// C[i][j] = sum_k A(i, k) B(k, j), float64, A(i, k) = A[i * as0 + k * as1],
// B(k, j) = B[k * bs0 + j * bs1], C row-major with leading dimension ldc.  64 x 64
// tiles, 16 values of k per step through LDS, 4 x 4 outputs per thread, k summed in
// ascending order.  Workgroup z takes k in [z kc, (z + 1) kc) and writes its partial
// product to C + z cz (one chunk: cz = 0, kc >= K).
__global__ void __launch_bounds__(256)
k_gemm_f64(const double* __restrict__ A, int64_t as0, int64_t as1, const double* __restrict__ B,
           int64_t bs0, int64_t bs1, double* __restrict__ C, int64_t ldc, int M, int N, int K,
           int kc, int64_t cz) {
  __shared__ double As[16][65], Bs[16][65];
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const int i0 = blockIdx.y * 64, j0 = blockIdx.x * 64;
  const int kbeg = blockIdx.z * kc, kend = min(K, kbeg + kc);
  C += blockIdx.z * cz;
  double c[4][4] = {};
  for (int k0 = kbeg; k0 < kend; k0 += 16) {
    for (int e = threadIdx.x; e < 16 * 64; e += 256) {
      const int kk = e >> 6, ii = e & 63;
      const int gi = i0 + ii, gk = k0 + kk;
      As[kk][ii] = (gi < M && gk < kend) ? A[gi * as0 + gk * as1] : 0.0;
      const int gj = j0 + ii;
      Bs[kk][ii] = (gj < N && gk < kend) ? B[gk * bs0 + gj * bs1] : 0.0;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk)
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) c[a][b] = fma(As[kk][ty + 16 * a], Bs[kk][tx + 16 * b], c[a][b]);
    __syncthreads();
  }
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int gi = i0 + ty + 16 * a, gj = j0 + tx + 16 * b;
      if (gi < M && gj < N) C[gi * ldc + gj] = c[a][b];
    }
}

// C[i][j] = sum_z P[z][i][j] over nz partial products [M][N], z ascending.
__global__ void __launch_bounds__(256)
k_sum_parts(const double* __restrict__ P, int nz, int M, int N, double* __restrict__ C, int64_t ldc) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= (int64_t)M * N) return;
  double v = 0.0;
#pragma unroll 8
  for (int z = 0; z < nz; ++z) v += P[z * (int64_t)M * N + e];
  C[(e / N) * ldc + e % N] = v;
}

// Lane `src` of v, broadcast to the wave (src a compile-time constant in the unrolled
// loops below).
__device__ __forceinline__ double lane_bcast(double v, int src) {
  const uint64_t u = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, src);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), src);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// Cholesky G = R^T R of an l x l Gram matrix, then Rinv = R^-1 (upper triangular), in
// one wave with lane c holding column c in registers.  The matrix is padded to LP >= l
// with an identity block, which factors to itself and leaves R and R^-1 of G unchanged.
// Right-looking factorization: at step j the pivot comes from lane j, row j of R is each
// lane's element j over the pivot, and the trailing matrix loses R[j][b] R[j][c]
// (row j of R staged in LDS and read back as broadcasts).  The inverse overwrites column
// c from the bottom: X[i][c] = (delta_ic - sum_{k>i} R[i][k] X[k][c]) / R[i][i], row i of
// R staged in LDS the same way before column c's element i is replaced; entries below the
// diagonal come out zero.  A non-positive pivot sets *fail (and is replaced by 1 so the kernel finishes).
template <int LP>
__global__ void __launch_bounds__(64)
k_chol_inv(const double* __restrict__ G, int l, double* __restrict__ Rinv, int* __restrict__ fail) {
  __shared__ double row[LP];
  const int c = threadIdx.x;
  double a[LP];
#pragma unroll
  for (int i = 0; i < LP; ++i) a[i] = (c < l && i < l) ? G[i * l + c] : (i == c ? 1.0 : 0.0);
  bool bad = false;
#pragma unroll
  for (int j = 0; j < LP; ++j) {
    const double d = lane_bcast(a[j], j);
    bad |= !(d > 0.0);
    const double piv = d > 0.0 ? sqrt(d) : 1.0;
    const double r = c == j ? piv : a[j] / piv;
    a[j] = r;
    if (c < LP) row[c] = r;
    __syncthreads();
#pragma unroll
    for (int b = j + 1; b < LP; ++b) a[b] = fma(-row[b], r, a[b]);
    __syncthreads();
  }
#pragma unroll
  for (int i = LP - 1; i >= 0; --i) {
    if (c < LP) row[c] = a[i];
    __syncthreads();
    double v = i == c ? 1.0 : 0.0;
#pragma unroll
    for (int k = i + 1; k < LP; ++k) v = fma(-row[k], a[k], v);
    a[i] = v / row[i];
    __syncthreads();
  }
  if (c < l)
#pragma unroll
    for (int i = 0; i < LP; ++i)
      if (i < l) Rinv[i * l + c] = a[i];
  if (c == 0 && bad) atomicOr(fail, 1);
}

// Eigen-decomposition of a symmetric l x l matrix C (one workgroup) by Jacobi
// rotations in the parallel round-robin ordering (Brent and Luk, "The solution of
// singular-value and symmetric eigenvalue problems on multiprocessor arrays", 1985;
// Golub and Van Loan, Matrix Computations, parallel Jacobi): each sweep has n - 1
// rounds of n / 2 disjoint pairs (n = l rounded up to even; pairs with the padding
// index are skipped), whose rotations are computed from the same matrix and applied
// together, columns then rows.  Sweeps stop once the off-diagonal mass is below 1e-30
// of the total.  Output: eigenvalues descending in ev[l], eigenvectors in the columns
// of V [l][l].
__global__ void __launch_bounds__(256)
k_jacobi(const double* __restrict__ C, int l, double* __restrict__ ev, double* __restrict__ V) {
  __shared__ double A[kMaxL][kMaxL + 1], Q[kMaxL][kMaxL + 1];
  __shared__ double rc[kMaxL / 2], rs[kMaxL / 2];
  __shared__ int rp[kMaxL / 2], rq[kMaxL / 2];
  __shared__ double roff[256], rtot[256];
  const int t = threadIdx.x;
  const int n = l + (l & 1), np = n / 2;
  for (int e = t; e < l * l; e += 256) {
    A[e / l][e % l] = C[e];
    Q[e / l][e % l] = (e / l == e % l) ? 1.0 : 0.0;
  }
  __syncthreads();
  for (int sweep = 0; sweep < 40; ++sweep) {
    {  // off-diagonal and total squared mass: strided partial sums, then a tree
      double o = 0.0, sum = 0.0;
      for (int e = t; e < l * l; e += 256) {
        const int a = e / l, b = e % l;
        const double v = A[a][b] * A[a][b];
        sum += v;
        if (a != b) o += v;
      }
      roff[t] = o;
      rtot[t] = sum;
      __syncthreads();
      for (int h = 128; h > 0; h >>= 1) {
        if (t < h) {
          roff[t] += roff[t + h];
          rtot[t] += rtot[t + h];
        }
        __syncthreads();
      }
    }
    const bool done = !(roff[0] > 1e-30 * rtot[0]);
    __syncthreads();
    if (done) break;
    for (int round = 0; round < n - 1; ++round) {
      if (t < np) {
        // players: position 0 fixed, positions 1 .. n-1 rotate; pair t = (pos t, pos n-1-t)
        auto player = [&](int pos) { return pos == 0 ? 0 : 1 + (pos - 1 + round) % (n - 1); };
        int p = player(t), q = player(n - 1 - t);
        if (p > q) {
          const int x = p;
          p = q;
          q = x;
        }
        double c = 1.0, sn = 0.0;
        if (q < l && A[p][q] != 0.0) {
          const double apq = A[p][q];
          const double theta = (A[q][q] - A[p][p]) / (2.0 * apq);
          const double tt = (theta >= 0.0 ? 1.0 : -1.0) / (fabs(theta) + sqrt(theta * theta + 1.0));
          c = 1.0 / sqrt(tt * tt + 1.0);
          sn = tt * c;
        }
        rp[t] = p;
        rq[t] = q < l ? q : p;  // a skipped pair rotates nothing
        rc[t] = c;
        rs[t] = q < l ? sn : 0.0;
      }
      __syncthreads();
      // columns: A = A J, Q = Q J
      for (int i = t >> 6, k = t & 63; i < np && k < l; i += 4) {
        const double c = rc[i], sn = rs[i];
        if (sn != 0.0) {
          const int p = rp[i], q = rq[i];
          const double akp = A[k][p], akq = A[k][q];
          A[k][p] = c * akp - sn * akq;
          A[k][q] = sn * akp + c * akq;
          const double qkp = Q[k][p], qkq = Q[k][q];
          Q[k][p] = c * qkp - sn * qkq;
          Q[k][q] = sn * qkp + c * qkq;
        }
      }
      __syncthreads();
      // rows: A = J^T A
      for (int i = t >> 6, k = t & 63; i < np && k < l; i += 4) {
        const double c = rc[i], sn = rs[i];
        if (sn != 0.0) {
          const int p = rp[i], q = rq[i];
          const double apk = A[p][k], aqk = A[q][k];
          A[p][k] = c * apk - sn * aqk;
          A[q][k] = sn * apk + c * aqk;
        }
      }
      __syncthreads();
    }
  }
  // sort descending (selection, one thread), move vectors along
  if (t == 0) {
    int idx[kMaxL];
    for (int a = 0; a < l; ++a) idx[a] = a;
    for (int a = 0; a < l; ++a) {
      int best = a;
      for (int b = a + 1; b < l; ++b)
        if (A[idx[b]][idx[b]] > A[idx[best]][idx[best]]) best = b;
      const int tmp = idx[a];
      idx[a] = idx[best];
      idx[best] = tmp;
    }
    for (int a = 0; a < l; ++a) {
      ev[a] = A[idx[a]][idx[a]];
      for (int k = 0; k < l; ++k) V[k * l + a] = Q[k][idx[a]];
    }
  }
}

// M1 = Ub_r diag(S_r) [l][r] and M2 = diag(1 / S_r) Ub_r^T [r][l] from the eigenpairs
// of B B^T (S = sqrt of the eigenvalue).  A non-positive eigenvalue among the top r
// sets *fail.
__global__ void k_prep_small(const double* __restrict__ ev, const double* __restrict__ V, int l,
                             int r, double* __restrict__ M1, double* __restrict__ M2,
                             int* __restrict__ fail) {
  const int t = threadIdx.x;
  for (int e = t; e < l * r; e += blockDim.x) {
    const int a = e / r, j = e % r;
    const double lam = ev[j];
    const double s = lam > 0.0 ? sqrt(lam) : 0.0;
    M1[a * r + j] = V[a * l + j] * s;
    M2[j * l + a] = s > 0.0 ? V[a * l + j] / s : 0.0;
  }
  if (t == 0)
    for (int j = 0; j < r; ++j)
      if (!(ev[j] > 0.0)) atomicOr(fail, 2);
}

// Sign of column j of L1 [K][r]: the entry of largest magnitude (first one on ties)
// made positive; the bf16 factors lora_down [r][K] = L1^T and lora_up [N][r] = L2^T.
__global__ void __launch_bounds__(256)
k_prep_sign(const double* __restrict__ L1, int K, int r, int* __restrict__ sgn) {
  __shared__ double bv[256];
  __shared__ int bi[256];
  const int j = blockIdx.x, t = threadIdx.x;
  double best = -1.0;
  int bidx = K;
  for (int k = t; k < K; k += 256) {
    const double v = fabs(L1[(size_t)k * r + j]);
    if (v > best) {
      best = v;
      bidx = k;
    }
  }
  bv[t] = best;
  bi[t] = bidx;
  __syncthreads();
  for (int h = 128; h > 0; h >>= 1) {
    if (t < h) {
      const double o = bv[t + h];
      const int oi = bi[t + h];
      if (o > bv[t] || (o == bv[t] && oi < bi[t])) {
        bv[t] = o;
        bi[t] = oi;
      }
    }
    __syncthreads();
  }
  if (t == 0) sgn[j] = L1[(size_t)bi[0] * r + j] < 0.0 ? -1 : 1;
}

__global__ void __launch_bounds__(256)
k_prep_factors(const double* __restrict__ L1, const double* __restrict__ L2,
               const int* __restrict__ sgn, int K, int N, int r, uint16_t* __restrict__ ldown,
               uint16_t* __restrict__ lup) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < (int64_t)K * r) {  // lora_down[j][k] = sign_j L1[k][j]
    const int j = (int)(i / K), k = (int)(i % K);
    ldown[i] = (uint16_t)f32_to_bf16_rne((float)(sgn[j] * L1[(size_t)k * r + j]));
  }
  if (i < (int64_t)N * r) {  // lora_up[n][j] = sign_j L2[j][n]
    const int n = (int)(i / r), j = (int)(i % r);
    lup[i] = (uint16_t)f32_to_bf16_rne((float)(sgn[j] * L2[(size_t)j * N + n]));
  }
}

// R[k][n] = What[k][n] - sum_j L1_bf16[k][j] L2_bf16[j][n] (float64, j ascending),
// stored as float32.
// R[k][n] = fl32(What[k][n] - sum_j L1b[k][j] L2b[j][n]) with the bf16 factors (j
// ascending), r <= 32.  One workgroup per 64 x 64 block of [K][N]: the factor slices go
// through LDS as float64, thread t takes column nn = t % 64 and the rows t / 64 + 4 a.
__global__ void __launch_bounds__(256)
k_prep_residual(const double* __restrict__ wh, const uint16_t* __restrict__ ldown,
                const uint16_t* __restrict__ lup, int K, int N, int r, float* __restrict__ R) {
  __shared__ double Ld[32][64], Lu[32][65];
  const int t = threadIdx.x, n0 = blockIdx.x * 64, k0 = blockIdx.y * 64;
  for (int e = t; e < r * 64; e += 256) {
    const int j = e >> 6, x = e & 63;
    Ld[j][x] = k0 + x < K ? (double)bf16_to_f32(ldown[(size_t)j * K + k0 + x]) : 0.0;
  }
  for (int e = t; e < r * 64; e += 256) {
    const int x = e / r, j = e % r;
    Lu[j][x] = n0 + x < N ? (double)bf16_to_f32(lup[(size_t)(n0 + x) * r + j]) : 0.0;
  }
  __syncthreads();
  const int nn = t & 63, kq = t >> 6;
  double acc[16] = {};
  for (int j = 0; j < r; ++j) {
    const double u = Lu[j][nn];
#pragma unroll
    for (int a = 0; a < 16; ++a) acc[a] = fma(Ld[j][kq + 4 * a], u, acc[a]);
  }
  if (n0 + nn >= N) return;
#pragma unroll
  for (int a = 0; a < 16; ++a) {
    const int k = k0 + kq + 4 * a;
    if (k < K) {
      const size_t i = (size_t)k * N + n0 + nn;
      R[i] = (float)(wh[i] - acc[a]);
    }
  }
}

// int4 quantization of R per output column n and group g of 64 values of k: one
// workgroup per (64 columns, group); the 64 x 64 block goes through LDS so that the
// reads of R rows and the writes of column codes are both contiguous.
__global__ void __launch_bounds__(256)
k_prep_quant(const float* __restrict__ R, int K, int N, uint8_t* __restrict__ qweight,
             uint16_t* __restrict__ wscales) {
  __shared__ float T[64][65];
  const int n0 = blockIdx.x * 64, g = blockIdx.y, t = threadIdx.x;
  for (int e = t; e < 64 * 64; e += 256) {
    const int kk = e >> 6, nn = e & 63;
    T[nn][kk] = (n0 + nn < N) ? R[(size_t)(64 * g + kk) * N + n0 + nn] : 0.f;
  }
  __syncthreads();
  if (t < 64 && n0 + t < N) {
    const int n = n0 + t;
    float amax = 0.f;
    for (int kk = 0; kk < 64; ++kk) amax = fmaxf(amax, fabsf(T[t][kk]));
    const uint32_t sb = f32_to_bf16_rne(amax / 7.0f);
    const double s = (double)__uint_as_float(sb << 16);
    wscales[(size_t)n * (K / 64) + g] = (uint16_t)sb;
    uint8_t* dst = qweight + (size_t)n * (K / 2) + 32 * g;
    for (int kk = 0; kk < 64; kk += 2) {
      int q[2];
      for (int u = 0; u < 2; ++u) {
        // the quotient in float64 decides the round-half-even exactly
        const double v = s > 0.0 ? rint((double)T[t][kk + u] / s) : 0.0;
        q[u] = (int)fmin(fmax(v, -8.0), 7.0);
      }
      dst[kk / 2] = (uint8_t)((q[0] & 15) | ((q[1] & 15) << 4));
    }
  }
}

// NVFP4: max |R| and max |bf16(x m)| over the calibration activations (float bits as
// unsigned: the maximum of non-negative floats, in any order), then the per-tensor
// scales g_w = fl32(amax_R / 2688) and g_x = fl32(amax_xhat / 2688).
__global__ void __launch_bounds__(256)
k_prep_absmax(const float* __restrict__ R, int64_t n, unsigned* __restrict__ out) {
  float a = 0.f;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    a = fmaxf(a, fabsf(R[i]));
  for (int d = 32; d > 0; d >>= 1) a = fmaxf(a, __shfl_xor(a, d));
  if ((threadIdx.x & 63) == 0) atomicMax(out, __float_as_uint(a));
}

__global__ void __launch_bounds__(256)
k_prep_absmax_xhat(const uint16_t* __restrict__ xc, int64_t n, int K, const uint16_t* __restrict__ m,
                   unsigned* __restrict__ out) {
  float a = 0.f;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const float xh = bf16_to_f32(f32_to_bf16_rne(bf16_to_f32(xc[i]) * bf16_to_f32(m[i % K])));
    a = fmaxf(a, fabsf(xh));
  }
  for (int d = 32; d > 0; d >>= 1) a = fmaxf(a, __shfl_xor(a, d));
  if ((threadIdx.x & 63) == 0) atomicMax(out, __float_as_uint(a));
}

__global__ void k_prep_globals(const unsigned* __restrict__ amax, float* __restrict__ g) {
  if (threadIdx.x < 2) g[threadIdx.x] = __uint_as_float(amax[threadIdx.x]) / 2688.0f;
}

// NVFP4 quantization of R per output column in blocks of 16 (nvfp4_quant32 on two
// blocks at a time), 64 x 64 blocks of R transposed through LDS: codes [N][K/2]
// (element 2j in bits 3:0), E4M3 scale codes [N][K/16].
__global__ void __launch_bounds__(256)
k_prep_quant_nvfp4(const float* __restrict__ R, int K, int N, const float* __restrict__ g,
                   uint8_t* __restrict__ qweight, uint8_t* __restrict__ wscales) {
  __shared__ float T[64][65];
  const int n0 = blockIdx.x * 64, kb = blockIdx.y, t = threadIdx.x;
  for (int e = t; e < 64 * 64; e += 256) {
    const int kk = e >> 6, nn = e & 63;
    T[nn][kk] = (n0 + nn < N) ? R[(size_t)(64 * kb + kk) * N + n0 + nn] : 0.f;
  }
  __syncthreads();
  if (t < 64 && n0 + t < N) {
    const int n = n0 + t;
    const float gw = g[0];
    for (int c = 0; c < 2; ++c) {
      float v[32], deq[32];
      uint32_t codes[32], sc[2];
      for (int i = 0; i < 32; ++i) v[i] = T[t][32 * c + i];
      nvfp4_quant32(v, gw, codes, deq, sc);
      uint8_t* dst = qweight + (size_t)n * (K / 2) + 32 * kb + 16 * c;
      for (int i = 0; i < 16; ++i) dst[i] = (uint8_t)(codes[2 * i] | (codes[2 * i + 1] << 4));
      wscales[(size_t)n * (K / 16) + 4 * kb + 2 * c] = (uint8_t)sc[0];
      wscales[(size_t)n * (K / 16) + 4 * kb + 2 * c + 1] = (uint8_t)sc[1];
    }
  }
}

// AWQ W4A16 weights: per output column n and group of 64 along K, asymmetric uint4
// with s = bf16(fl32((max - min) / 15)), z = clamp(rne(-min / s), 0, 15),
// q = clamp(rne(w / s) + z, 0, 15) (the quotients in float64; s = 0 gives zeros).
__global__ void __launch_bounds__(256)
k_prep_awq(const float* __restrict__ W, int K, int N, uint8_t* __restrict__ qweight,
           uint16_t* __restrict__ scales, uint8_t* __restrict__ zeros) {
  __shared__ float T[64][65];
  const int n0 = blockIdx.x * 64, g = blockIdx.y, t = threadIdx.x;
  for (int e = t; e < 64 * 64; e += 256) {
    const int kk = e >> 6, nn = e & 63;
    T[nn][kk] = (n0 + nn < N) ? W[(size_t)(64 * g + kk) * N + n0 + nn] : 0.f;
  }
  __syncthreads();
  if (t < 64 && n0 + t < N) {
    const int n = n0 + t;
    float mx = T[t][0], mn = T[t][0];
    for (int kk = 1; kk < 64; ++kk) {
      mx = fmaxf(mx, T[t][kk]);
      mn = fminf(mn, T[t][kk]);
    }
    const uint32_t sb = f32_to_bf16_rne((mx - mn) / 15.0f);
    const double s = (double)__uint_as_float(sb << 16);
    const double z = s > 0.0 ? fmin(fmax(rint(-(double)mn / s), 0.0), 15.0) : 0.0;
    scales[(size_t)n * (K / 64) + g] = (uint16_t)sb;
    zeros[(size_t)n * (K / 64) + g] = (uint8_t)z;
    uint8_t* dst = qweight + (size_t)n * (K / 2) + 32 * g;
    for (int kk = 0; kk < 64; kk += 2) {
      int q[2];
      for (int u = 0; u < 2; ++u)
        q[u] = s > 0.0 ? (int)fmin(fmax(rint((double)T[t][kk + u] / s) + z, 0.0), 15.0) : 0;
      dst[kk / 2] = (uint8_t)(q[0] | (q[1] << 4));
    }
  }
}

size_t al(size_t b) { return (b + 255) & ~size_t(255); }

// eigenvalues (kMaxL), then M1 [l][r] and M2 [r][l] with r <= 32
constexpr size_t kSmallBytes = (kMaxL + 2 * kMaxL * 32) * 8;
// partial products of the GEMMs that have few output tiles (split along k)
constexpr size_t kPartBytes = size_t(8) << 20;

}  // namespace

size_t prep_workspace_bytes(int64_t K, int64_t N, int rank, int l) {
  return al(K * N * 8) + al(K * l * 8) + al(std::max(K, N) * l * 8) + al(N * l * 8) + al(l * N * 8) + 3 * al(64 * 64 * 8) +
         al(kSmallBytes) + al(K * rank * 8) + al(rank * N * 8) + al(K * N * 4) + al(256) +
         al(kPartBytes);
}

hipError_t launch_prep(bool nvfp4, int K, int N, int rank, int l, int iters, const float* w,
                       const uint16_t* xc, int64_t Mc, const double* omega, uint8_t* qweight,
                       void* wscales, uint16_t* smooth, uint16_t* ldown, uint16_t* lup,
                       float* residual, void* ws, int* fail_host, float* globals_host,
                       hipStream_t st) {
  uint8_t* p = static_cast<uint8_t*>(ws);
  auto take = [&](size_t b) { uint8_t* q = p; p += al(b); return q; };
  double* wh = reinterpret_cast<double*>(take((size_t)K * N * 8));
  double* Y = reinterpret_cast<double*>(take((size_t)K * l * 8));
  // the CholeskyQR2 output, for Y [K][l] and Z [N][l]
  double* Y2 = reinterpret_cast<double*>(take((size_t)std::max(K, N) * l * 8));
  double* Z = reinterpret_cast<double*>(take((size_t)N * l * 8));
  double* Bm = reinterpret_cast<double*>(take((size_t)l * N * 8));
  double* G = reinterpret_cast<double*>(take(64 * 64 * 8));
  double* Rinv = reinterpret_cast<double*>(take(64 * 64 * 8));
  double* Vv = reinterpret_cast<double*>(take(64 * 64 * 8));
  double* small = reinterpret_cast<double*>(take(kSmallBytes));
  double* L1 = reinterpret_cast<double*>(take((size_t)K * rank * 8));
  double* L2 = reinterpret_cast<double*>(take((size_t)rank * N * 8));
  float* R = residual ? residual : reinterpret_cast<float*>(take((size_t)K * N * 4));
  if (residual) take((size_t)K * N * 4);
  double* parts = reinterpret_cast<double*>(take(kPartBytes));
  int* flags = reinterpret_cast<int*>(take(256));  // fail flag, signs, amax bits, globals
  int* sgn = flags + 1;
  unsigned* amax = reinterpret_cast<unsigned*>(flags + 40);
  float* globals = reinterpret_cast<float*>(flags + 42);

  // a product with fewer than 128 output tiles is split along k into nz chunks (at most
  // 64, at least 64 values of k each, partials within kPartBytes), summed in order
  auto gemm = [&](const double* A, int64_t as0, int64_t as1, const double* B, int64_t bs0,
                  int64_t bs1, double* C, int64_t ldc, int M, int Nn, int Kk) {
    const int tiles = ((Nn + 63) / 64) * ((M + 63) / 64);
    int nz = 1;
    if (tiles < 128)
      nz = (int)std::max<int64_t>(1, std::min<int64_t>({64, Kk / 64, (int64_t)(kPartBytes / 8) / ((int64_t)M * Nn)}));
    if (nz <= 1) {
      dim3 grid((Nn + 63) / 64, (M + 63) / 64);
      hipLaunchKernelGGL(k_gemm_f64, grid, dim3(256), 0, st, A, as0, as1, B, bs0, bs1, C, ldc, M, Nn,
                         Kk, Kk, (int64_t)0);
      return;
    }
    const int kc = ((Kk + nz - 1) / nz + 15) / 16 * 16;
    nz = (Kk + kc - 1) / kc;
    dim3 grid((Nn + 63) / 64, (M + 63) / 64, nz);
    hipLaunchKernelGGL(k_gemm_f64, grid, dim3(256), 0, st, A, as0, as1, B, bs0, bs1, parts,
                       (int64_t)Nn, M, Nn, Kk, kc, (int64_t)M * Nn);
    const int64_t mn = (int64_t)M * Nn;
    hipLaunchKernelGGL(k_sum_parts, dim3((unsigned)((mn + 255) / 256)), dim3(256), 0, st, parts, nz,
                       M, Nn, C, ldc);
  };
  // orth(Y [n][l]) in place by CholeskyQR2; the first failed copy is kept in copy_err
  hipError_t copy_err = hipSuccess;
  auto orth = [&](double* Yp, int n) {
    for (int pass = 0; pass < 2; ++pass) {
      gemm(Yp, 1, l, Yp, l, 1, G, l, l, l, n);                       // G = Y^T Y
      if (l <= 16)
        hipLaunchKernelGGL(k_chol_inv<16>, dim3(1), dim3(64), 0, st, G, l, Rinv, flags);
      else if (l <= 32)
        hipLaunchKernelGGL(k_chol_inv<32>, dim3(1), dim3(64), 0, st, G, l, Rinv, flags);
      else if (l <= 48)
        hipLaunchKernelGGL(k_chol_inv<48>, dim3(1), dim3(64), 0, st, G, l, Rinv, flags);
      else
        hipLaunchKernelGGL(k_chol_inv<64>, dim3(1), dim3(64), 0, st, G, l, Rinv, flags);
      gemm(Yp, l, 1, Rinv, l, 1, Y2, l, n, l, l);                    // Y2 = Y R^-1
      const hipError_t ce = hipMemcpyAsync(Yp, Y2, (size_t)n * l * 8, hipMemcpyDeviceToDevice, st);
      if (copy_err == hipSuccess) copy_err = ce;
    }
  };

  hipError_t e = hipMemsetAsync(flags, 0, 256, st);
  if (e != hipSuccess) return e;
  {  // channel amax in row chunks of at least 64 (at most 128 chunks, within kPartBytes)
    float* part = reinterpret_cast<float*>(parts);
    const int64_t nzmax = std::max<int64_t>(1, std::min<int64_t>(128, (int64_t)(kPartBytes / 4) / K));
    const int64_t nz0 = std::max<int64_t>(1, std::min<int64_t>(nzmax, (Mc + 63) / 64));
    const int64_t rc = std::max<int64_t>(1, (Mc + nz0 - 1) / nz0);
    const int nz = (int)std::max<int64_t>(1, (Mc + rc - 1) / rc);
    hipLaunchKernelGGL(k_prep_amax_part, dim3((K / 2 + 255) / 256, nz), dim3(256), 0, st, xc, Mc, K,
                       rc, part);
    hipLaunchKernelGGL(k_prep_smooth, dim3((K + 255) / 256), dim3(256), 0, st, part, nz, K, smooth);
  }
  const int64_t KN = (int64_t)K * N;
  hipLaunchKernelGGL(k_prep_what, dim3((unsigned)((KN + 255) / 256)), dim3(256), 0, st, w, smooth,
                     wh, K, N);
  if (rank > 0) {
    gemm(wh, N, 1, omega, l, 1, Y, l, K, l, N);                      // Y = What Omega
    orth(Y, K);
    for (int it = 0; it < iters; ++it) {
      gemm(wh, 1, N, Y, l, 1, Z, l, N, l, K);                        // Z = What^T Q
      orth(Z, N);
      gemm(wh, N, 1, Z, l, 1, Y, l, K, l, N);                        // Y = What Z
      orth(Y, K);
    }
    gemm(Y, 1, l, wh, N, 1, Bm, N, l, N, K);                         // B = Q^T What [l][N]
    gemm(Bm, N, 1, Bm, 1, N, G, l, l, l, N);                         // C = B B^T
    double* ev = small;
    double* M1 = small + kMaxL;
    double* M2 = small + kMaxL + kMaxL * 32;
    hipLaunchKernelGGL(k_jacobi, dim3(1), dim3(256), 0, st, G, l, ev, Vv);
    hipLaunchKernelGGL(k_prep_small, dim3(1), dim3(256), 0, st, ev, Vv, l, rank, M1, M2, flags);
    gemm(Y, l, 1, M1, rank, 1, L1, rank, K, rank, l);                // L1 = Q Ub_r S_r
    gemm(M2, l, 1, Bm, N, 1, L2, N, rank, N, l);                     // L2 = S_r^-1 Ub_r^T B
    hipLaunchKernelGGL(k_prep_sign, dim3(rank), dim3(256), 0, st, L1, K, rank, sgn);
    const int64_t nf = std::max<int64_t>((int64_t)K * rank, (int64_t)N * rank);
    hipLaunchKernelGGL(k_prep_factors, dim3((unsigned)((nf + 255) / 256)), dim3(256), 0, st, L1,
                       L2, sgn, K, N, rank, ldown, lup);
  }
  hipLaunchKernelGGL(k_prep_residual, dim3((N + 63) / 64, (K + 63) / 64), dim3(256), 0, st, wh,
                     ldown, lup, K, N, rank, R);
  if (nvfp4) {
    const unsigned gb = (unsigned)std::min<int64_t>((KN + 255) / 256, 1024);
    hipLaunchKernelGGL(k_prep_absmax, dim3(gb), dim3(256), 0, st, R, KN, amax);
    const int64_t xn = Mc * K;
    const unsigned gx = (unsigned)std::min<int64_t>((xn + 255) / 256, 1024);
    hipLaunchKernelGGL(k_prep_absmax_xhat, dim3(gx), dim3(256), 0, st, xc, xn, K, smooth, amax + 1);
    hipLaunchKernelGGL(k_prep_globals, dim3(1), dim3(64), 0, st, amax, globals);
    hipLaunchKernelGGL(k_prep_quant_nvfp4, dim3((N + 63) / 64, K / 64), dim3(256), 0, st, R, K, N,
                       globals, qweight, static_cast<uint8_t*>(wscales));
  } else {
    hipLaunchKernelGGL(k_prep_quant, dim3((N + 63) / 64, K / 64), dim3(256), 0, st, R, K, N,
                       qweight, static_cast<uint16_t*>(wscales));
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (copy_err != hipSuccess) return copy_err;
  e = hipMemcpyAsync(fail_host, flags, sizeof(int), hipMemcpyDeviceToHost, st);
  if (e != hipSuccess) return e;
  if (nvfp4) {
    e = hipMemcpyAsync(globals_host, globals, 2 * sizeof(float), hipMemcpyDeviceToHost, st);
    if (e != hipSuccess) return e;
  }
  return hipStreamSynchronize(st);
}

hipError_t launch_prep_awq(int K, int N, const float* w, uint8_t* qweight, uint16_t* scales,
                           uint8_t* zeros, hipStream_t st) {
  hipLaunchKernelGGL(k_prep_awq, dim3((N + 63) / 64, K / 64), dim3(256), 0, st, w, K, N, qweight,
                     scales, zeros);
  return hipGetLastError();
}

}  // namespace svdq
