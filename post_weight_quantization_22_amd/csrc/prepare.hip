// Damping, processing order and the inverse-Hessian factor on gfx950 (fp64).
//
// "GPTQ deep dive" (hncyxsy.com news 243429): section 3.1 steps 1-2 (H =
// 2XX^T + lambda I, then a Cholesky factorization), section 2.4 (the Cholesky
// factorization replaces repeated O(n^3), unstable inversion), section 3.3
// (damp_percent, default 0.01, a damping ratio on the Hessian diagonal;
// desc_act processes columns by importance).  "Calibration algorithms guide"
// (bhfrc.com news 5741) section 2.3: the order is by descending Hessian
// diagonal.
//
// The column loop needs U, the upper Cholesky factor of H_d^-1
// (H_d^-1 = U^T U).  With H_d = R R^T, R upper (a Cholesky factorization taken
// from the last index backwards), U = R^-1, which costs one factorization and
// one triangular inverse (2n^3/3 flops).  Reversing the index order turns it
// into the textbook form: with J the reversal, A = J H_d J = L L^T (L lower),
// R = J L J and U = J L^-1 J.  So the kernels build A (permuted, damped,
// reversed) in fp64, run a blocked right-looking lower Cholesky and a blocked
// lower triangular inverse in place, and write U[k][l] = L^-1[n-1-k][n-1-l]
// rounded to fp32.
//
// Blocked with NB = 64: per panel a one-workgroup factorization of the 64x64
// diagonal block (which also inverts it), a triangular solve of the panel
// below it and a lower-triangle SYRK of the trailing matrix; then per block
// column (last to first) one kernel forms L^-1 below the diagonal.
#include "kernels.hpp"

namespace gptq {

namespace {

constexpr int NB = 64;
constexpr int NBP = NB + 1;

struct PrepWs {
  double* A;     // [n, n]
  double* Dinv;  // [nblk, NB, NB]
  double* P;     // [n, NB]
  double* diag;  // [n]
  double* lam;   // [1]
  int32_t* perm; // [n]
};

PrepWs carve(void* ws, int64_t n) {
  const int64_t nblk = ceil_div(n, NB);
  char* p = reinterpret_cast<char*>(ws);
  PrepWs w;
  w.A = reinterpret_cast<double*>(p);
  p += align_up((size_t)n * n * sizeof(double), 256);
  w.Dinv = reinterpret_cast<double*>(p);
  p += align_up((size_t)nblk * NB * NB * sizeof(double), 256);
  w.P = reinterpret_cast<double*>(p);
  p += align_up((size_t)n * NB * sizeof(double), 256);
  w.diag = reinterpret_cast<double*>(p);
  p += align_up((size_t)n * sizeof(double), 256);
  w.lam = reinterpret_cast<double*>(p);
  p += 256;
  w.perm = reinterpret_cast<int32_t*>(p);
  return w;
}

// diag(H) with the dead-column fix, lambda = perc_damp * mean(diag H), info reset.
__global__ __launch_bounds__(1024) void diag_damp_kernel(const float* __restrict__ S, int64_t n,
                                                         int64_t lds, float perc_damp,
                                                         double* __restrict__ diag,
                                                         uint8_t* __restrict__ dead,
                                                         double* __restrict__ lam,
                                                         float* __restrict__ lambda_out,
                                                         int32_t* __restrict__ info) {
  __shared__ double part[1024];
  __shared__ int bad;
  if (threadIdx.x == 0) bad = 0;
  __syncthreads();
  double sum = 0.0;
  for (int64_t i = threadIdx.x; i < n; i += blockDim.x) {
    const float s = S[i * lds + i];
    if (!isfinite(s)) bad = 1;
    double d = 2.0 * (double)s;
    const bool is_dead = d == 0.0;
    if (is_dead) d = 1.0;
    if (dead) dead[i] = is_dead ? 1 : 0;
    diag[i] = d;
    sum += d;
  }
  part[threadIdx.x] = sum;
  __syncthreads();
  for (int off = blockDim.x / 2; off > 0; off >>= 1) {
    if ((int)threadIdx.x < off) part[threadIdx.x] += part[threadIdx.x + off];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const double l = (double)perc_damp * (part[0] / (double)n);
    *lam = l;
    if (lambda_out) *lambda_out = (float)l;
    *info = bad ? -1 : 0;
  }
}

// Stable descending order of diag: rank_i = #{j: d_j > d_i or (d_j == d_i and j < i)}.
__global__ __launch_bounds__(256) void rank_kernel(const double* __restrict__ diag, int64_t n,
                                                   int32_t* __restrict__ perm) {
  __shared__ double key[1024];
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const double di = i < n ? diag[i] : 0.0;
  int64_t rank = 0;
  for (int64_t base = 0; base < n; base += 1024) {
    __syncthreads();
    for (int t = threadIdx.x; t < 1024; t += blockDim.x)
      key[t] = base + t < n ? diag[base + t] : 0.0;
    __syncthreads();
    const int cnt = (int)min<int64_t>(1024, n - base);
    for (int t = 0; t < cnt; ++t) {
      const double dj = key[t];
      const int64_t j = base + t;
      rank += (dj > di) || (dj == di && j < i);
    }
  }
  if (i < n) perm[rank] = (int32_t)i;
}

__global__ void iota_kernel(int32_t* __restrict__ perm, int64_t n) {
  const int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (k < n) perm[k] = (int32_t)k;
}

// A[a][b] (a >= b) = H_d[perm[n-1-a]][perm[n-1-b]], H = 2S (lower of S authoritative).
__global__ __launch_bounds__(256) void build_a_kernel(const float* __restrict__ S, int64_t n,
                                                      int64_t lds,
                                                      const int32_t* __restrict__ perm,
                                                      const double* __restrict__ diag,
                                                      const double* __restrict__ lam,
                                                      double* __restrict__ A,
                                                      int32_t* __restrict__ info) {
  const int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const double l = *lam;
  for (int64_t a = blockIdx.y; a < n; a += gridDim.y) {
    if (b > a) continue;
    const int64_t p = perm[n - 1 - a], q = perm[n - 1 - b];
    double v;
    if (a == b) {
      v = diag[p] + l;
    } else {
      const float s = p > q ? S[p * lds + q] : S[q * lds + p];
      if (!isfinite(s)) *info = -1;
      v = 2.0 * (double)s;
    }
    A[a * n + b] = v;
  }
}

// Factor the diagonal block at kb (lower Cholesky) and invert it.
__global__ __launch_bounds__(256) void potrf_diag_kernel(double* __restrict__ A, int64_t n,
                                                         int64_t kb, double* __restrict__ Dinv,
                                                         int32_t* __restrict__ info) {
  __shared__ double Ls[NB][NBP];
  __shared__ double Li[NB][NBP];
  const int tid = threadIdx.x;
  const int nb = (int)min<int64_t>(NB, n - kb);
  for (int e = tid; e < NB * NB; e += blockDim.x) {
    const int i = e / NB, j = e % NB;
    Ls[i][j] = (i < nb && j <= i) ? A[(kb + i) * n + kb + j] : (i == j ? 1.0 : 0.0);
    Li[i][j] = i == j ? 1.0 : 0.0;
  }
  __syncthreads();
  for (int k = 0; k < nb; ++k) {
    if (tid == 0) {
      double d = Ls[k][k];
      if (!(d > 0.0) || !isfinite(d)) {
        if (*info == 0) *info = (int32_t)(n - (kb + k));  // processing position + 1
        d = 1.0;
      }
      Ls[k][k] = sqrt(d);
    }
    __syncthreads();
    for (int i = k + 1 + tid; i < nb; i += blockDim.x) Ls[i][k] /= Ls[k][k];
    __syncthreads();
    const int rem = nb - k - 1;
    for (int e = tid; e < rem * rem; e += blockDim.x) {
      const int i = k + 1 + e / rem, j = k + 1 + e % rem;
      if (j <= i) Ls[i][j] -= Ls[i][k] * Ls[j][k];
    }
    __syncthreads();
  }
  // Li = Ls^-1 by forward elimination applied to the identity
  for (int k = 0; k < nb; ++k) {
    for (int c = tid; c <= k; c += blockDim.x) Li[k][c] /= Ls[k][k];
    __syncthreads();
    const int rem = nb - k - 1;
    for (int e = tid; e < rem * (k + 1); e += blockDim.x) {
      const int i = k + 1 + e / (k + 1), c = e % (k + 1);
      Li[i][c] -= Ls[i][k] * Li[k][c];
    }
    __syncthreads();
  }
  const int64_t blk = kb / NB;
  for (int e = tid; e < NB * NB; e += blockDim.x) {
    const int i = e / NB, j = e % NB;
    if (i < nb && j <= i) A[(kb + i) * n + kb + j] = Ls[i][j];
    Dinv[(blk * NB + i) * NB + j] = (i < nb && j < nb && j <= i) ? Li[i][j] : 0.0;
  }
}

// 64x64 fp64 tile product, 256 threads x 4x4 outputs.  acc[u][v] accumulates
// sum_k Aop(ty + 16u, k) * Bop(k, tx + 16v) for k in [0, K).
// Aop(i, k) = Ablk[i * lda + k]; Bop(k, j) = Bblk[k * ldb + j] if b_kmajor
// else Bblk[j * ldb + k].  Rows/cols past (mi, nj) read as 0.
__device__ void tile_gemm64(const double* __restrict__ Ablk, int64_t lda, int mi,
                            const double* __restrict__ Bblk, int64_t ldb, int nj, bool b_kmajor,
                            int K, double (*As)[NBP], double (*Bs)[NBP], double acc[4][4]) {
  constexpr int KC = 16;
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  for (int k0 = 0; k0 < K; k0 += KC) {
    __syncthreads();
    for (int e = tid; e < KC * NB; e += blockDim.x) {
      const int kk = e % KC, ii = e / KC;
      const bool kin = k0 + kk < K;
      As[kk][ii] = (kin && ii < mi) ? Ablk[ii * lda + k0 + kk] : 0.0;
      if (!b_kmajor) Bs[kk][ii] = (kin && ii < nj) ? Bblk[ii * ldb + k0 + kk] : 0.0;
    }
    if (b_kmajor) {
      for (int e = tid; e < KC * NB; e += blockDim.x) {
        const int kk = e / NB, jj = e % NB;
        Bs[kk][jj] = (k0 + kk < K && jj < nj) ? Bblk[(k0 + kk) * ldb + jj] : 0.0;
      }
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < KC; ++kk) {
      double a[4], b[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        a[u] = As[kk][ty + 16 * u];
        b[u] = Bs[kk][tx + 16 * u];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[u][v] = fma(a[u], b[v], acc[u][v]);
    }
  }
}

// Panel below the diagonal block: A[i, kb:kb+nb] <- A[i, kb:kb+nb] * Dinv_kb^T.
__global__ __launch_bounds__(256) void trsm_panel_kernel(double* __restrict__ A, int64_t n,
                                                         int64_t kb,
                                                         const double* __restrict__ Dinv) {
  __shared__ double As[16][NBP], Bs[16][NBP];
  __shared__ double Out[NB][NBP];
  const int nb = (int)min<int64_t>(NB, n - kb);
  const int64_t r0 = kb + nb + (int64_t)blockIdx.x * NB;
  const int mi = (int)min<int64_t>(NB, n - r0);
  double acc[4][4] = {};
  tile_gemm64(A + r0 * n + kb, n, mi, Dinv + (kb / NB) * NB * NB, NB, nb, false, nb, As, Bs, acc);
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int v = 0; v < 4; ++v) Out[ty + 16 * u][tx + 16 * v] = acc[u][v];
  __syncthreads();  // every read of this row block precedes the write-back
  for (int e = threadIdx.x; e < NB * NB; e += blockDim.x) {
    const int i = e / NB, j = e % NB;
    if (i < mi && j < nb) A[(r0 + i) * n + kb + j] = Out[i][j];
  }
}

// Trailing update: A[i][j] -= sum_k L[i][kb+k] L[j][kb+k], lower tiles past the panel.
__device__ __forceinline__ void lower_tile(int64_t L, int64_t& ti, int64_t& tj) {
  int64_t t = (int64_t)((sqrt(8.0 * (double)L + 1.0) - 1.0) * 0.5);
  while (t * (t + 1) / 2 > L) --t;
  while ((t + 1) * (t + 2) / 2 <= L) ++t;
  ti = t;
  tj = L - t * (t + 1) / 2;
}

__global__ __launch_bounds__(256) void syrk_update_kernel(double* __restrict__ A, int64_t n,
                                                          int64_t kb) {
  __shared__ double As[16][NBP], Bs[16][NBP];
  const int nb = (int)min<int64_t>(NB, n - kb);
  const int64_t base = kb + nb;
  int64_t ti, tj;
  lower_tile(blockIdx.x, ti, tj);
  const int64_t i0 = base + ti * NB, j0 = base + tj * NB;
  const int mi = (int)min<int64_t>(NB, n - i0), nj = (int)min<int64_t>(NB, n - j0);
  double acc[4][4] = {};
  tile_gemm64(A + i0 * n + kb, n, mi, A + j0 * n + kb, n, nj, false, nb, As, Bs, acc);
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t gi = i0 + ty + 16 * u, gj = j0 + tx + 16 * v;
      if (gi < n && gj < n && gj <= gi) A[gi * n + gj] -= acc[u][v];
    }
}

// Copy the L column block jb below its diagonal block into P[k - (jb+1)NB][0:NB].
__global__ __launch_bounds__(256) void copy_panel_kernel(const double* __restrict__ A, int64_t n,
                                                         int64_t jb, double* __restrict__ P) {
  const int64_t k = (jb + 1) * NB + blockIdx.x;
  if (k >= n) return;
  for (int c = threadIdx.x; c < NB; c += blockDim.x) P[(k - (jb + 1) * NB) * NB + c] = A[k * n + jb * NB + c];
}

// L^-1 block column jb: for row block i > jb,
//   X[i, jb] = -(sum_{kb=jb+1}^{i} X[i, kb] L[kb, jb]) X[jb, jb],
// X[i, kb] for kb > jb already in A (kb < i) or Dinv (kb == i); L[kb, jb] in P.
__global__ __launch_bounds__(256) void trtri_step_kernel(double* __restrict__ A, int64_t n,
                                                         int64_t jb,
                                                         const double* __restrict__ Dinv,
                                                         const double* __restrict__ P) {
  __shared__ double As[16][NBP], Bs[16][NBP];
  __shared__ double T[NB][NBP];
  const int64_t ib = jb + 1 + blockIdx.x;
  const int64_t i0 = ib * NB;
  const int mi = (int)min<int64_t>(NB, n - i0);
  double acc[4][4] = {};
  // off-diagonal part: X[i, (jb+1)NB : i0] * P[0 : i0 - (jb+1)NB]
  const int64_t koff = (jb + 1) * NB;
  const int64_t K1 = i0 - koff;
  for (int64_t k0 = 0; k0 < K1; k0 += NB)
    tile_gemm64(A + i0 * n + koff + k0, n, mi, P + k0 * NB, NB, NB, true, NB, As, Bs, acc);
  // diagonal part: Dinv_ib * P[i0 - koff : i0 - koff + mi]
  tile_gemm64(Dinv + ib * NB * NB, NB, mi, P + K1 * NB, NB, NB, true, mi, As, Bs, acc);
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  __syncthreads();
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int v = 0; v < 4; ++v) T[ty + 16 * u][tx + 16 * v] = acc[u][v];
  // out = -T * Dinv_jb   (Dinv_jb k-major: Dinv[jb][k][c])
  double acc2[4][4] = {};
  tile_gemm64(&T[0][0], NBP, mi, Dinv + jb * NB * NB, NB, NB, true, NB, As, Bs, acc2);
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int i = ty + 16 * u, c = tx + 16 * v;
      if (i < mi) A[(i0 + i) * n + jb * NB + c] = -acc2[u][v];
    }
}

// U[k][l] = L^-1[n-1-k][n-1-l] for l >= k (fp32), 0 below the diagonal.
__global__ __launch_bounds__(256) void write_u_kernel(const double* __restrict__ A,
                                                      const double* __restrict__ Dinv, int64_t n,
                                                      float* __restrict__ U, int64_t ldu) {
  const int64_t l = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (l >= n) return;
  for (int64_t k = blockIdx.y; k < n; k += gridDim.y) {
    float v = 0.0f;
    if (l >= k) {
      const int64_t a = n - 1 - k, b = n - 1 - l;
      const int64_t ba = a / NB, bb = b / NB;
      v = (float)(ba == bb ? Dinv[(ba * NB + a % NB) * NB + b % NB] : A[a * n + b]);
    }
    U[k * ldu + l] = v;
  }
}

}  // namespace

size_t prepare_ws_bytes(int64_t n) {
  const int64_t nblk = ceil_div(n, NB);
  size_t b = align_up((size_t)n * n * sizeof(double), 256);
  b += align_up((size_t)nblk * NB * NB * sizeof(double), 256);
  b += align_up((size_t)n * NB * sizeof(double), 256);
  b += align_up((size_t)n * sizeof(double), 256);
  b += 256;
  b += align_up((size_t)n * sizeof(int32_t), 256);
  return b;
}

hipError_t launch_prepare(const float* S, int64_t n, int64_t lds, float perc_damp, int desc_act,
                          float* U, int64_t ldu, int32_t* perm, uint8_t* dead, float* lambda_out,
                          int32_t* info, void* ws, hipStream_t stream) {
  PrepWs w = carve(ws, n);
  int32_t* pm = perm ? perm : w.perm;
  const int64_t nblk = ceil_div(n, NB);
  hipLaunchKernelGGL(diag_damp_kernel, dim3(1), dim3(1024), 0, stream, S, n, lds, perc_damp,
                     w.diag, dead, w.lam, lambda_out, info);
  if (desc_act) {
    hipLaunchKernelGGL(rank_kernel, dim3((unsigned)ceil_div(n, 256)), dim3(256), 0, stream, w.diag,
                       n, pm);
  } else {
    hipLaunchKernelGGL(iota_kernel, dim3((unsigned)ceil_div(n, 256)), dim3(256), 0, stream, pm, n);
  }
  {
    const dim3 grid((unsigned)ceil_div(n, 256), (unsigned)hmin(n, 2048));
    hipLaunchKernelGGL(build_a_kernel, grid, dim3(256), 0, stream, S, n, lds, pm, w.diag, w.lam,
                       w.A, info);
  }
  for (int64_t kb = 0; kb < n; kb += NB) {
    hipLaunchKernelGGL(potrf_diag_kernel, dim3(1), dim3(256), 0, stream, w.A, n, kb, w.Dinv, info);
    const int64_t rest = n - kb - NB;
    if (rest > 0) {
      const int64_t rb = ceil_div(rest, NB);
      hipLaunchKernelGGL(trsm_panel_kernel, dim3((unsigned)rb), dim3(256), 0, stream, w.A, n, kb,
                         w.Dinv);
      hipLaunchKernelGGL(syrk_update_kernel, dim3((unsigned)(rb * (rb + 1) / 2)), dim3(256), 0,
                         stream, w.A, n, kb);
    }
  }
  for (int64_t jb = nblk - 2; jb >= 0; --jb) {
    const int64_t rows = n - (jb + 1) * NB;
    hipLaunchKernelGGL(copy_panel_kernel, dim3((unsigned)rows), dim3(64), 0, stream, w.A, n, jb,
                       w.P);
    hipLaunchKernelGGL(trtri_step_kernel, dim3((unsigned)(nblk - 1 - jb)), dim3(256), 0, stream,
                       w.A, n, jb, w.Dinv, w.P);
  }
  {
    const dim3 grid((unsigned)ceil_div(n, 256), (unsigned)hmin(n, 2048));
    hipLaunchKernelGGL(write_u_kernel, grid, dim3(256), 0, stream, w.A, w.Dinv, n, U, ldu);
  }
  return hipGetLastError();
}

}  // namespace gptq
