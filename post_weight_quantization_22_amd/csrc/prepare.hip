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
// from the last index backwards), U = R^-1: one factorization and one
// triangular inverse, 2n^3/3 flops.  Reversing the index order gives the
// textbook form: with J the reversal, A = J H_d J = L L^T (L lower), R = J L J
// and U = J L^-1 J.  So the kernels build A (permuted, damped, reversed) in
// fp64 and compute X = L^-1 directly, then write U[k][l] = X[n-1-k][n-1-l]
// rounded to fp32.
//
// X = L^-1 by recursive halving.  For A = [[A11, .], [A21, A22]]:
//   X11 = chol_inv(A11)                  (recursion; nodes of <= 128 in one kernel)
//   T   = A21 X11^T          (= L21)     GEMM, X11 lower
//   A22 = A22 - T T^T                    SYRK, lower tiles
//   M   = T X11              (= L21 X11) GEMM, stored over A21
//   X22 = chol_inv(A22)                  (recursion)
//   X21 = -X22 M                         GEMM, X22 lower
// which follows from A21 = L21 L11^T, A22 = L21 L21^T + L22 L22^T and
// L^-1 = [[X11, 0], [-X22 L21 X11, X22]].  The leaves run in order; everything
// between them is a large GEMM on v_mfma_f64_16x16x4_f64, so no kernel carries
// a long serial reduction.
#include "kernels.hpp"

namespace gptq {

namespace {

constexpr int NB = 64;     // register-blocked factor/inverse size
constexpr int NODE = 128;  // subproblems up to this size run in one workgroup

typedef double f64x4 __attribute__((ext_vector_type(4)));

struct PrepWs {
  double* A;     // [n, n] lower: damped, permuted, reversed Hessian (overwritten)
  double* X;     // [n, n] lower: L^-1
  double* T;     // [s2, s1] of the top split
  double* diag;  // [n]
  double* lam;   // [1]
  int32_t* perm; // [n]
};

int64_t split_first(int64_t s) {
  const int64_t blocks = ceil_div(s, NODE);
  return ((blocks + 1) / 2) * NODE;
}

size_t t_elems(int64_t n) {
  if (n <= NODE) return 0;
  const int64_t s1 = split_first(n);
  return (size_t)(n - s1) * (size_t)s1;
}

PrepWs carve(void* ws, int64_t n) {
  char* p = reinterpret_cast<char*>(ws);
  PrepWs w;
  w.A = reinterpret_cast<double*>(p);
  p += align_up((size_t)n * n * sizeof(double), 256);
  w.X = reinterpret_cast<double*>(p);
  p += align_up((size_t)n * n * sizeof(double), 256);
  w.T = reinterpret_cast<double*>(p);
  p += align_up(t_elems(n) * sizeof(double), 256);
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

// ---------------------------------------------------------------------------
// Register-blocked 64x64 factor + inverse, shared by the node kernel.
// 16 x 16 threads, each owning the 4 x 4 entries (ty + 16u, tx + 16v).  One
// sweep over the columns k does both: the right-looking Cholesky step (column
// k of L from the updated column of A, rank-1 update of the trailing part) and
// the forward elimination of X = L^-1 (row k of X becomes final as x_kj / l_kk,
// then x_ij -= l_ik x_kj below it), which needs exactly column k of L and the
// reciprocal pivot of the same step.  Column k of A and row k of X travel
// through LDS, double buffered: one barrier per column.  L itself is never
// stored.  Entries of `a` above the diagonal are scratch; rows/cols >= s hold
// the identity.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void chol_inv_regs(double (&a)[4][4], double (&x)[4][4], int s,
                                              int64_t n, int64_t off, int32_t* info,
                                              double (*colb)[NB], double (*rowb)[NB]) {
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int v = 0; v < 4; ++v) x[u][v] = (ty + 16 * u == tx + 16 * v) ? 1.0 : 0.0;
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    for (int kk = 0; kk < 16; ++kk) {
      const int k = 16 * kb + kk;
      if (k >= s) break;
      double* cb = colb[k & 1];
      double* xb = rowb[k & 1];
      if (tx == kk) {
#pragma unroll
        for (int u = 0; u < 4; ++u) cb[ty + 16 * u] = a[u][kb];
      }
      if (ty == kk) {
#pragma unroll
        for (int v = 0; v < 4; ++v) xb[tx + 16 * v] = x[kb][v];
      }
      __syncthreads();
      double d = cb[k];
      const bool bad = !(d > 0.0) || !isfinite(d);
      if (bad) {
        if (threadIdx.x == 0 && *info == 0) *info = (int32_t)(n - (off + k));  // position + 1
        d = 1.0;
      }
      const double rp = 1.0 / sqrt(d);  // 1 / l_kk
      double ci[4], cj[4], xk[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = ty + 16 * u;
        ci[u] = (i > k && i < s) ? cb[i] * rp : 0.0;  // l_ik
      }
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int j = tx + 16 * v;
        cj[v] = (j > k && j < s) ? cb[j] * rp : 0.0;  // l_jk
        xk[v] = j <= k ? xb[j] * rp : 0.0;            // final x_kj
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          a[u][v] = fma(-ci[u], cj[v], a[u][v]);
          x[u][v] = fma(-ci[u], xk[v], x[u][v]);
        }
      if (ty == kk) {
#pragma unroll
        for (int v = 0; v < 4; ++v) x[kb][v] = xk[v];
      }
    }
  }
  __syncthreads();
}

// acc[u][v] (+)= sum_k P(ty + 16u, k) * Q(k, tx + 16v), k < 64, operands in LDS.
// P is read as Ps[i][k]; Q as Qs[k][j] (QT == false) or Qs[j][k] (QT == true).
template <bool QT>
__device__ __forceinline__ void mm64(const double (*Ps)[NB + 1], const double (*Qs)[NB + 1],
                                     double (&acc)[4][4]) {
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
#pragma unroll 4
  for (int k = 0; k < NB; ++k) {
    double p[4], q[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) p[u] = Ps[ty + 16 * u][k];
#pragma unroll
    for (int v = 0; v < 4; ++v) q[v] = QT ? Qs[tx + 16 * v][k] : Qs[k][tx + 16 * v];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[u][v] = fma(p[u], q[v], acc[u][v]);
  }
}

__device__ __forceinline__ void to_lds(double (*S)[NB + 1], const double (&r)[4][4]) {
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int v = 0; v < 4; ++v) S[ty + 16 * u][tx + 16 * v] = r[u][v];
}

// A node of size s <= 128 in one workgroup: X[off:off+s, off:off+s] = inverse of
// the Cholesky factor of A[off:off+s, off:off+s], by the same split as chol_inv
// (64 + rest) with every product done from LDS.
__global__ __launch_bounds__(256) void node_kernel(const double* __restrict__ A,
                                                   double* __restrict__ X, int64_t n,
                                                   int64_t off, int s,
                                                   int32_t* __restrict__ info) {
  __shared__ double Ls[NB][NB + 1];
  __shared__ double Rs[NB][NB + 1];
  __shared__ double colb[2][NB];
  __shared__ double rowb[2][NB];
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const int s1 = s < NB ? s : NB;
  const int s2 = s - s1;
  double a[4][4], x11[4][4];
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int i = ty + 16 * u, j = tx + 16 * v;
      a[u][v] = (i < s1 && j <= i) ? A[(off + i) * n + off + j] : (i == j ? 1.0 : 0.0);
    }
  chol_inv_regs(a, x11, s1, n, off, info, colb, rowb);
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int i = ty + 16 * u, j = tx + 16 * v;
      if (i < s1 && j < s1) X[(off + i) * n + off + j] = x11[u][v];
    }
  if (s2 <= 0) return;
  const int64_t o2 = off + NB;
  // T = A21 X11^T
  double t[4][4] = {};
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int i = ty + 16 * u, j = tx + 16 * v;
      Ls[i][j] = i < s2 ? A[(o2 + i) * n + off + j] : 0.0;
    }
  to_lds(Rs, x11);  // Rs[j][k] = X11(j, k)
  __syncthreads();
  mm64<true>(Ls, Rs, t);
  __syncthreads();
  // A22 -= T T^T (lower), M = T X11
  to_lds(Ls, t);  // Ls[i][k] = T(i, k)
  double a22[4][4], m[4][4] = {};
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int i = ty + 16 * u, j = tx + 16 * v;
      a22[u][v] = (i < s2 && j <= i) ? A[(o2 + i) * n + o2 + j] : (i == j ? 1.0 : 0.0);
    }
  __syncthreads();
  double tt[4][4] = {};
  mm64<true>(Ls, Ls, tt);  // sum_k T(i,k) T(j,k)
  mm64<false>(Ls, Rs, m);  // sum_k T(i,k) X11(k,j), Rs[k][j] = X11(k, j)
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int i = ty + 16 * u, j = tx + 16 * v;
      if (i < s2 && j <= i) a22[u][v] -= tt[u][v];
    }
  double x22[4][4];
  chol_inv_regs(a22, x22, s2, n, o2, info, colb, rowb);
  // X21 = -X22 M
  to_lds(Ls, x22);
  to_lds(Rs, m);
  __syncthreads();
  double x21[4][4] = {};
  mm64<false>(Ls, Rs, x21);
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int i = ty + 16 * u, j = tx + 16 * v;
      if (i < s2) {
        X[(o2 + i) * n + off + j] = -x21[u][v];
        if (j < s2) X[(o2 + i) * n + o2 + j] = x22[u][v];
      }
    }
}

// C = alpha * opA * opB + beta * C with v_mfma_f64_16x16x4_f64 on TILE x TILE
// output tiles (4 waves, each (TILE/2)^2), K staged through LDS in chunks of 32
// with the next chunk prefetched into registers.
// opA(i, k) = TA ? A[k * lda + i] : A[i * lda + k];
// opB(k, j) = TB ? B[j * ldb + k] : B[k * ldb + j].
// K range per tile for triangular operands: KLO_J: k >= j0; KHI_J: k < j0 + TILE;
// KHI_I: k < i0 + TILE (the skipped part is all zero; entries of a triangular
// operand inside the range but outside its triangle are stored zeros).
// LOWER: only tiles and entries with i >= j (M == N).  beta == 0 never reads C.
enum { KLO_J = 1, KHI_J = 2, KHI_I = 4 };

struct GemmArgs {
  const double* A;
  int64_t lda;
  const double* B;
  int64_t ldb;
  double* C;
  int64_t ldc;
  int64_t M, N, K;
  double alpha, beta;
  int kmode;
  int lower;
  int64_t tiles_n;
};

constexpr int GK = 32;

template <int TILE, bool TA, bool TB>
__global__ __launch_bounds__(256) void gemm_f64_kernel(GemmArgs g) {
  constexpr int HALF = TILE / 2;          // per-wave edge
  constexpr int SUB = HALF / 16;          // MFMA sub-tiles per wave edge
  constexpr int PER = GK * TILE / 256;    // staged elements per thread per operand
  __shared__ double As[GK][TILE + 1];
  __shared__ double Bs[GK][TILE + 1];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const int wr = wv >> 1, wc = wv & 1;
  int64_t ti, tj;
  if (g.lower) {
    const int64_t L = blockIdx.x;
    int64_t t = (int64_t)((sqrt(8.0 * (double)L + 1.0) - 1.0) * 0.5);
    while (t * (t + 1) / 2 > L) --t;
    while ((t + 1) * (t + 2) / 2 <= L) ++t;
    ti = t;
    tj = L - t * (t + 1) / 2;
  } else {
    ti = blockIdx.x / g.tiles_n;
    tj = blockIdx.x % g.tiles_n;
  }
  const int64_t i0 = ti * TILE, j0 = tj * TILE;
  int64_t kb = 0, ke = g.K;
  if (g.kmode & KLO_J) kb = j0;
  if (g.kmode & KHI_J) ke = min(ke, j0 + TILE);
  if (g.kmode & KHI_I) ke = min(ke, i0 + TILE);

  f64x4 acc[SUB][SUB];
#pragma unroll
  for (int a = 0; a < SUB; ++a)
#pragma unroll
    for (int b = 0; b < SUB; ++b) acc[a][b] = f64x4{0.0, 0.0, 0.0, 0.0};

  double ra[PER], rb[PER];
  auto fetch = [&](int64_t k0) {
#pragma unroll
    for (int r = 0; r < PER; ++r) {
      const int e = tid + 256 * r;
      int ii, kk;
      if (TA) { ii = e % TILE; kk = e / TILE; } else { kk = e % GK; ii = e / GK; }
      const int64_t gi = i0 + ii, gk = k0 + kk;
      ra[r] = (gi < g.M && gk < ke) ? (TA ? g.A[gk * g.lda + gi] : g.A[gi * g.lda + gk]) : 0.0;
    }
#pragma unroll
    for (int r = 0; r < PER; ++r) {
      const int e = tid + 256 * r;
      int jj, kk;
      if (TB) { kk = e % GK; jj = e / GK; } else { jj = e % TILE; kk = e / TILE; }
      const int64_t gj = j0 + jj, gk = k0 + kk;
      rb[r] = (gj < g.N && gk < ke) ? (TB ? g.B[gj * g.ldb + gk] : g.B[gk * g.ldb + gj]) : 0.0;
    }
  };
  auto stash = [&]() {
#pragma unroll
    for (int r = 0; r < PER; ++r) {
      const int e = tid + 256 * r;
      if (TA) As[e / TILE][e % TILE] = ra[r]; else As[e % GK][e / GK] = ra[r];
      if (TB) Bs[e % GK][e / GK] = rb[r]; else Bs[e / TILE][e % TILE] = rb[r];
    }
  };

  if (kb < ke) fetch(kb);
  for (int64_t k0 = kb; k0 < ke; k0 += GK) {
    __syncthreads();
    stash();
    __syncthreads();
    if (k0 + GK < ke) fetch(k0 + GK);
#pragma unroll
    for (int ks = 0; ks < GK; ks += 4) {
      double af[SUB], bf[SUB];
#pragma unroll
      for (int a = 0; a < SUB; ++a) af[a] = As[ks + (lane >> 4)][HALF * wr + 16 * a + (lane & 15)];
#pragma unroll
      for (int b = 0; b < SUB; ++b) bf[b] = Bs[ks + (lane >> 4)][HALF * wc + 16 * b + (lane & 15)];
#pragma unroll
      for (int a = 0; a < SUB; ++a)
#pragma unroll
        for (int b = 0; b < SUB; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f64_16x16x4f64(af[a], bf[b], acc[a][b], 0, 0, 0);
    }
  }
  // D layout of the f64 16x16x4 MFMA (measured): lane l, element q -> row l/16 + 4q,
  // column l%16 of the 16x16 tile (rows interleaved, unlike the f32 variant)
#pragma unroll
  for (int a = 0; a < SUB; ++a)
#pragma unroll
    for (int b = 0; b < SUB; ++b)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t gi = i0 + HALF * wr + 16 * a + (lane >> 4) + 4 * q;
        const int64_t gj = j0 + HALF * wc + 16 * b + (lane & 15);
        if (gi >= g.M || gj >= g.N) continue;
        if (g.lower && gj > gi) continue;
        double* c = g.C + gi * g.ldc + gj;
        const double v = g.alpha * acc[a][b][q];
        *c = g.beta == 0.0 ? v : fma(g.beta, *c, v);
      }
}

template <int TILE>
void launch_gemm_tile(const GemmArgs& g0, bool ta, bool tb, hipStream_t stream) {
  GemmArgs g = g0;
  const int64_t tm = ceil_div(g.M, TILE), tn = ceil_div(g.N, TILE);
  g.tiles_n = tn;
  const int64_t tiles = g.lower ? tm * (tm + 1) / 2 : tm * tn;
  if (tiles == 0) return;
  const dim3 grid((unsigned)tiles);
  if (!ta && !tb) hipLaunchKernelGGL((gemm_f64_kernel<TILE, false, false>), grid, dim3(256), 0, stream, g);
  else if (!ta && tb) hipLaunchKernelGGL((gemm_f64_kernel<TILE, false, true>), grid, dim3(256), 0, stream, g);
  else if (ta && !tb) hipLaunchKernelGGL((gemm_f64_kernel<TILE, true, false>), grid, dim3(256), 0, stream, g);
  else hipLaunchKernelGGL((gemm_f64_kernel<TILE, true, true>), grid, dim3(256), 0, stream, g);
}

hipError_t gemm(const double* A, int64_t lda, bool ta, const double* B, int64_t ldb, bool tb,
                double* C, int64_t ldc, int64_t M, int64_t N, int64_t K, double alpha, double beta,
                int kmode, bool lower, hipStream_t stream) {
  GemmArgs g;
  g.A = A; g.lda = lda; g.B = B; g.ldb = ldb; g.C = C; g.ldc = ldc;
  g.M = M; g.N = N; g.K = K; g.alpha = alpha; g.beta = beta; g.kmode = kmode;
  g.lower = lower ? 1 : 0;
  g.tiles_n = 0;
  // large problems: 128-wide tiles (better operand reuse) while they still fill the chip
  const bool big = ceil_div(M, 128) * ceil_div(N, 128) >= 192;
  if (big) launch_gemm_tile<128>(g, ta, tb, stream);
  else launch_gemm_tile<64>(g, ta, tb, stream);
  return hipGetLastError();
}

__global__ void fill_f64_kernel(double* __restrict__ p, int64_t count) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t k = i; k < count; k += stride) p[k] = 0.0;
}

// X[off:off+s, off:off+s] = inverse of the Cholesky factor of A[off:off+s, off:off+s].
hipError_t chol_inv(const PrepWs& w, int64_t n, int64_t off, int64_t s, int32_t* info,
                    hipStream_t stream) {
  if (s <= NODE) {
    hipLaunchKernelGGL(node_kernel, dim3(1), dim3(256), 0, stream, w.A, w.X, n, off, (int)s,
                       info);
    return hipGetLastError();
  }
  const int64_t s1 = split_first(s), s2 = s - s1;
  double* A21 = w.A + (off + s1) * n + off;
  double* A22 = w.A + (off + s1) * n + off + s1;
  const double* X11 = w.X + off * n + off;
  double* X21 = w.X + (off + s1) * n + off;
  const double* X22 = w.X + (off + s1) * n + off + s1;
  hipError_t e = chol_inv(w, n, off, s1, info, stream);
  if (e != hipSuccess) return e;
  // T = A21 X11^T   (X11(j, k) = 0 for k > j)
  e = gemm(A21, n, false, X11, n, true, w.T, s1, s2, s1, s1, 1.0, 0.0, KHI_J, false, stream);
  if (e != hipSuccess) return e;
  // A22 -= T T^T    (lower tiles)
  e = gemm(w.T, s1, false, w.T, s1, true, A22, n, s2, s2, s1, -1.0, 1.0, 0, true, stream);
  if (e != hipSuccess) return e;
  // A21 := T X11    (X11(k, j) = 0 for k < j)
  e = gemm(w.T, s1, false, X11, n, false, A21, n, s2, s1, s1, 1.0, 0.0, KLO_J, false, stream);
  if (e != hipSuccess) return e;
  e = chol_inv(w, n, off + s1, s2, info, stream);
  if (e != hipSuccess) return e;
  // X21 = -X22 A21  (X22(i, k) = 0 for k > i)
  return gemm(X22, n, false, A21, n, false, X21, n, s2, s1, s2, -1.0, 0.0, KHI_I, false, stream);
}

// U[k][l] = X[n-1-k][n-1-l] for l >= k (fp32), 0 below the diagonal.
__global__ __launch_bounds__(256) void write_u_kernel(const double* __restrict__ X, int64_t n,
                                                      float* __restrict__ U, int64_t ldu) {
  const int64_t l = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (l >= n) return;
  for (int64_t k = blockIdx.y; k < n; k += gridDim.y) {
    float v = 0.0f;
    if (l >= k) v = (float)X[(n - 1 - k) * n + (n - 1 - l)];
    U[k * ldu + l] = v;
  }
}

}  // namespace

size_t prepare_ws_bytes(int64_t n) {
  size_t b = 2 * align_up((size_t)n * n * sizeof(double), 256);
  b += align_up(t_elems(n) * sizeof(double), 256);
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
  // X's strict upper triangle must read as zero for the 128-wide GEMM tiles
  hipLaunchKernelGGL(fill_f64_kernel, dim3(2048), dim3(256), 0, stream, w.X, n * n);
  hipError_t e = chol_inv(w, n, 0, n, info, stream);
  if (e != hipSuccess) return e;
  {
    const dim3 grid((unsigned)ceil_div(n, 256), (unsigned)hmin(n, 2048));
    hipLaunchKernelGGL(write_u_kernel, grid, dim3(256), 0, stream, w.X, n, U, ldu);
  }
  return hipGetLastError();
}

}  // namespace gptq
