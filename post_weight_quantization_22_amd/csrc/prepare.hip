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
#include <mutex>

#include "kernels.hpp"

namespace gptq {

namespace {

constexpr int NB = 64;     // half of a diagonal node
constexpr int NODE = 128;  // subproblems up to this size run in one workgroup

typedef double f64x4 __attribute__((ext_vector_type(4)));

constexpr int MAXDEPTH = 24;

struct PrepWs {
  double* A;               // [n, n] lower: damped, permuted, reversed Hessian (overwritten)
  double* X;               // [n, n] lower: L^-1
  double* T[MAXDEPTH];     // per recursion depth: [s2, s1] of that depth's split
  double* diag;            // [n]
  double* lam;             // [1]
  int32_t* perm;           // [n]
};

int64_t split_first(int64_t s) {
  const int64_t blocks = ceil_div(s, NODE);
  return ((blocks + 1) / 2) * NODE;
}

// Largest T of each depth: t[d] = max over the depth-d splits of s2 * s1.
void t_sizes(int64_t s, int d, size_t (&t)[MAXDEPTH]) {
  if (s <= NODE || d >= MAXDEPTH) return;
  const int64_t s1 = split_first(s), s2 = s - s1;
  t[d] = hmax((int64_t)t[d], s1 * s2);
  t_sizes(s1, d + 1, t);
  t_sizes(s2, d + 1, t);
}

size_t t_bytes(int64_t n) {
  size_t t[MAXDEPTH] = {};
  t_sizes(n, 0, t);
  size_t b = 0;
  for (int d = 0; d < MAXDEPTH; ++d) b += align_up(t[d] * sizeof(double), 256);
  return b;
}

PrepWs carve(void* ws, int64_t n) {
  char* p = reinterpret_cast<char*>(ws);
  PrepWs w;
  w.A = reinterpret_cast<double*>(p);
  p += align_up((size_t)n * n * sizeof(double), 256);
  w.X = reinterpret_cast<double*>(p);
  p += align_up((size_t)n * n * sizeof(double), 256);
  size_t t[MAXDEPTH] = {};
  t_sizes(n, 0, t);
  for (int d = 0; d < MAXDEPTH; ++d) {
    w.T[d] = reinterpret_cast<double*>(p);
    p += align_up(t[d] * sizeof(double), 256);
  }
  w.diag = reinterpret_cast<double*>(p);
  p += align_up((size_t)n * sizeof(double), 256);
  w.lam = reinterpret_cast<double*>(p);
  p += 256;
  w.perm = reinterpret_cast<int32_t*>(p);
  return w;
}

// Second stream (default priority) for work off the critical path, with one
// pair of events per recursion depth; created once per device.
struct SideStream {
  hipStream_t s = nullptr;
  hipEvent_t t_done[MAXDEPTH];
  hipEvent_t m_done[MAXDEPTH];
};

hipError_t side_stream(SideStream*& out) {
  static std::mutex mu;
  static SideStream sides[64];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  SideStream& sd = sides[dev];
  if (!sd.s) {
    hipStream_t st;
    e = hipStreamCreateWithFlags(&st, hipStreamNonBlocking);
    if (e != hipSuccess) return e;
    for (int d = 0; d < MAXDEPTH; ++d) {
      e = hipEventCreateWithFlags(&sd.t_done[d], hipEventDisableTiming);
      if (e == hipSuccess) e = hipEventCreateWithFlags(&sd.m_done[d], hipEventDisableTiming);
      if (e != hipSuccess) return e;
    }
    sd.s = st;
  }
  out = &sd;
  return hipSuccess;
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
// Diagonal nodes (s <= 128) in one workgroup, everything in LDS.
//
// The serial part of the factorization is the column sweep inside the
// smallest blocks: column k of L needs every earlier column.  It runs on
// 32 x 32 leaves, each swept by ONE wave with no workgroup barrier: lane
// 32h + r owns row r, columns 16h .. 16h + 15, of A and of X = L^-1.  A step
// publishes column k of A (masked to the rows below the pivot, pivot in its
// own slot) and row k of X through LDS, whose requests a wave issues and
// completes in order, so the reads that follow see the writes.  Each lane then
// applies the right-looking Cholesky update a_ij -= l_ik l_jk = (a_ik / d) a_jk
// and the forward elimination of X, x_ij -= l_ik x_kj(final) = (a_ik / d) x_kj;
// row k of X becomes final as x_kj / l_kk.  Between the leaves the node
// combines halves with the same split as the recursion above it (64 = 32 +
// 32, 128 = 64 + 64), the products on v_mfma_f64_16x16x4_f64 from LDS.
// ---------------------------------------------------------------------------
constexpr int PS = NB + 1;  // LDS row stride of the 64 x 64 node buffers (doubles)

// 1/sqrt(d) in fp64: the hardware estimate refined by two Newton steps
// y <- y (3 - d y^2) / 2, each of which roughly squares the relative error.
__device__ __forceinline__ double rsqrt_f64(double d) {
  double y = __builtin_amdgcn_rsq(d);
  const double h = 0.5 * d;
  y = y * fma(-h * y, y, 1.5);
  y = y * fma(-h * y, y, 1.5);
  return y;
}

// One wave: Q (32 x 32, stride PS) = inverse of the Cholesky factor of the
// lower s x s block of P (stride PS), identity beyond s.  `pos` is the global
// index of the block's first row (for the non-positive pivot report).
// Lane 8 ty + tx owns the 4 x 4 entries (4 ty + u, 4 tx + v) of A and of X.
// All 32 steps always run: beyond s the block is the identity, whose steps
// change nothing.  The steps are software-pipelined: step k first updates
// what step k + 1 publishes (column k + 1 of A, row k + 1 of X and the next
// pivot, fetched with readlane so that its reciprocal square root is under
// way early), publishes it to LDS, and only then finishes its own rank-1
// update, which overlaps the LDS round trip.  The loop is unrolled by 4
// (compile-time register indices) inside a rolled loop of 8, small enough to
// stay in the instruction cache.  A non-positive or non-finite pivot is
// replaced by 1 and the first such position is reported once at the end.
__device__ __forceinline__ void leaf_publish(const double (&a)[4][4], const double (&x)[4][4],
                                             int kv, int k, int kb, int ty, int tx, int lane,
                                             double* cb, double* xb) {
  double cv[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) cv[u] = (4 * ty + u > k) ? a[u][kv] : 0.0;
  double* cdst = cb + (tx == kb ? 4 * ty : 40 + 4 * lane);
  *reinterpret_cast<double2*>(cdst) = make_double2(cv[0], cv[1]);
  *reinterpret_cast<double2*>(cdst + 2) = make_double2(cv[2], cv[3]);
  double* xdst = xb + (ty == kb ? 4 * tx : 40 + 4 * lane);
  *reinterpret_cast<double2*>(xdst) = make_double2(x[kv][0], x[kv][1]);
  *reinterpret_cast<double2*>(xdst + 2) = make_double2(x[kv][2], x[kv][3]);
}

// pivot a_kk (held by lane 9 (k / 4), register (k % 4, k % 4)) to every lane
__device__ __forceinline__ double leaf_pivot(double v, int kb) {
  const int src = (9 * kb) & 63;
  const int lo = __builtin_amdgcn_readlane(__double2loint(v), src);
  const int hi = __builtin_amdgcn_readlane(__double2hiint(v), src);
  return __hiloint2double(hi, lo);
}

__device__ __forceinline__ void leaf32(const double* P, double* Q, int s, double* cbuf,
                                       double* xbuf, int64_t n, int64_t pos, int32_t* info) {
  const int lane = threadIdx.x & 63;
  const int ty = lane >> 3, tx = lane & 7;
  double a[4][4], x[4][4];
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int i = 4 * ty + u, j = 4 * tx + v;
      const double val = P[i * PS + j];
      a[u][v] = (i < s && j <= i) ? val : (i == j ? 1.0 : 0.0);
      x[u][v] = i == j ? 1.0 : 0.0;
    }
  int first_bad = 32;
  // step 0's pivot and publication
  double d = leaf_pivot(a[0][0], 0);
  {
    const bool bad = !(d > 0.0) || !isfinite(d);
    first_bad = bad ? 0 : first_bad;
    d = bad ? 1.0 : d;
  }
  double rp = rsqrt_f64(d);
  leaf_publish(a, x, 0, 0, 0, ty, tx, lane, cbuf, xbuf);
#pragma unroll 1
  for (int kb = 0; kb < 8; ++kb) {
#pragma unroll
    for (int kv = 0; kv < 4; ++kv) {
      const int k = 4 * kb + kv;
      // LDS buffers alternate with the step parity: step k reads what step k - 1
      // published while it publishes step k + 1 into the other one
      const double* rc = cbuf + (kv & 1) * 348;
      const double* rx = xbuf + (kv & 1) * 348;
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      const double2 c01 = *reinterpret_cast<const double2*>(rc + 4 * ty);
      const double2 c23 = *reinterpret_cast<const double2*>(rc + 4 * ty + 2);
      const double2 j01 = *reinterpret_cast<const double2*>(rc + 4 * tx);
      const double2 j23 = *reinterpret_cast<const double2*>(rc + 4 * tx + 2);
      const double2 x01 = *reinterpret_cast<const double2*>(rx + 4 * tx);
      const double2 x23 = *reinterpret_cast<const double2*>(rx + 4 * tx + 2);
      const double rd = rp * rp;
      const double ci[4] = {c01.x * rd, c01.y * rd, c23.x * rd, c23.y * rd};  // l_ik / l_kk
      const double cj[4] = {j01.x, j01.y, j23.x, j23.y};                      // a_jk
      const double xk[4] = {x01.x, x01.y, x23.x, x23.y};                      // x_kj
      double cx[4];  // row k itself becomes x_kj / l_kk (its ci is zero, its xk its own row)
#pragma unroll
      for (int u = 0; u < 4; ++u) cx[u] = (4 * ty + u == k) ? rp - 1.0 : -ci[u];
      // What step k + 1 needs first: column k + 1 of A, row k + 1 of X, its
      // pivot.  After the last step this looks ahead to a column 32 that does
      // not exist: its lanes own nothing (everything goes to spare slots) and
      // the pivot is never used, so the same code serves every step.
      const int nv = (kv + 1) & 3;  // register column / row of step k + 1
      const int nkb = kb + (kv == 3 ? 1 : 0);
      {
#pragma unroll
        for (int u = 0; u < 4; ++u) a[u][nv] = fma(-ci[u], cj[nv], a[u][nv]);
#pragma unroll
        for (int v = 0; v < 4; ++v) x[nv][v] = fma(cx[nv], xk[v], x[nv][v]);
        d = leaf_pivot(a[nv][nv], nkb);
        const bool bad = !(d > 0.0) || !isfinite(d);
        first_bad = (bad && first_bad == 32) ? k + 1 : first_bad;
        d = bad ? 1.0 : d;
        leaf_publish(a, x, nv, k + 1, nkb, ty, tx, lane, cbuf + ((kv + 1) & 1) * 348,
                     xbuf + ((kv + 1) & 1) * 348);
      }
      // the rest of step k's update
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          if (v != nv) a[u][v] = fma(-ci[u], cj[v], a[u][v]);
          if (u != nv) x[u][v] = fma(cx[u], xk[v], x[u][v]);
        }
      rp = rsqrt_f64(d);
    }
  }
  if (lane == 0 && first_bad < s && *info == 0) *info = (int32_t)(n - (pos + first_bad));
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int v = 0; v < 4; ++v) Q[(4 * ty + u) * PS + 4 * tx + v] = x[u][v];
}

// One 16 x 16 tile of a product with K <= 32 on v_mfma_f64_16x16x4_f64:
// sum_{kmin <= k < kmax} P(i0 + i, k) Q(k, j0 + j), P(i, k) = P[i * PS + k],
// Q(k, j) = QT ? Qm[j * PS + k] : Qm[k * PS + j].  Element q of lane l is
// (i0 + l/16 + 4q, j0 + l%16).
template <bool QT>
__device__ __forceinline__ f64x4 tile16(const double* P, const double* Qm, int i0, int j0,
                                        int kmin, int kmax) {
  const int lane = threadIdx.x & 63;
  f64x4 acc = {0.0, 0.0, 0.0, 0.0};
  for (int k0 = kmin; k0 < kmax; k0 += 4) {
    const int kl = k0 + (lane >> 4);
    const double av = P[(i0 + (lane & 15)) * PS + kl];
    const double bv = QT ? Qm[(j0 + (lane & 15)) * PS + kl] : Qm[kl * PS + j0 + (lane & 15)];
    acc = __builtin_amdgcn_mfma_f64_16x16x4f64(av, bv, acc, 0, 0, 0);
  }
  return acc;
}

// Q (64 x 64 lower, stride PS) = inverse of the Cholesky factor of the lower
// s x s block of P (stride PS, rows/cols >= s zero); P is overwritten.
// 64 = 32 + 32: X11 = leaf(A11); T = A21 X11^T; A22 -= T T^T; M = T X11;
// X22 = leaf(A22); X21 = -X22 M.  Wave w owns 16 x 16 tile (w / 2, w % 2) of
// each 32 x 32 product.  The two leaves share one copy of the leaf code (a
// rolled loop over the halves).
__device__ __forceinline__ void node64(double* P, double* Q, int s, double* cbuf, double* xbuf,
                                       int64_t n, int64_t pos, int32_t* info) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int s1 = s < 32 ? s : 32, s2 = s - s1;
  const int ti = wv >> 1, tj = wv & 1;
  const int rr = lane >> 4, cc = lane & 15;
  double* A21 = P + 32 * PS;
  double* A22 = P + 32 * PS + 32;
  double* X21 = Q + 32 * PS;
  double* X22 = Q + 32 * PS + 32;
#pragma unroll 1
  for (int half = 0; half < 2; ++half) {
    if (wv == 0) {
      leaf32(half ? A22 : P, half ? X22 : Q, half ? s2 : s1, cbuf, xbuf, n, pos + 32 * half, info);
    } else if (half == 0) {
      // the block right of X11 is zero (read as such by the products above)
      for (int e = threadIdx.x - 64; e < 32 * 32; e += 192) Q[(e >> 5) * PS + 32 + (e & 31)] = 0.0;
    }
    __syncthreads();
    if (s2 <= 0) return;
    if (half == 0) {
      {  // T = A21 X11^T (X11(j, k) = 0 for k > j) into the free X21 block
        const f64x4 t = tile16<true>(A21, Q, 16 * ti, 16 * tj, 0, 16 * tj + 16);
#pragma unroll
        for (int q = 0; q < 4; ++q) X21[(16 * ti + rr + 4 * q) * PS + 16 * tj + cc] = t[q];
      }
      __syncthreads();
      {  // A22 -= T T^T (lower tiles) in place; M = T X11 (X11(k, j) = 0 for k < j) over A21
        const f64x4 m = tile16<false>(X21, Q, 16 * ti, 16 * tj, 16 * tj, 32);
        if (wv < 3) {
          const int si = wv == 0 ? 0 : 1, sj = wv == 2 ? 1 : 0;
          const f64x4 t = tile16<true>(X21, X21, 16 * si, 16 * sj, 0, 32);
#pragma unroll
          for (int q = 0; q < 4; ++q) A22[(16 * si + rr + 4 * q) * PS + 16 * sj + cc] -= t[q];
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) A21[(16 * ti + rr + 4 * q) * PS + 16 * tj + cc] = m[q];
      }
      __syncthreads();
    } else {
      // X21 = -X22 M (X22(i, k) = 0 for k > i), over T
      const f64x4 x = tile16<false>(X22, A21, 16 * ti, 16 * tj, 0, 16 * ti + 16);
#pragma unroll
      for (int q = 0; q < 4; ++q) X21[(16 * ti + rr + 4 * q) * PS + 16 * tj + cc] = -x[q];
      __syncthreads();
    }
  }
}

// 64 x 64 x 64 products on v_mfma_f64_16x16x4_f64 with both operands in LDS.
// Wave w computes the 32 x 32 quadrant (32 (w / 2), 32 (w % 2)) as 2 x 2 tiles:
// acc[a][b] = sum_k P(i, k) Q(k, j), P read as Ps[i][k], Q as Qs[k][j]
// (QT == false) or Qs[j][k] (QT == true).  MODE skips what is structurally
// zero: MF_KHI_J k <= j (Q lower-triangular, transposed), MF_KLO_J k >= j (Q
// lower-triangular), MF_KHI_I k <= i (P lower-triangular), MF_LOWER only the
// tiles on or below the diagonal (the rest of acc stays zero).
enum { MF_FULL = 0, MF_KHI_J = 1, MF_KLO_J = 2, MF_KHI_I = 3, MF_LOWER = 4 };

template <bool QT, int MODE>
__device__ __forceinline__ void mfma64(const double (*Ps)[PS], const double (*Qs)[PS],
                                       f64x4 (&acc)[2][2]) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int wr = wv >> 1, wc = wv & 1;
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = f64x4{0.0, 0.0, 0.0, 0.0};
  if (MODE == MF_LOWER && wr < wc) return;
  int kmin = 0, kmax = NB;
  if (MODE == MF_KHI_J) kmax = 32 * wc + 32;
  if (MODE == MF_KLO_J) kmin = 32 * wc;
  if (MODE == MF_KHI_I) kmax = 32 * wr + 32;
#pragma unroll
  for (int k0 = 0; k0 < NB; k0 += 4) {
    if (k0 < kmin || k0 >= kmax) continue;  // uniform per wave
    const int kl = k0 + (lane >> 4);
    double af[2], bf[2];
#pragma unroll
    for (int a = 0; a < 2; ++a) af[a] = Ps[32 * wr + 16 * a + (lane & 15)][kl];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int j = 32 * wc + 16 * b + (lane & 15);
      bf[b] = QT ? Qs[j][kl] : Qs[kl][j];
    }
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        bool on = true;
        if (MODE == MF_KHI_J) on = k0 < 32 * wc + 16 * b + 16;
        if (MODE == MF_KLO_J) on = k0 >= 32 * wc + 16 * b;
        if (MODE == MF_KHI_I) on = k0 < 32 * wr + 16 * a + 16;
        if (MODE == MF_LOWER) on = !(wr == wc && a < b);
        if (on) acc[a][b] = __builtin_amdgcn_mfma_f64_16x16x4f64(af[a], bf[b], acc[a][b], 0, 0, 0);
      }
  }
}

// Row and column of element q of tile (a, b) of this wave's quadrant.  D layout
// of the f64 16x16x4 MFMA (measured): lane l, element q -> row l/16 + 4q,
// column l%16.
__device__ __forceinline__ int mfma_row(int a, int q) {
  const int lane = threadIdx.x & 63, wr = (threadIdx.x >> 6) >> 1;
  return 32 * wr + 16 * a + (lane >> 4) + 4 * q;
}
__device__ __forceinline__ int mfma_col(int b) {
  const int lane = threadIdx.x & 63, wc = (threadIdx.x >> 6) & 1;
  return 32 * wc + 16 * b + (lane & 15);
}

__device__ __forceinline__ void acc_to_lds(double (*D)[PS], const f64x4 (&acc)[2][2]) {
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int q = 0; q < 4; ++q) D[mfma_row(a, q)][mfma_col(b)] = acc[a][b][q];
}

// A node of size s <= 128 in one workgroup: X[off:off+s, off:off+s] = inverse of
// the Cholesky factor of A[off:off+s, off:off+s], by the split 64 + rest: two
// 64-nodes in LDS and the four 64 x 64 products between them.  The three
// blocks of A come in at the start, every load in flight at once.
__device__ __forceinline__ void load_block64(const double* __restrict__ A, int64_t n, int64_t r0,
                                             int64_t c0, int rows, int cols, bool lower,
                                             double (*B)[PS]) {
  // thread t covers rows t / 16 + 16 m (m = 0..3), columns 4 (t % 16) .. + 3
  const int t = threadIdx.x;
  const int jc = 4 * (t & 15);
  double v[4][4];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int i = (t >> 4) + 16 * m;
    const int64_t gi = r0 + (i < rows ? i : 0);
#pragma unroll
    for (int q = 0; q < 4; ++q) v[m][q] = A[gi * n + c0 + (jc + q < cols ? jc + q : 0)];
  }
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int i = (t >> 4) + 16 * m;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int j = jc + q;
      B[i][j] = (i < rows && j < cols && (!lower || j <= i)) ? v[m][q] : 0.0;
    }
  }
}

__global__ __launch_bounds__(256) void node_kernel(const double* __restrict__ A,
                                                   double* __restrict__ X, int64_t n,
                                                   int64_t off, int s,
                                                   int32_t* __restrict__ info) {
  __shared__ double B0[NB][PS];
  __shared__ double B1[NB][PS];
  __shared__ double B2[NB][PS];
  __shared__ double B3[NB][PS];
  __shared__ __align__(16) double cbuf[2 * 348];
  __shared__ __align__(16) double xbuf[2 * 348];
  const int tid = threadIdx.x;
  const int s1 = s < NB ? s : NB;
  const int s2 = s - s1;
  const int64_t o2 = off + NB;
  load_block64(A, n, off, off, s1, s1, true, B0);  // A11
  if (s2 > 0) {
    load_block64(A, n, o2, off, s2, s1, false, B2);  // A21
    load_block64(A, n, o2, o2, s2, s2, true, B3);    // A22
  }
  __syncthreads();
#pragma unroll 1
  for (int half = 0; half < 2; ++half) {
    const int sh = half ? s2 : s1;
    const int64_t oh = half ? o2 : off;
    node64(half ? &B3[0][0] : &B0[0][0], &B1[0][0], sh, cbuf, xbuf, n, oh, info);  // X11 / X22 -> B1
    for (int e = tid; e < NB * NB; e += 256) {
      const int i = e / NB, j = e % NB;
      if (i < sh && j <= i) X[(oh + i) * n + oh + j] = B1[i][j];
    }
    if (s2 <= 0) return;
    f64x4 acc[2][2];
    if (half == 0) {
      mfma64<true, MF_KHI_J>(B2, B1, acc);  // T = A21 X11^T
      acc_to_lds(B0, acc);
      __syncthreads();
      f64x4 accm[2][2];
      mfma64<true, MF_LOWER>(B0, B0, acc);    // T T^T (lower)
      mfma64<false, MF_KLO_J>(B0, B1, accm);  // M = T X11
      __syncthreads();
      // A22 -= T T^T in place (B3), M -> B0
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int i = mfma_row(a, q), j = mfma_col(b);
            if (i < s2 && j <= i) B3[i][j] -= acc[a][b][q];
          }
      acc_to_lds(B0, accm);
      __syncthreads();
    } else {
      mfma64<false, MF_KHI_I>(B1, B0, acc);  // X21 = -X22 M
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int i = mfma_row(a, q), j = mfma_col(b);
            if (i < s2) X[(o2 + i) * n + off + j] = -acc[a][b][q];
          }
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
  int64_t tiles_m, tiles_n;
};

constexpr int GK = 32;

// Tile (ti, tj) of workgroup `bid`.  With a triangular operand the K range of
// a tile depends on its column (or row) and varies up to the whole K; tiles
// are numbered longest range first so that in-order dispatch balances the CUs.
__device__ __forceinline__ void gemm_tile_of(const GemmArgs& g, int64_t bid, int64_t& ti,
                                             int64_t& tj) {
  if (g.lower) {
    int64_t t = (int64_t)((sqrt(8.0 * (double)bid + 1.0) - 1.0) * 0.5);
    while (t * (t + 1) / 2 > bid) --t;
    while ((t + 1) * (t + 2) / 2 <= bid) ++t;
    ti = t;
    tj = bid - t * (t + 1) / 2;
  } else if (g.kmode & KHI_J) {
    tj = g.tiles_n - 1 - bid / g.tiles_m;
    ti = bid % g.tiles_m;
  } else if (g.kmode & KLO_J) {
    tj = bid / g.tiles_m;
    ti = bid % g.tiles_m;
  } else if (g.kmode & KHI_I) {
    ti = g.tiles_m - 1 - bid / g.tiles_n;
    tj = bid % g.tiles_n;
  } else {
    ti = bid / g.tiles_n;
    tj = bid % g.tiles_n;
  }
}

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
  gemm_tile_of(g, blockIdx.x, ti, tj);
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
  g.tiles_m = tm;
  g.tiles_n = tn;
  const int64_t tiles = g.lower ? tm * (tm + 1) / 2 : tm * tn;
  if (tiles == 0) return;
  const dim3 grid((unsigned)tiles);
  if (!ta && !tb) hipLaunchKernelGGL((gemm_f64_kernel<TILE, false, false>), grid, dim3(256), 0, stream, g);
  else if (!ta && tb) hipLaunchKernelGGL((gemm_f64_kernel<TILE, false, true>), grid, dim3(256), 0, stream, g);
  else if (ta && !tb) hipLaunchKernelGGL((gemm_f64_kernel<TILE, true, false>), grid, dim3(256), 0, stream, g);
  else hipLaunchKernelGGL((gemm_f64_kernel<TILE, true, true>), grid, dim3(256), 0, stream, g);
}

// Latency-bound products (the lower levels of the recursion): TILE x TILE
// output tiles, the K range of a tile split over the 4 waves in chunks of 16
// (wave w takes chunks w, w + 4, ...).  Fragments go from global memory (L2)
// straight into registers, the next chunk in flight while the current one is
// multiplied; the four partial tiles are summed through LDS in a fixed order
// (deterministic).  A is never transposed; opB as in gemm_f64_kernel.
template <int TILE, bool TB>
__global__ __launch_bounds__(256) void gemm_splitk_kernel(GemmArgs g) {
  constexpr int SUB = TILE / 16;
  __shared__ double red[3 * TILE * TILE];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int r = lane & 15, kq = lane >> 4;
  int64_t ti, tj;
  gemm_tile_of(g, blockIdx.x, ti, tj);
  const int64_t i0 = ti * TILE, j0 = tj * TILE;
  int64_t kb = 0, ke = g.K;
  if (g.kmode & KLO_J) kb = j0;
  if (g.kmode & KHI_J) ke = min(ke, j0 + TILE);
  if (g.kmode & KHI_I) ke = min(ke, i0 + TILE);

  // operand rows / columns of this lane; out-of-range ones read row 0 and are zeroed
  const double* pa[SUB];
  const double* pb[SUB];
  bool va[SUB], vb[SUB];
#pragma unroll
  for (int a = 0; a < SUB; ++a) {
    const int64_t i = i0 + 16 * a + r;
    va[a] = i < g.M;
    pa[a] = g.A + (va[a] ? i : 0) * g.lda;
  }
#pragma unroll
  for (int b = 0; b < SUB; ++b) {
    const int64_t j = j0 + 16 * b + r;
    vb[b] = j < g.N;
    pb[b] = TB ? g.B + (vb[b] ? j : 0) * g.ldb : g.B + (vb[b] ? j : 0);
  }
  auto load = [&](int64_t c0, double (&af)[4][SUB], double (&bf)[4][SUB]) {
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const int64_t k = c0 + 4 * st + kq;
      const bool kin = k < ke;
      const int64_t kc = kin ? k : kb;
#pragma unroll
      for (int a = 0; a < SUB; ++a) {
        const double v = pa[a][kc];
        af[st][a] = (kin && va[a]) ? v : 0.0;
      }
#pragma unroll
      for (int b = 0; b < SUB; ++b) {
        const double v = TB ? pb[b][kc] : pb[b][kc * g.ldb];
        bf[st][b] = (kin && vb[b]) ? v : 0.0;
      }
    }
  };

  f64x4 acc[SUB][SUB];
#pragma unroll
  for (int a = 0; a < SUB; ++a)
#pragma unroll
    for (int b = 0; b < SUB; ++b) acc[a][b] = f64x4{0.0, 0.0, 0.0, 0.0};
  double af[4][SUB], bf[4][SUB];
  int64_t c0 = kb + 16 * wv;
  if (c0 < ke) load(c0, af, bf);
  for (; c0 < ke; c0 += 64) {
    double an[4][SUB], bn[4][SUB];
    const bool more = c0 + 64 < ke;
    if (more) load(c0 + 64, an, bn);
#pragma unroll
    for (int st = 0; st < 4; ++st)
#pragma unroll
      for (int a = 0; a < SUB; ++a)
#pragma unroll
        for (int b = 0; b < SUB; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f64_16x16x4f64(af[st][a], bf[st][b], acc[a][b], 0, 0, 0);
    if (more) {
#pragma unroll
      for (int st = 0; st < 4; ++st)
#pragma unroll
        for (int a = 0; a < SUB; ++a) {
          af[st][a] = an[st][a];
          bf[st][a] = bn[st][a];
        }
    }
  }
  if (wv > 0) {
#pragma unroll
    for (int a = 0; a < SUB; ++a)
#pragma unroll
      for (int b = 0; b < SUB; ++b)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          red[(((wv - 1) * SUB * SUB + a * SUB + b) * 4 + q) * 64 + lane] = acc[a][b][q];
  }
  __syncthreads();
  if (wv != 0) return;
#pragma unroll
  for (int a = 0; a < SUB; ++a)
#pragma unroll
    for (int b = 0; b < SUB; ++b)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        double v = acc[a][b][q];
#pragma unroll
        for (int w = 0; w < 3; ++w) v += red[((w * SUB * SUB + a * SUB + b) * 4 + q) * 64 + lane];
        // D layout of the f64 16x16x4 MFMA: row l/16 + 4q, column l%16
        const int64_t gi = i0 + 16 * a + kq + 4 * q;
        const int64_t gj = j0 + 16 * b + r;
        if (gi >= g.M || gj >= g.N) continue;
        if (g.lower && gj > gi) continue;
        double* c = g.C + gi * g.ldc + gj;
        const double o = g.alpha * v;
        *c = g.beta == 0.0 ? o : fma(g.beta, *c, o);
      }
}

template <int TILE>
void launch_splitk(const GemmArgs& g0, bool tb, hipStream_t stream) {
  GemmArgs g = g0;
  const int64_t tm = ceil_div(g.M, TILE), tn = ceil_div(g.N, TILE);
  g.tiles_m = tm;
  g.tiles_n = tn;
  const int64_t tiles = g.lower ? tm * (tm + 1) / 2 : tm * tn;
  if (tiles == 0) return;
  if (tb) hipLaunchKernelGGL((gemm_splitk_kernel<TILE, true>), dim3((unsigned)tiles), dim3(256), 0, stream, g);
  else hipLaunchKernelGGL((gemm_splitk_kernel<TILE, false>), dim3((unsigned)tiles), dim3(256), 0, stream, g);
}

hipError_t gemm(const double* A, int64_t lda, bool ta, const double* B, int64_t ldb, bool tb,
                double* C, int64_t ldc, int64_t M, int64_t N, int64_t K, double alpha, double beta,
                int kmode, bool lower, hipStream_t stream) {
  GemmArgs g;
  g.A = A; g.lda = lda; g.B = B; g.ldb = ldb; g.C = C; g.ldc = ldc;
  g.M = M; g.N = N; g.K = K; g.alpha = alpha; g.beta = beta; g.kmode = kmode;
  g.lower = lower ? 1 : 0;
  g.tiles_m = g.tiles_n = 0;
  // Up to 256 tiles of 32 x 32 (the lower levels of the recursion, bound by
  // latency) the split-K kernel; above, 64-wide tiles staged through LDS,
  // dispatched longest K range first.  (Measured on the levels n/2 .. 128 of a
  // 4096 factorization; 128-wide tiles lost at every size.)
  if (!ta && ceil_div(M, 32) * ceil_div(N, 32) <= 256) launch_splitk<32>(g, tb, stream);
  else launch_gemm_tile<64>(g, ta, tb, stream);
  return hipGetLastError();
}

__global__ void fill_f64_kernel(double* __restrict__ p, int64_t count) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t k = i; k < count; k += stride) p[k] = 0.0;
}

// X[off:off+s, off:off+s] = inverse of the Cholesky factor of A[off:off+s, off:off+s].
// M = T X11 is needed only by the last product, so it runs on the side stream
// while the main stream goes on with A22 -= T T^T and the whole recursion on
// A22 (mostly single-CU nodes and small products, which leave the chip idle).
// T has one buffer per depth: a depth's splits follow each other, and each
// joins its side work before returning.
hipError_t chol_inv(const PrepWs& w, int64_t n, int64_t off, int64_t s, int d, int32_t* info,
                    hipStream_t stream, SideStream* side) {
  if (s <= NODE) {
    hipLaunchKernelGGL(node_kernel, dim3(1), dim3(256), 0, stream, w.A, w.X, n, off, (int)s,
                       info);
    return hipGetLastError();
  }
  if (d >= MAXDEPTH) return hipErrorInvalidValue;
  const int64_t s1 = split_first(s), s2 = s - s1;
  double* A21 = w.A + (off + s1) * n + off;
  double* A22 = w.A + (off + s1) * n + off + s1;
  const double* X11 = w.X + off * n + off;
  double* X21 = w.X + (off + s1) * n + off;
  const double* X22 = w.X + (off + s1) * n + off + s1;
  double* T = w.T[d];
  hipError_t e = chol_inv(w, n, off, s1, d + 1, info, stream, side);
  if (e != hipSuccess) return e;
  // T = A21 X11^T   (X11(j, k) = 0 for k > j)
  e = gemm(A21, n, false, X11, n, true, T, s1, s2, s1, s1, 1.0, 0.0, KHI_J, false, stream);
  if (e != hipSuccess) return e;
  // A21 := T X11    (X11(k, j) = 0 for k < j), on the side stream
  if ((e = hipEventRecord(side->t_done[d], stream)) != hipSuccess) return e;
  if ((e = hipStreamWaitEvent(side->s, side->t_done[d], 0)) != hipSuccess) return e;
  e = gemm(T, s1, false, X11, n, false, A21, n, s2, s1, s1, 1.0, 0.0, KLO_J, false, side->s);
  if (e != hipSuccess) return e;
  if ((e = hipEventRecord(side->m_done[d], side->s)) != hipSuccess) return e;
  // A22 -= T T^T    (lower tiles)
  e = gemm(T, s1, false, T, s1, true, A22, n, s2, s2, s1, -1.0, 1.0, 0, true, stream);
  if (e != hipSuccess) return e;
  e = chol_inv(w, n, off + s1, s2, d + 1, info, stream, side);
  if (e != hipSuccess) return e;
  // X21 = -X22 A21  (X22(i, k) = 0 for k > i)
  if ((e = hipStreamWaitEvent(stream, side->m_done[d], 0)) != hipSuccess) return e;
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
  b += t_bytes(n);
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
  SideStream* side = nullptr;
  hipError_t e = side_stream(side);
  if (e != hipSuccess) return e;
  e = chol_inv(w, n, 0, n, 0, info, stream, side);
  if (e != hipSuccess) return e;
  {
    const dim3 grid((unsigned)ceil_div(n, 256), (unsigned)hmin(n, 2048));
    hipLaunchKernelGGL(write_u_kernel, grid, dim3(256), 0, stream, w.X, n, U, ldu);
  }
  return hipGetLastError();
}

}  // namespace gptq
