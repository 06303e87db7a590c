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
// X = L^-1 in two phases, with 128-wide blocks (block k = rows 128k ..).
//
// 1. Blocked Cholesky in outer blocks of ob 128-wide blocks (ob = 4 for
//    large n, else 1).  Step k: the diagonal node kernel turns the (fully
//    updated) block A_kk into X_kk = L_kk^-1 in one workgroup; the panel
//    L_ik = A_ik X_kk^T (i > k) is a GEMM, stored in X's block (i, k); the
//    updates A_ij -= L_ik L_jk^T follow from A = L L^T.  Inside an outer
//    block they are applied left-looking (block k's columns take the outer
//    block's earlier panels just before its node); past it, once per outer
//    block with K = 128 ob: the next outer block's columns on the main stream
//    (the lookahead), the rest of the trailing matrix on a side stream, where
//    it overlaps the next outer block.  Before its next lookahead the main
//    stream waits for that side update (both write those columns).
// 2. X = L^-1 by groups of GRP blocks (rows c .. c + 128 GRP; GRP = 8 for
//    n >= 16384, else 4), from L X = I:
//    X[g, 0:c] = -X_gg L[g, 0:c] X[0:c, 0:c].  Per group, on a third stream:
//      X_gg, the inverse of the group's own diagonal block, joins the nodes'
//      X_ii pairwise: for a split [[L11, 0], [L21, L22]] the inverse is
//      [[X11, 0], [-X22 L21 X11, X22]] (M = L21 X11, X21 = -X22 M);
//      M_g = L[g, 0:c] X[0:c, 0:c] needs only the panels of L in the
//      group's rows (all written before the group's first node) and the
//      groups above, so it runs while the group's nodes are factored;
//      X[g, 0:c] = -X_gg M_g once X_gg exists.
//    So all that follows the last node is the last group's joins and one
//    product.  L's blocks sit in X's lower blocks and are overwritten by X's.
//
// The products run on v_mfma_f64_16x16x4_f64, so no kernel carries a long
// serial reduction; the serial part is the chain of 128-wide nodes.
#include <mutex>

#include "kernels.hpp"

namespace gptq {

namespace {

constexpr int NB = 64;     // half of a diagonal node
constexpr int NODE = 128;  // subproblems up to this size run in one workgroup

typedef double f64x4 __attribute__((ext_vector_type(4)));

struct PrepWs {
  double* A;               // [n, n] lower: damped, permuted, reversed Hessian (overwritten)
  double* X;               // [n, n] lower: L^-1 (holds the panels of L while phase 1 runs)
  double* M;               // phase-2 products: M_g, then the joins' M
  double* diag;            // [n]
  double* lam;             // [1]
  int32_t* perm;           // [n]
  int32_t* rank;           // [n] descending-order rank of each column (desc_act)
  double* skey;            // [n rounded up to RANK_CHUNK] keys sorted within chunks (desc_act)
  int32_t* sidx;           // [same] their columns
};

// Blocks per group of the inverse: a group's head product M_g reads the
// whole inverse above it once for every 128 of its rows, so larger groups
// read it fewer times; smaller ones leave less after the last node (the last
// group's joins and product), which bounds small n.
int64_t grp_blocks(int64_t n) { return n >= 16384 ? 8 : 4; }

// Phase-2 product buffers: M_g ([GRP NODE, n]) and the joins' M (at most
// [GRP/2 NODE, GRP/2 NODE]).
int64_t m_elems(int64_t n) {
  const int64_t g = grp_blocks(n);
  return n > NODE ? g * NODE * n + (g / 2) * (g / 2) * NODE * NODE : 0;
}

constexpr int RANK_CHUNK = 1024;  // keys per sorted chunk of the desc_act order
int64_t rank_pad(int64_t n) { return ceil_div(n, (int64_t)RANK_CHUNK) * RANK_CHUNK; }

PrepWs carve(void* ws, int64_t n) {
  char* p = reinterpret_cast<char*>(ws);
  PrepWs w;
  w.A = reinterpret_cast<double*>(p);
  p += align_up((size_t)n * n * sizeof(double), 256);
  w.X = reinterpret_cast<double*>(p);
  p += align_up((size_t)n * n * sizeof(double), 256);
  w.M = reinterpret_cast<double*>(p);
  p += align_up((size_t)m_elems(n) * sizeof(double), 256);
  w.diag = reinterpret_cast<double*>(p);
  p += align_up((size_t)n * sizeof(double), 256);
  w.lam = reinterpret_cast<double*>(p);
  p += 256;
  w.perm = reinterpret_cast<int32_t*>(p);
  p += align_up((size_t)n * sizeof(int32_t), 256);
  w.rank = reinterpret_cast<int32_t*>(p);
  p += align_up((size_t)n * sizeof(int32_t), 256);
  w.skey = reinterpret_cast<double*>(p);
  p += align_up((size_t)rank_pad(n) * sizeof(double), 256);
  w.sidx = reinterpret_cast<int32_t*>(p);
  return w;
}

// Two more streams (default priority), one for the trailing updates and one
// for the block rows of the inverse, and the events that order them against
// the main stream; created once per device.
struct SideStream {
  hipStream_t s = nullptr;    // trailing updates
  hipStream_t inv = nullptr;  // block rows of X
  hipEvent_t step_done;       // main -> s, inv: an outer block's panels and lookahead are done
  hipEvent_t trailing_done;   // s -> main: the trailing update is applied
  hipEvent_t last_node;       // main -> inv: the last node is done
  hipEvent_t inv_done;        // inv -> main: the last group of X is written
  std::mutex run;             // one call at a time enqueues on a device's side streams
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
    hipStream_t st, si;
    e = hipStreamCreateWithFlags(&st, hipStreamNonBlocking);
    if (e != hipSuccess) return e;
    e = hipStreamCreateWithFlags(&si, hipStreamNonBlocking);
    if (e != hipSuccess) return e;
    for (hipEvent_t* ev : {&sd.step_done, &sd.trailing_done, &sd.last_node, &sd.inv_done}) {
      e = hipEventCreateWithFlags(ev, hipEventDisableTiming);
      if (e != hipSuccess) return e;
    }
    sd.inv = si;
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
                                                         int32_t* __restrict__ rank,
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
    if (rank) rank[i] = 0;
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

// Stable descending order of diag.  The key of column i is its diagonal
// entry, with a NaN taken as -inf, so that the keys are totally ordered:
// column j precedes column i when key_j > key_i, or key_j == key_i and j < i,
// and rank_i, the number of columns preceding i, is a permutation of
// 0 .. n-1 whatever the values (a non-finite diagonal is reported through
// info by diag_damp_kernel; the order stays well formed).  The count goes
// through sorted chunks: chunk_sort_kernel sorts each run of RANK_CHUNK
// columns into that order in LDS (bitonic; padding entries (-inf, INT32_MAX)
// sort last and precede nothing), then rank_search_kernel gives each column,
// for each sorted chunk, the number of its entries that precede the column
// (a binary search in LDS), added to rank[i] (zeroed by diag_damp_kernel).
// n^2 / RANK_CHUNK log2(RANK_CHUNK) comparisons instead of n^2.
// rank_scatter_kernel then writes perm.
__device__ __forceinline__ double order_key(double d) { return d != d ? -INFINITY : d; }

__device__ __forceinline__ bool precedes(double ka, int32_t ia, double kb, int32_t ib) {
  return ka > kb || (ka == kb && ia < ib);
}

__global__ __launch_bounds__(512) void chunk_sort_kernel(const double* __restrict__ diag,
                                                         int64_t n, double* __restrict__ skey,
                                                         int32_t* __restrict__ sidx) {
  __shared__ double k[RANK_CHUNK];
  __shared__ int32_t x[RANK_CHUNK];
  const int t = threadIdx.x;
  const int64_t base = (int64_t)blockIdx.x * RANK_CHUNK;
  for (int e = t; e < RANK_CHUNK; e += 512) {
    const int64_t j = base + e;
    k[e] = j < n ? order_key(diag[j]) : -INFINITY;
    x[e] = j < n ? (int32_t)j : INT32_MAX;
  }
  __syncthreads();
  // 512 pairs a step: pair t is (lo, lo + stride); blocks of `size` alternate
  // direction until the last merge
  for (int size = 2; size <= RANK_CHUNK; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      const int lo = 2 * t - (t & (stride - 1)), hi = lo + stride;
      const double ka = k[lo], kb = k[hi];
      const int32_t ia = x[lo], ib = x[hi];
      const bool up = (lo & size) == 0;
      if (up ? precedes(kb, ib, ka, ia) : precedes(ka, ia, kb, ib)) {
        k[lo] = kb;
        k[hi] = ka;
        x[lo] = ib;
        x[hi] = ia;
      }
      __syncthreads();
    }
  }
  for (int e = t; e < RANK_CHUNK; e += 512) {
    skey[base + e] = k[e];
    sidx[base + e] = x[e];
  }
}

__global__ __launch_bounds__(256) void rank_search_kernel(const double* __restrict__ diag,
                                                          int64_t n,
                                                          const double* __restrict__ skey,
                                                          const int32_t* __restrict__ sidx,
                                                          int32_t* __restrict__ rank) {
  __shared__ double k[RANK_CHUNK];
  __shared__ int32_t x[RANK_CHUNK];
  const int64_t base = (int64_t)blockIdx.y * RANK_CHUNK;
  for (int e = threadIdx.x; e < RANK_CHUNK; e += 256) {
    k[e] = skey[base + e];
    x[e] = sidx[base + e];
  }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int64_t i = (int64_t)blockIdx.x * 1024 + threadIdx.x + 256 * u;
    if (i >= n) continue;
    const double ki = order_key(diag[i]);
    // entries [0, lo) precede column i, entries [hi, RANK_CHUNK) do not
    int lo = 0, hi = RANK_CHUNK;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (precedes(k[mid], x[mid], ki, (int32_t)i)) lo = mid + 1;
      else hi = mid;
    }
    if (lo) atomicAdd(rank + i, lo);
  }
}

__global__ __launch_bounds__(256) void rank_scatter_kernel(const int32_t* __restrict__ rank,
                                                           int64_t n, int32_t* __restrict__ perm) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) {
    const int32_t r = rank[i];
    if (r >= 0 && r < n) perm[r] = (int32_t)i;
  }
}

__global__ void iota_kernel(int32_t* __restrict__ perm, int64_t n) {
  const int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (k < n) perm[k] = (int32_t)k;
}

// A[a][b] (a >= b) = H_d[perm[n-1-a]][perm[n-1-b]], H = 2S (lower of S authoritative).
// 32 x 32 tiles of A through LDS: without reordering, entry (a, b) comes from
// S[n-1-b][n-1-a], so the tile is read along rows of S (lanes along a) and
// written along rows of A (lanes along b).
__global__ __launch_bounds__(256) void build_a_kernel(const float* __restrict__ S, int64_t n,
                                                      int64_t lds,
                                                      const int32_t* __restrict__ perm,
                                                      const double* __restrict__ diag,
                                                      const double* __restrict__ lam,
                                                      double* __restrict__ A,
                                                      int32_t* __restrict__ info) {
  __shared__ double tile[32][33];  // [b - b0][a - a0]
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  const int64_t a0 = (int64_t)blockIdx.y * 32, b0 = (int64_t)blockIdx.x * 32;
  if (b0 > a0) return;  // the whole tile lies above the diagonal
  const double l = *lam;
  for (int r = ty; r < 32; r += 8) {
    const int64_t a = a0 + tx, b = b0 + r;
    double v = 0.0;
    if (a < n && b <= a) {
      // perm comes from this library's own order kernels, but an index
      // outside 0 .. n-1 must never address S
      const int64_t p = min<int64_t>(max<int64_t>(perm[n - 1 - a], 0), n - 1);
      const int64_t q = min<int64_t>(max<int64_t>(perm[n - 1 - b], 0), n - 1);
      if (a == b) {
        v = diag[p] + l;
      } else {
        const float sv = p > q ? S[p * lds + q] : S[q * lds + p];
        if (!isfinite(sv)) *info = -1;
        v = 2.0 * (double)sv;
      }
    }
    tile[r][tx] = v;
  }
  __syncthreads();
  for (int r = ty; r < 32; r += 8) {
    const int64_t a = a0 + r, b = b0 + tx;
    if (a < n && b <= a) A[a * n + b] = tile[tx][r];
  }
}

// With desc_act, entry (a, b) of a tile of A comes from a scattered row and
// column of S, so build_a_kernel reads 4 useful bytes of every line it
// fetches (~44 GB for a 28672-wide S).  Two coalesced passes instead, through
// the X workspace (free until the factorization): sym_kernel writes the whole
// symmetric S in fp32 (Sf[i][j] = S[max][min]), then gather_a_kernel builds
// each row a of A from row perm[n-1-a] of Sf staged in LDS, the columns read
// in the order perm[n-1-b] from there.
//
// sym_kernel: one workgroup per lower 64 x 64 tile (the grid enumerates the
// lower triangle of tiles only).  The tile comes in by 16-byte loads (VEC:
// lds and n multiples of 4, S 16-byte aligned; else element by element) and
// is staged in LDS; it leaves as itself in its own place and, off the
// diagonal, transposed in the mirrored place, both by 16-byte stores.  On a
// diagonal tile the entries above the diagonal are mirrored from below (S's
// upper triangle is never read).
constexpr int SYM_T = 64;

template <bool VEC>
__global__ __launch_bounds__(256) void sym_kernel(const float* __restrict__ S, int64_t n,
                                                  int64_t lds, float* __restrict__ Sf) {
  __shared__ float tile[SYM_T][SYM_T + 1];
  const int64_t L = blockIdx.x;
  int64_t ti = (int64_t)((sqrt(8.0 * (double)L + 1.0) - 1.0) * 0.5);
  while (ti * (ti + 1) / 2 > L) --ti;
  while ((ti + 1) * (ti + 2) / 2 <= L) ++ti;
  const int64_t tj = L - ti * (ti + 1) / 2;
  const int64_t i0 = ti * SYM_T, j0 = tj * SYM_T;
  const int c4 = threadIdx.x & 15, rr = threadIdx.x >> 4;  // float4 column, row in 16
  float4 v[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int64_t i = i0 + rr + 16 * k, j = j0 + 4 * c4;
    const float* src = S + i * lds + j;
    if (VEC && i < n && j + 3 <= i && j + 4 <= n) {
      v[k] = *reinterpret_cast<const float4*>(src);
    } else {
      float t[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) t[e] = (i < n && j + e <= i) ? src[e] : 0.0f;
      v[k] = make_float4(t[0], t[1], t[2], t[3]);
    }
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    float* d = &tile[rr + 16 * k][4 * c4];
    d[0] = v[k].x; d[1] = v[k].y; d[2] = v[k].z; d[3] = v[k].w;
  }
  __syncthreads();
  auto put4 = [&](int64_t row, int64_t col, const float (&t)[4]) {
    if (row >= n) return;
    float* dst = Sf + row * n + col;
    if (VEC && col + 4 <= n) {
      *reinterpret_cast<float4*>(dst) = make_float4(t[0], t[1], t[2], t[3]);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (col + e < n) dst[e] = t[e];
    }
  };
  const bool diag = ti == tj;
#pragma unroll
  for (int k = 0; k < 4; ++k) {  // the tile itself (mirrored above a diagonal)
    const int r = rr + 16 * k;
    float t[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int c = 4 * c4 + e;
      t[e] = (diag && c > r) ? tile[c][r] : tile[r][c];
    }
    put4(i0 + r, j0 + 4 * c4, t);
  }
  if (diag) return;
#pragma unroll
  for (int k = 0; k < 4; ++k) {  // its transpose: Sf[j][i] = S[i][j]
    const int r = rr + 16 * k;    // row j0 + r of Sf, columns i0 + 4 c4 ..
    float t[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) t[e] = tile[4 * c4 + e][r];
    put4(j0 + r, i0 + 4 * c4, t);
  }
}

constexpr int GATHER_NCAP = 32768;  // columns of a row staged in LDS (128 KB)
constexpr int GATHER_T = 1024;      // threads of gather_a_kernel
constexpr int GATHER_PER = GATHER_NCAP / GATHER_T / 2;  // packed position words a thread

// Thread t writes columns b = t + GATHER_T j of every row; their sources
// perm[n-1-b] (16-bit, two to a word) stay in registers for all the
// workgroup's rows, so perm is read once per workgroup.
__global__ __launch_bounds__(GATHER_T) void gather_a_kernel(const float* __restrict__ Sf,
                                                            int64_t n,
                                                            const int32_t* __restrict__ perm,
                                                            const double* __restrict__ diag,
                                                            const double* __restrict__ lam,
                                                            int64_t rows_per_wg,
                                                            double* __restrict__ A,
                                                            int32_t* __restrict__ info) {
  __shared__ __align__(16) float row[GATHER_NCAP];
  const int tid = threadIdx.x;
  const double l = *lam;
  const int64_t a0 = (int64_t)blockIdx.x * rows_per_wg;
  const int64_t a1 = min(n, a0 + rows_per_wg);
  if (a0 >= a1) return;
  uint32_t pq[GATHER_PER];
#pragma unroll
  for (int j = 0; j < GATHER_PER; ++j) {
    uint32_t h[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int64_t b = tid + (int64_t)GATHER_T * (2 * j + e);
      h[e] = b < n ? (uint32_t)min<int64_t>(max<int64_t>(perm[n - 1 - b], 0), n - 1) : 0u;
    }
    pq[j] = h[0] | (h[1] << 16);
  }
  bool bad = false;
  for (int64_t a = a0; a < a1; ++a) {
    const int64_t p = min<int64_t>(max<int64_t>(perm[n - 1 - a], 0), n - 1);
    const float* src = Sf + p * n;
    __syncthreads();  // the previous row has been read by every thread
    if (n % 4 == 0) {
      for (int64_t c = tid; c < n / 4; c += GATHER_T)
        reinterpret_cast<float4*>(row)[c] = reinterpret_cast<const float4*>(src)[c];
    } else {
      for (int64_t c = tid; c < n; c += GATHER_T) row[c] = src[c];
    }
    __syncthreads();
    double* dst = A + a * n;
#pragma unroll
    for (int j = 0; j < GATHER_PER; ++j) {
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int64_t b = tid + (int64_t)GATHER_T * (2 * j + e);
        if (b < a) {
          const float sv = row[(pq[j] >> (16 * e)) & 0xFFFFu];
          bad |= !isfinite(sv);
          dst[b] = 2.0 * (double)sv;
        } else if (b == a) {
          dst[b] = diag[p] + l;
        }
      }
    }
  }
  if (bad) *info = -1;
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
// (At most 8 k-steps: every operand read is issued before the first MFMA.)
template <bool QT>
__device__ __forceinline__ f64x4 tile16(const double* P, const double* Qm, int i0, int j0,
                                        int kmin, int kmax) {
  const int lane = threadIdx.x & 63;
  f64x4 acc = {0.0, 0.0, 0.0, 0.0};
  double av[8], bv[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const int k0 = kmin + 4 * t;
    if (k0 < kmax) {  // uniform in the wave
      const int kl = k0 + (lane >> 4);
      av[t] = P[(i0 + (lane & 15)) * PS + kl];
      bv[t] = QT ? Qm[(j0 + (lane & 15)) * PS + kl] : Qm[kl * PS + j0 + (lane & 15)];
    }
  }
#pragma unroll
  for (int t = 0; t < 8; ++t)
    if (kmin + 4 * t < kmax) acc = __builtin_amdgcn_mfma_f64_16x16x4f64(av[t], bv[t], acc, 0, 0, 0);
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
    // the diagonal block of X, its upper part as zeros: the products read
    // triangular operands by whole tiles of 32 or 64 inside these blocks
    for (int e = tid; e < NB * NB; e += 256) {
      const int i = e / NB, j = e % NB;
      if (i < sh && j < sh) X[(oh + i) * n + oh + j] = j <= i ? B1[i][j] : 0.0;
      if (half == 0 && i < s1 && j < s2) X[(off + i) * n + o2 + j] = 0.0;
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
  int64_t tiles;  // workgroup b takes tiles b, b + gridDim.x, ...
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
  for (int64_t bid = blockIdx.x; bid < g.tiles; bid += gridDim.x) {
  int64_t ti, tj;
  gemm_tile_of(g, bid, ti, tj);
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
}

template <int TILE>
void launch_gemm_tile(const GemmArgs& g0, bool ta, bool tb, int64_t max_wg, hipStream_t stream) {
  GemmArgs g = g0;
  const int64_t tm = ceil_div(g.M, TILE), tn = ceil_div(g.N, TILE);
  g.tiles_m = tm;
  g.tiles_n = tn;
  const int64_t tiles = g.lower ? tm * (tm + 1) / 2 : tm * tn;
  if (tiles == 0) return;
  g.tiles = tiles;
  const dim3 grid((unsigned)(max_wg > 0 ? hmin(tiles, max_wg) : tiles));
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
  for (int64_t bid = blockIdx.x; bid < g.tiles; bid += gridDim.x) {
  int64_t ti, tj;
  gemm_tile_of(g, bid, ti, tj);
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
  if (wv == 0) {
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
  __syncthreads();  // red is refilled by the next tile
  }
}

template <int TILE>
void launch_splitk(const GemmArgs& g0, bool tb, int64_t max_wg, hipStream_t stream) {
  GemmArgs g = g0;
  const int64_t tm = ceil_div(g.M, TILE), tn = ceil_div(g.N, TILE);
  g.tiles_m = tm;
  g.tiles_n = tn;
  const int64_t tiles = g.lower ? tm * (tm + 1) / 2 : tm * tn;
  if (tiles == 0) return;
  g.tiles = tiles;
  const dim3 grid((unsigned)(max_wg > 0 ? hmin(tiles, max_wg) : tiles));
  if (tb) hipLaunchKernelGGL((gemm_splitk_kernel<TILE, true>), grid, dim3(256), 0, stream, g);
  else hipLaunchKernelGGL((gemm_splitk_kernel<TILE, false>), grid, dim3(256), 0, stream, g);
}

// Large products (the trailing updates and the inverse's block-row products
// at large n): 128 x 128 output tiles, NW waves (8: waves of 64 x 32, four
// per SIMD at two workgroups per CU; 4: waves of 64 x 64), each a grid of
// v_mfma_f64_16x16x4_f64 accumulators.  K goes through LDS in stages of 16,
// double-buffered: a stage is fetched into registers (16-byte loads) while
// the previous one is multiplied, then stored k-major (As[k][i], Bs[k][j]),
// one barrier per stage.  The LDS row stride of 144 doubles puts two
// consecutive k rows on opposite halves of the 64 banks, so the 16 x 4
// operand reads of a half-wave are conflict-free; k rows 4-7 and 12-15 of a
// stage hold their columns XOR 16 (the other half of the banks), so the
// transposing stores of the row loads, whose lanes write k rows 0, 4, 8, 12
// at once, meet at most two to a bank, and the k-row loads of op(B) store
// 16-byte pairs 2 KPT columns apart so 32 lanes cover all 64 banks.
// (Measured before the swizzle: 4-6 bank-conflict cycles per LDS
// instruction, MFMA pipes 0.57-0.68 busy.)  op(A) is A itself
// (row-major, A[i * lda + k]); op(B) as in gemm_f64_kernel.  Needs even
// leading dimensions and 16-byte aligned A, B (checked by the caller).
// (Measured, 20480-wide products: 8 waves 49 TF/s against 41 for 4 on the
// K = 512 trailing update, 41 against 35 on the inverse's head product; an
// LDS-DMA variant with four stages in flight at one workgroup per CU was
// slower than both.)
constexpr int BIG = 128;   // tile edge
constexpr int BKC = 16;    // K per stage
constexpr int BLD = 144;   // LDS row stride (doubles)

// Tile of workgroup `bid` for the 128 x 128 products, XCD-aware (workgroup b
// runs on XCD b % 8, and the ~64 in flight on one XCD share its 4 MB L2):
//  - lower (the trailing updates, one K for every tile): the triangle in bands
//    of 8 tile rows, a band column by column, each XCD a contiguous range of
//    that order, so an XCD's tiles in flight read ~8 row blocks and ~8 column
//    blocks of the panel;
//  - K from the column's start (the inverse's head products: long, unequal K):
//    the tiles_m row tiles of a column on one XCD, columns in increasing order
//    (longest K first), so those tiles read the column's op(B) panel together;
//  - otherwise as gemm_tile_of.
// (Measured in isolation, bit-identical: +4 % on a K = 512 trailing update,
// +3-5 % on the head product.)
__device__ __forceinline__ void big_tile_of(const GemmArgs& g, int64_t bid, int64_t& ti,
                                            int64_t& tj) {
  if (g.lower) {
    const int64_t T = g.tiles_m, U = g.tiles, U8 = (U / 8) * 8;
    const int64_t u = bid < U8 ? (bid % 8) * (U8 / 8) + bid / 8 : bid;
    // band b (tile rows 8b .. 8b + 7) starts at 32 b^2 + 4 b: 64 tiles for
    // each earlier band of 8 rows, plus the bands' 36-tile diagonal triangles
    int64_t b = (int64_t)((-4.0 + sqrt(16.0 + 128.0 * (double)u)) / 64.0);
    while (b > 0 && 32 * b * b + 4 * b > u) --b;
    while (32 * (b + 1) * (b + 1) + 4 * (b + 1) <= u) ++b;
    const int64_t r0 = 8 * b, h = min((int64_t)8, T - r0);
    int64_t d = u - (32 * b * b + 4 * b);
    if (d < r0 * h) {  // the band's full columns 0 .. r0 - 1
      tj = d / h;
      ti = r0 + d % h;
      return;
    }
    d -= r0 * h;  // its diagonal triangle: column r0 + c has h - c tiles
    int64_t c = 0;
    while (d >= h - c) {
      d -= h - c;
      ++c;
    }
    tj = r0 + c;
    ti = r0 + c + d;
    return;
  }
  if (g.kmode & KLO_J) {
    const int64_t tm = g.tiles_m, tn = g.tiles_n;
    const int64_t full = (tn / 8) * 8 * tm;
    if (bid < full) {
      const int64_t s = bid / 8;
      ti = s % tm;
      tj = 8 * (s / tm) + bid % 8;
    } else {
      const int64_t u = bid - full;
      ti = u % tm;
      tj = (tn / 8) * 8 + u / tm;
    }
    return;
  }
  gemm_tile_of(g, bid, ti, tj);
}

template <bool TB, int NW>
__global__ __launch_bounds__(64 * NW, NW / 2) void gemm_f64_big_kernel(GemmArgs g) {
  // NW = 4: waves of 64 x 64 (2 x 2); NW = 8: waves of 64 x 32 (2 x 4)
  constexpr int NT = 64 * NW;           // threads
  constexpr int WCOL = 128 / (NW / 2);  // columns per wave
  constexpr int NB = WCOL / 16;         // MFMA tiles per wave row
  constexpr int PER = BIG * BKC / NT;   // doubles per thread per operand per stage
  constexpr int RPT = BKC / PER;        // threads per row in the row loads
  constexpr int KPT = BIG / PER;        // threads per k-row in the k-row loads
  __shared__ __align__(16) double As[2][BKC][BLD];
  __shared__ __align__(16) double Bs[2][BKC][BLD];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int wr = wv / (NW / 2), wc = wv % (NW / 2);
  // loader roles: "row" loads (PER consecutive k of one row i / column j) and
  // "k-row" loads (PER consecutive i / j of one k)
  const int rl_i = tid / RPT, rl_k = (tid % RPT) * PER;  // row loads
  const int kl_k = tid / KPT, kl_i = (tid % KPT) * 2;    // k-row loads: pairs kl_i + 2 KPT p
  // column swizzle of k row k (see above)
  auto sw = [](int k) { return ((k >> 2) & 1) << 4; };
  for (int64_t bid = blockIdx.x; bid < g.tiles; bid += gridDim.x) {
    int64_t ti, tj;
    big_tile_of(g, bid, ti, tj);
    const int64_t i0 = ti * BIG, j0 = tj * BIG;
    int64_t kb = 0, ke = g.K;
    if (g.kmode & KLO_J) kb = j0;
    if (g.kmode & KHI_J) ke = min(ke, j0 + BIG);
    if (g.kmode & KHI_I) ke = min(ke, i0 + BIG);
    f64x4 acc[4][NB];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < NB; ++b) acc[a][b] = f64x4{0.0, 0.0, 0.0, 0.0};
    double ra[PER], rb[PER];
    // op(A) row i0 + rl_i, k = k0 + rl_k .. + PER - 1
    const int64_t ai = i0 + rl_i;
    const bool a_ok = ai < g.M;
    const double* arow = g.A + (a_ok ? ai : 0) * g.lda;
    // op(B): TB -> row j0 + rl_i of B, k = k0 + rl_k ..; else k-row k0 + kl_k, j = j0 + kl_i ..
    const int64_t bj = j0 + (TB ? rl_i : kl_i);
    const bool b_ok = TB ? bj < g.N : true;
    const double* brow = TB ? g.B + (b_ok ? bj : 0) * g.ldb : g.B;
    // whole stages of a tile inside op(A) and op(B) take unchecked 16-byte
    // loads (k0 and rl_k even, lda and ldb even); the others, per element
    const bool full_tile = i0 + BIG <= g.M && j0 + BIG <= g.N;
    auto fetch = [&](int64_t k0) {
      if (full_tile && k0 + BKC <= ke) {  // uniform over the workgroup
#pragma unroll
        for (int p = 0; p < PER / 2; ++p) {
          const double2 v = *reinterpret_cast<const double2*>(arow + k0 + rl_k + 2 * p);
          ra[2 * p] = v.x;
          ra[2 * p + 1] = v.y;
        }
        if (TB) {
#pragma unroll
          for (int p = 0; p < PER / 2; ++p) {
            const double2 v = *reinterpret_cast<const double2*>(brow + k0 + rl_k + 2 * p);
            rb[2 * p] = v.x;
            rb[2 * p + 1] = v.y;
          }
        } else {
          const double* src = g.B + (k0 + kl_k) * g.ldb + bj;
#pragma unroll
          for (int p = 0; p < PER / 2; ++p) {
            const double2 v = *reinterpret_cast<const double2*>(src + 2 * KPT * p);
            rb[2 * p] = v.x;
            rb[2 * p + 1] = v.y;
          }
        }
        return;
      }
#pragma unroll
      for (int e = 0; e < PER; ++e) {
        const int64_t k = k0 + rl_k + e;
        ra[e] = (a_ok && k < ke) ? arow[k] : 0.0;
      }
      if (TB) {
#pragma unroll
        for (int e = 0; e < PER; ++e) {
          const int64_t k = k0 + rl_k + e;
          rb[e] = (b_ok && k < ke) ? brow[k] : 0.0;
        }
      } else {
        const int64_t k = k0 + kl_k;
        const bool kin = k < ke;
        const double* src = g.B + (kin ? k : kb) * g.ldb;
#pragma unroll
        for (int e = 0; e < PER; ++e) {
          const int64_t j = bj + 2 * KPT * (e / 2) + (e % 2);
          rb[e] = (kin && j < g.N) ? src[j] : 0.0;
        }
      }
    };
    auto stash = [&](int buf) {
#pragma unroll
      for (int e = 0; e < PER; ++e) As[buf][rl_k + e][rl_i ^ sw(rl_k + e)] = ra[e];
      if (TB) {
#pragma unroll
        for (int e = 0; e < PER; ++e) Bs[buf][rl_k + e][rl_i ^ sw(rl_k + e)] = rb[e];
      } else {
#pragma unroll
        for (int p = 0; p < PER / 2; ++p)
          *reinterpret_cast<double2*>(&Bs[buf][kl_k][(kl_i + 2 * KPT * p) ^ sw(kl_k)]) =
              make_double2(rb[2 * p], rb[2 * p + 1]);
      }
    };
    __syncthreads();  // the previous tile's last stage has been read by every wave
    if (kb < ke) fetch(kb);
    int buf = 0;
    for (int64_t k0 = kb; k0 < ke; k0 += BKC, buf ^= 1) {
      stash(buf);
      __syncthreads();
      if (k0 + BKC < ke) fetch(k0 + BKC);
#pragma unroll
      for (int ks = 0; ks < BKC; ks += 4) {
        double af[4], bf[NB];
        const int x = sw(ks);  // the same for the k-step's four rows
#pragma unroll
        for (int a = 0; a < 4; ++a)
          af[a] = As[buf][ks + (lane >> 4)][(64 * wr + 16 * a + (lane & 15)) ^ x];
#pragma unroll
        for (int b = 0; b < NB; ++b)
          bf[b] = Bs[buf][ks + (lane >> 4)][(WCOL * wc + 16 * b + (lane & 15)) ^ x];
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
          for (int b = 0; b < NB; ++b)
            acc[a][b] = __builtin_amdgcn_mfma_f64_16x16x4f64(af[a], bf[b], acc[a][b], 0, 0, 0);
      }
    }
    // D layout of the f64 16x16x4 MFMA: lane l, element q -> row l/16 + 4q, column l%16
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int64_t gi = i0 + 64 * wr + 16 * a + (lane >> 4) + 4 * q;
          const int64_t gj = j0 + WCOL * wc + 16 * b + (lane & 15);
          if (gi >= g.M || gj >= g.N) continue;
          if (g.lower && gj > gi) continue;
          double* c = g.C + gi * g.ldc + gj;
          const double v = g.alpha * acc[a][b][q];
          *c = g.beta == 0.0 ? v : fma(g.beta, *c, v);
        }
  }
}

// Products with at least this many 128 x 128 tiles take gemm_f64_big_kernel.
constexpr int64_t BIG_MIN_TILES = 256;

// The two products on the factorization's critical path, the panel
// L_k = A_k X_kk^T and the next column's update A[:, k+1] -= L_k L_{k+1,k}^T,
// are M x 128 x 128 (M up to n - 128): C[M, 128] = alpha A[M, 128] op(B) + beta
// C with op(B)(k, j) = B[j * ldb + k].  A workgroup takes TR rows and all 128
// columns: its A rows are staged in LDS (row stride 132 doubles: the 16 rows x
// 4 k of an operand read land on distinct bank pairs); 8 waves, wave w takes
// columns 32 (w % 4) .. + 31 over half of K (w / 4), keeps that part of op(B)
// in registers (32 doubles a lane, every load in flight at once) and runs its
// 16 k-steps back to back; the upper half's sums are added through LDS in a
// fixed order.  Triangular operands are read whole (their zero parts are
// stored zeros).  beta == 0 never reads C.
constexpr int TALL_LDA = 132;

template <int TR>
__global__ __launch_bounds__(512) void gemm_tall128_kernel(const double* __restrict__ A,
                                                           int64_t lda,
                                                           const double* __restrict__ B,
                                                           int64_t ldb, double* C, int64_t ldc,
                                                           int64_t M, double alpha, double beta) {
  constexpr int TA = TR / 16;
  __shared__ double As[TR][TALL_LDA];
  __shared__ double red[4][TA * 2 * 4][64];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int wc = wv & 3, kh = wv >> 2;
  const int r = lane & 15, kq = lane >> 4;
  const int64_t i0 = (int64_t)blockIdx.x * TR;
  // this wave's part of op(B): bf[b][s] = op(B)(64 kh + 4 s + kq, 32 wc + 16 b + r)
  double bf[2][16];
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const double* src = B + (int64_t)(32 * wc + 16 * b + r) * ldb + 64 * kh + kq;
#pragma unroll
    for (int st = 0; st < 16; ++st) bf[b][st] = src[4 * st];
  }
  // the workgroup's rows of A (rows past M as zeros): thread t covers row
  // t / 8 (+ 64 q), k 16 (t % 8) .. + 15
  {
    const int rr = tid >> 3;
    if (rr < TR) {
      const int kk = 16 * (tid & 7);
      const int64_t gi = i0 + rr;
      const double* src = A + (gi < M ? gi : 0) * lda + kk;
      double2 v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = *reinterpret_cast<const double2*>(src + 2 * e);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        As[rr][kk + 2 * e] = gi < M ? v[e].x : 0.0;
        As[rr][kk + 2 * e + 1] = gi < M ? v[e].y : 0.0;
      }
    }
  }
  __syncthreads();
  f64x4 acc[TA][2];
#pragma unroll
  for (int a = 0; a < TA; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = f64x4{0.0, 0.0, 0.0, 0.0};
#pragma unroll
  for (int st = 0; st < 16; ++st) {
    double af[TA];
#pragma unroll
    for (int a = 0; a < TA; ++a) af[a] = As[16 * a + r][64 * kh + 4 * st + kq];
#pragma unroll
    for (int a = 0; a < TA; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b)
        acc[a][b] = __builtin_amdgcn_mfma_f64_16x16x4f64(af[a], bf[b][st], acc[a][b], 0, 0, 0);
  }
  if (kh == 1) {
#pragma unroll
    for (int a = 0; a < TA; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int q = 0; q < 4; ++q) red[wc][(a * 2 + b) * 4 + q][lane] = acc[a][b][q];
  }
  __syncthreads();
  if (kh == 1) return;
#pragma unroll
  for (int a = 0; a < TA; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t i = i0 + 16 * a + kq + 4 * q;
        const int64_t j = 32 * wc + 16 * b + r;
        if (i < M) {
          double v = alpha * (acc[a][b][q] + red[wc][(a * 2 + b) * 4 + q][lane]);
          if (beta != 0.0) v = fma(beta, C[i * ldc + j], v);
          C[i * ldc + j] = v;
        }
      }
}

// C[M, 128] = alpha A[M, 128] B^T-indexed (op(B)(k, j) = B[j * ldb + k]) + beta C;
// A's rows 16-byte aligned (lda even, A 16-byte aligned).
void gemm_tall128(const double* A, int64_t lda, const double* B, int64_t ldb, double* C,
                  int64_t ldc, int64_t M, double alpha, double beta, hipStream_t stream) {
  if (M <= 0) return;
  if (ceil_div(M, 32) >= 256)
    hipLaunchKernelGGL(gemm_tall128_kernel<32>, dim3((unsigned)ceil_div(M, 32)), dim3(512), 0,
                       stream, A, lda, B, ldb, C, ldc, M, alpha, beta);
  else
    hipLaunchKernelGGL(gemm_tall128_kernel<16>, dim3((unsigned)ceil_div(M, 16)), dim3(512), 0,
                       stream, A, lda, B, ldb, C, ldc, M, alpha, beta);
}

hipError_t gemm(const double* A, int64_t lda, bool ta, const double* B, int64_t ldb, bool tb,
                double* C, int64_t ldc, int64_t M, int64_t N, int64_t K, double alpha, double beta,
                int kmode, bool lower, hipStream_t stream, int64_t max_wg = 0) {
  if (M <= 0 || N <= 0) return hipSuccess;
  GemmArgs g;
  g.A = A; g.lda = lda; g.B = B; g.ldb = ldb; g.C = C; g.ldc = ldc;
  g.M = M; g.N = N; g.K = K; g.alpha = alpha; g.beta = beta; g.kmode = kmode;
  g.lower = lower ? 1 : 0;
  g.tiles_m = g.tiles_n = g.tiles = 0;
  // Fewer than 256 tiles of 64 x 64 (too few to fill the chip, or a long K
  // over a narrow output) the split-K kernel on 32 x 32 tiles; otherwise
  // 64-wide tiles staged through LDS, dispatched longest K range first.
  // (Measured on products of 128 to 2048; 128-wide tiles lost at every size.)
  const int64_t t64 = lower ? ceil_div(M, 64) * (ceil_div(M, 64) + 1) / 2
                            : ceil_div(M, 64) * ceil_div(N, 64);
  const int64_t tm = ceil_div(M, BIG), tn = ceil_div(N, BIG);
  const int64_t t128 = lower ? tm * (tm + 1) / 2 : tm * tn;
  const bool big_ok = !ta && lda % 2 == 0 && ldb % 2 == 0 &&
                      reinterpret_cast<uintptr_t>(A) % 16 == 0 &&
                      reinterpret_cast<uintptr_t>(B) % 16 == 0;
  if (big_ok && t128 >= BIG_MIN_TILES) {
    g.tiles_m = tm;
    g.tiles_n = tn;
    g.tiles = t128;
    const dim3 grid((unsigned)(max_wg > 0 ? hmin(t128, max_wg) : t128));
    if (tb) hipLaunchKernelGGL((gemm_f64_big_kernel<true, 8>), grid, dim3(512), 0, stream, g);
    else hipLaunchKernelGGL((gemm_f64_big_kernel<false, 8>), grid, dim3(512), 0, stream, g);
  } else if (!ta && t64 < 256) {
    launch_splitk<32>(g, tb, max_wg, stream);
  } else {
    launch_gemm_tile<64>(g, ta, tb, max_wg, stream);
  }
  return hipGetLastError();
}

// X's blocks below the diagonal inside rows o .. o + s1 + s2: join the
// inverted neighbours [o, o + s1) and [o + s1, o + s1 + s2) through the
// panel L21 that sits where X21 goes.
hipError_t join(const PrepWs& w, int64_t n, int64_t o, int64_t s1, int64_t s2, double* Mj,
                hipStream_t st) {
  const int64_t o2 = o + s1;
  // M = L21 X11   (X11(c, j) = 0 for c < j)
  hipError_t e = gemm(w.X + o2 * n + o, n, false, w.X + o * n + o, n, false, Mj, s1, s2, s1, s1,
                      1.0, 0.0, KLO_J, false, st);
  // X21 = -X22 M  (X22(i, c) = 0 for c > i)
  if (e == hipSuccess)
    e = gemm(w.X + o2 * n + o2, n, false, Mj, s1, false, w.X + o2 * n + o, n, s2, s1, s2, -1.0,
             0.0, KHI_I, false, st);
  return e;
}

// X_gg for the group of blocks [b0, b0 + cnt): pairs of blocks, then pairs of those, ...
hipError_t invert_group_diag(const PrepWs& w, int64_t n, int64_t b0, int64_t cnt, double* Mj,
                             hipStream_t st) {
  hipError_t e = hipSuccess;
  for (int64_t wd = 1; wd < cnt && e == hipSuccess; wd *= 2) {
    for (int64_t a = 0; a + wd < cnt && e == hipSuccess; a += 2 * wd) {
      const int64_t o = NODE * (b0 + a), s1 = NODE * wd;
      const int64_t s2 = hmin(n, NODE * (b0 + hmin(a + 2 * wd, cnt))) - (o + s1);
      e = join(w, n, o, s1, s2, Mj, st);
    }
  }
  return e;
}

// Both phases: X's diagonal blocks from the nodes, L's panels into X's lower
// blocks, then X group by group over them.
//
// The factorization runs in outer blocks of `ob` 128-wide blocks.  Inside an
// outer block it is left-looking: before block k's node, its columns receive
// the updates of the outer block's earlier panels in one product (K = 128 j
// for the j-th block), then the node and the panel.  Past the outer block the
// updates go out with K = 128 ob: the next outer block's columns on the main
// stream (the lookahead, which the next nodes need) and everything beyond on
// the side stream, overlapping the next outer block; the main stream waits
// for the side stream's previous update before its lookahead (both write
// those columns).  With ob = 4 (large n) the trailing matrix is read and
// written once per 512 columns instead of once per 128, which is what bounds
// the rank-128 update in fp64; with ob = 1 (small n) the chain per 128
// columns is shortest.  The side products are released once the main stream
// has finished its lookahead and is about to start the next node.
hipError_t factor_invert(const PrepWs& w, int64_t n, int32_t* info, hipStream_t stream,
                         SideStream* side) {
  const int64_t nb = ceil_div(n, NODE);
  // measured: 8192 x 8192 prepare 13.6 ms with 4, 15.2 ms with 1; 4096 x 4096 about the
  // same either way (the node chain bounds it)
  const int64_t ob = n >= 6144 ? 4 : 1;
  const int64_t GRP = grp_blocks(n);
  double* Mg = w.M;
  double* Mj = w.M + GRP * NODE * n;
  auto node = [&](int64_t k) {
    const int64_t o = NODE * k;
    hipLaunchKernelGGL(node_kernel, dim3(1), dim3(256), 0, stream, w.A, w.X, n, o,
                       (int)hmin(n - o, (int64_t)NODE), info);
    return hipGetLastError();
  };
  // the inverse stream's work for group g once its last node is done
  auto group_tail = [&](int64_t g) {
    const int64_t b0 = GRP * g, cnt = hmin((int64_t)GRP, nb - b0);
    const int64_t c = NODE * b0, sg = hmin(n, c + GRP * NODE) - c;
    hipError_t e = invert_group_diag(w, n, b0, cnt, Mj, side->inv);
    // X[g, 0:c] = -X_gg M_g   (X_gg(i, j) = 0 for j > i)
    if (e == hipSuccess && g > 0)
      e = gemm(w.X + c * n + c, n, false, Mg, c, false, w.X + c * n, n, sg, c, sg, -1.0, 0.0,
               KHI_I, false, side->inv);
    return e;
  };
  // M_g = L[g, 0:c] X[0:c, 0:c] (X(r, j) = 0 for r < j): needs the groups above
  // and the panels of L in the group's rows, all written once group g - 1's
  // last node and panel are
  auto group_head = [&](int64_t g) {
    const int64_t c = NODE * GRP * g, sg = hmin(n, c + GRP * NODE) - c;
    return gemm(w.X + c * n, n, false, w.X, n, false, Mg, c, sg, c, c, 1.0, 0.0, KLO_J, false,
                side->inv);
  };
  // the whole-K product needs 16-byte aligned rows for its staged loads
  const bool tall = n % 2 == 0;
  hipError_t e = hipSuccess;
  bool pending = false;  // a trailing update is queued on the side stream
  int64_t groups_done = 0;  // groups whose inverse is enqueued
  for (int64_t k0 = 0; k0 < nb && e == hipSuccess; k0 += ob) {
    const int64_t k1 = hmin(nb, k0 + ob);
    const int64_t c0 = NODE * k0;  // first column of the outer block
    for (int64_t k = k0; k < k1 && e == hipSuccess; ++k) {
      const int64_t rk = NODE * k, sk = hmin(n - rk, (int64_t)NODE);
      if (k > k0) {
        // A[rk.., k] -= L[rk.., k0..k) L[k, k0..k)^T: the outer block's earlier panels
        // (stored in X's blocks), the diagonal block's upper part included (never read)
        const double* Lr = w.X + rk * n + c0;
        const int64_t K = rk - c0;
        if (tall && K == NODE && sk == NODE && n - rk >= 1024) {
          gemm_tall128(Lr, n, Lr, n, w.A + rk * n + rk, n, n - rk, -1.0, 1.0, stream);
          e = hipGetLastError();
        } else {
          e = gemm(Lr, n, false, Lr, n, true, w.A + rk * n + rk, n, n - rk, sk, K, -1.0, 1.0, 0,
                   false, stream);
        }
      }
      if (e == hipSuccess) e = node(k);
      const int64_t r1 = rk + NODE;
      if (e == hipSuccess && r1 < n) {
        // L_ik = A_ik X_kk^T  (X_kk(j, c) = 0 for c > j, stored as zeros: whole-K exact)
        const int64_t rows = n - r1;
        double* Lk = w.X + r1 * n + rk;
        if (tall && rows >= 3072) {
          gemm_tall128(w.A + r1 * n + rk, n, w.X + rk * n + rk, n, Lk, n, rows, 1.0, 0.0, stream);
          e = hipGetLastError();
        } else {
          e = gemm(w.A + r1 * n + rk, n, false, w.X + rk * n + rk, n, true, Lk, n, rows, NODE,
                   NODE, 1.0, 0.0, KHI_J, false, stream);
        }
      }
    }
    if (e != hipSuccess) break;
    const int64_t R = NODE * k1;  // first column past the outer block
    if (R >= n) break;
    const int64_t R2 = hmin(n, NODE * hmin(nb, k1 + ob));  // end of the next outer block
    const double* Lo = w.X + R * n + c0;                   // L[R.., outer block]
    const int64_t K = R - c0;
    // lookahead: the next outer block's columns (also written by the previous
    // trailing update, which must be applied first)
    if (pending) e = hipStreamWaitEvent(stream, side->trailing_done, 0);
    if (e == hipSuccess) {
      if (tall && K == NODE && R2 - R == NODE && n - R >= 1024) {
        gemm_tall128(Lo, n, Lo, n, w.A + R * n + R, n, n - R, -1.0, 1.0, stream);
        e = hipGetLastError();
      } else {
        e = gemm(Lo, n, false, Lo, n, true, w.A + R * n + R, n, n - R, R2 - R, K, -1.0, 1.0, 0,
                 false, stream);
      }
    }
    // release the side streams as the next node starts
    if (e == hipSuccess) e = hipEventRecord(side->step_done, stream);
    // everything past the next outer block, off the critical path
    if (e == hipSuccess && R2 < n) {
      e = hipStreamWaitEvent(side->s, side->step_done, 0);
      const double* L2 = w.X + R2 * n + c0;
      if (e == hipSuccess)
        e = gemm(L2, n, false, L2, n, true, w.A + R2 * n + R2, n, n - R2, n - R2, K, -1.0, 1.0, 0,
                 true, side->s);
      if (e == hipSuccess) e = hipEventRecord(side->trailing_done, side->s);
      pending = true;
    }
    // groups whose blocks are all factored: their inverse, and the next group's head
    const int64_t gready = k1 / GRP;
    if (e == hipSuccess && gready > groups_done)
      e = hipStreamWaitEvent(side->inv, side->step_done, 0);
    for (; groups_done < gready && e == hipSuccess; ++groups_done) {
      e = group_tail(groups_done);
      if (e == hipSuccess) e = group_head(groups_done + 1);
    }
  }
  if (e == hipSuccess && pending) e = hipStreamWaitEvent(stream, side->trailing_done, 0);
  // the last group, closed by node nb - 1
  if (e == hipSuccess) e = hipEventRecord(side->last_node, stream);
  if (e == hipSuccess) e = hipStreamWaitEvent(side->inv, side->last_node, 0);
  for (; groups_done <= (nb - 1) / GRP && e == hipSuccess; ++groups_done) {
    e = group_tail(groups_done);
    if (e == hipSuccess && groups_done < (nb - 1) / GRP) e = group_head(groups_done + 1);
  }
  if (e == hipSuccess) e = hipEventRecord(side->inv_done, side->inv);
  if (e == hipSuccess) e = hipStreamWaitEvent(stream, side->inv_done, 0);
  return e;
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
  b += align_up((size_t)m_elems(n) * sizeof(double), 256);
  b += align_up((size_t)n * sizeof(double), 256);
  b += 256;
  b += 2 * align_up((size_t)n * sizeof(int32_t), 256);  // perm, rank
  b += align_up((size_t)rank_pad(n) * sizeof(double), 256);  // sorted chunk keys
  b += align_up((size_t)rank_pad(n) * sizeof(int32_t), 256);  // and their columns
  return b;
}

hipError_t launch_prepare(const float* S, int64_t n, int64_t lds, float perc_damp, int desc_act,
                          float* U, int64_t ldu, int32_t* perm, uint8_t* dead, float* lambda_out,
                          int32_t* info, void* ws, hipStream_t stream) {
  PrepWs w = carve(ws, n);
  int32_t* pm = perm ? perm : w.perm;
  hipLaunchKernelGGL(diag_damp_kernel, dim3(1), dim3(1024), 0, stream, S, n, lds, perc_damp,
                     w.diag, dead, w.lam, lambda_out, desc_act ? w.rank : nullptr, info);
  if (desc_act) {
    const unsigned nch = (unsigned)ceil_div(n, (int64_t)RANK_CHUNK);
    hipLaunchKernelGGL(chunk_sort_kernel, dim3(nch), dim3(512), 0, stream, w.diag, n, w.skey,
                       w.sidx);
    hipLaunchKernelGGL(rank_search_kernel, dim3((unsigned)ceil_div(n, (int64_t)1024), nch),
                       dim3(256), 0, stream, w.diag, n, w.skey, w.sidx, w.rank);
    hipLaunchKernelGGL(rank_scatter_kernel, dim3((unsigned)ceil_div(n, 256)), dim3(256), 0, stream,
                       w.rank, n, pm);
  } else {
    hipLaunchKernelGGL(iota_kernel, dim3((unsigned)ceil_div(n, 256)), dim3(256), 0, stream, pm, n);
  }
  if (desc_act && n <= GATHER_NCAP && n >= 1024) {
    // permuted: symmetric S into X's memory (fp32), then A row by row
    float* Sf = reinterpret_cast<float*>(w.X);
    const int64_t T = ceil_div(n, (int64_t)SYM_T);
    const dim3 grid((unsigned)(T * (T + 1) / 2));
    const bool vec = lds % 4 == 0 && n % 4 == 0 && (reinterpret_cast<uintptr_t>(S) & 15) == 0;
    if (vec)
      hipLaunchKernelGGL(sym_kernel<true>, grid, dim3(256), 0, stream, S, n, lds, Sf);
    else
      hipLaunchKernelGGL(sym_kernel<false>, grid, dim3(256), 0, stream, S, n, lds, Sf);
    const int64_t wgs = hmin(n, (int64_t)256);
    const int64_t rpw = ceil_div(n, wgs);
    hipLaunchKernelGGL(gather_a_kernel, dim3((unsigned)ceil_div(n, rpw)), dim3(GATHER_T), 0,
                       stream, Sf, n, pm, w.diag, w.lam, rpw, w.A, info);
  } else {
    const dim3 grid((unsigned)ceil_div(n, 32), (unsigned)ceil_div(n, 32));
    hipLaunchKernelGGL(build_a_kernel, grid, dim3(256), 0, stream, S, n, lds, pm, w.diag, w.lam,
                       w.A, info);
  }
  SideStream* side = nullptr;
  hipError_t e = side_stream(side);
  if (e != hipSuccess) return e;
  // the side streams and their events are shared by every call on the device:
  // two host threads enqueueing at once would interleave the event records
  std::lock_guard<std::mutex> lock(side->run);
  e = factor_invert(w, n, info, stream, side);
  if (e != hipSuccess) return e;
  {
    const dim3 grid((unsigned)ceil_div(n, 256), (unsigned)hmin(n, 2048));
    hipLaunchKernelGGL(write_u_kernel, grid, dim3(256), 0, stream, w.X, n, U, ldu);
  }
  return hipGetLastError();
}

}  // namespace gptq
