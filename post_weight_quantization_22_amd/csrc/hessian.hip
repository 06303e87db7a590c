// Layer Hessian accumulation S += X^T X on gfx950.
//
// "GPTQ deep dive" (hncyxsy.com news 243429) section 3.1 step 1: the layer
// Hessian is built from the layer's calibration inputs X as 2 X X^T (the
// factor 2 and the damping are applied by gptq_prepare).  X arrives
// token-major, X[tokens, n], so X X^T = sum over tokens of x_t x_t^T: a SYRK
// whose reduction axis is the token axis.
//
// bf16 path (the dense contraction, on MFMA v_mfma_f32_32x32x16_bf16):
// lower-triangle 256 x 256 output tiles, 64-token stages, bf16 x bf16
// products exact in fp32, fp32 accumulation.  The MFMA operands need the
// token axis in the per-lane k slots while X is contiguous along channels:
//  - interior kernel (n a multiple of 256, whole stages, aligned rows): the
//    stage goes global -> LDS by DMA in X's own layout (XOR-swizzled 16-byte
//    chunks) and the operands are read back with the transposing LDS read
//    ds_read_b64_tr_b16; 8 waves of 128 x 64, LDS double buffer with the
//    next stage's first operands read across the barrier.
//  - general kernel (any shape): each lane loads an 8-token x 8-channel
//    block into registers (bounds-checked), transposes it with v_perm and
//    stores channel rows of 144 bytes (9 x 16 B: conflict-free) to LDS;
//    4 waves of 128 x 128.
// Tiles are few when n is small, so the token axis is split P ways; each
// split writes its partial tile to the workspace and a reduction kernel adds
// the P partials to S in a fixed order (deterministic, no atomics).  With
// P == 1 the tile is added to S directly, by one launch per 65,536 tokens
// (shorter units keep an XCD's workgroups on the same token rows, so they
// share them through its L2).
//
// fp32 path (fp32 activations; small layers): 64 x 64 lower tiles on the fp32
// MFMA (v_mfma_f32_16x16x4_f32).
#include "kernels.hpp"

namespace gptq {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int HT = 256;        // output tile edge (channels)
constexpr int HK = 64;         // tokens per stage
constexpr int HROW = HK + 8;   // LDS row length in bf16: 144 B = 9 x 16 B (odd, conflict-free)
constexpr int HWT = HT / 2;    // per-wave tile edge (2 x 2 waves)
constexpr int HSUB = HWT / 32; // 32x32 MFMA sub-tiles per wave edge

__device__ __forceinline__ void tile_coords(int64_t L, int64_t& ti, int64_t& tj) {
  // lower-triangle tile L -> (ti >= tj), row-major over the triangle
  int64_t t = (int64_t)((sqrt(8.0 * (double)L + 1.0) - 1.0) * 0.5);
  while (t * (t + 1) / 2 > L) --t;
  while ((t + 1) * (t + 2) / 2 <= L) ++t;
  ti = t;
  tj = L - t * (t + 1) / 2;
}

// Order of the lower-triangle tiles for the interior kernel: by 4 x 4
// super-tiles (rows of super-tiles, then rows of tiles), so that consecutive
// tiles share few channel blocks; needs T % 4 == 0, else tiles go row by row.
__device__ __forceinline__ void tile_of_order(int64_t Lb, int64_t T, int64_t& ti, int64_t& tj) {
  if (T % 4 != 0) {
    tile_coords(Lb, ti, tj);
    return;
  }
  // super-row bi holds 16 bi + 10 tiles; 8 bi^2 + 2 bi tiles precede it
  int64_t bi = (int64_t)((sqrt(4.0 + 32.0 * (double)Lb) - 2.0) / 16.0);
  while (8 * bi * bi + 2 * bi > Lb) --bi;
  while (8 * (bi + 1) * (bi + 1) + 2 * (bi + 1) <= Lb) ++bi;
  const int64_t r = Lb - (8 * bi * bi + 2 * bi);
  int64_t bj, li, lj;
  if (r < 16 * bi) {
    bj = r / 16;
    li = (r % 16) / 4;
    lj = r % 4;
  } else {
    const int64_t d = r - 16 * bi;  // lower triangle of the diagonal super-tile
    bj = bi;
    li = d >= 6 ? 3 : d >= 3 ? 2 : d >= 1 ? 1 : 0;
    lj = d - li * (li + 1) / 2;
  }
  ti = 4 * bi + li;
  tj = 4 * bj + lj;
}

// Position of tile (ti, tj) in that order.
__device__ __forceinline__ int64_t order_of_tile(int64_t ti, int64_t tj, int64_t T) {
  if (T % 4 != 0) return ti * (ti + 1) / 2 + tj;
  const int64_t bi = ti / 4, bj = tj / 4, li = ti % 4, lj = tj % 4;
  const int64_t base = 8 * bi * bi + 2 * bi;
  return bj < bi ? base + 16 * bj + 4 * li + lj : base + 16 * bi + li * (li + 1) / 2 + lj;
}

// Order of the tiles for T % 16 == 0: first the regions of
// 16 x 16 tiles below the diagonal (rows of regions), each as 8 runs of 32
// tiles that are 4 x 8 blocks (12 channel blocks a run, 32 a region); then
// the diagonal regions, each in the 4 x 4 super-tile order.  With the units
// dealt as below, the 32 workgroups of an XCD run one such block (~12
// channel blocks of the stage instead of ~15 in the super-tile order) and,
// unsplit, the 8 XCDs one region at a time: a round's units read ~33 channel
// blocks instead of ~81 (the other XCDs' requests for them can be served
// beyond the L2 without HBM).
__device__ __forceinline__ void region_tile(int64_t Lb, int64_t T, int64_t& ti, int64_t& tj) {
  const int64_t Ts = T / 16, noff = Ts * (Ts - 1) / 2 * 256;
  if (Lb < noff) {
    int64_t a, b;
    tile_coords(Lb / 256, a, b);  // region (a + 1, b), b <= a
    const int64_t k = Lb % 256, c = k / 32, e = k % 32;
    ti = 16 * (a + 1) + 4 * (c / 2) + e / 8;
    tj = 16 * b + 8 * (c % 2) + e % 8;
  } else {
    const int64_t d = Lb - noff, R = d / 136;
    int64_t li, lj;
    tile_of_order(d % 136, 16, li, lj);
    ti = 16 * R + li;
    tj = 16 * R + lj;
  }
}

// Position of tile (ti, tj) in the region order (T % 16 == 0).
__device__ __forceinline__ int64_t order_of_region_tile(int64_t ti, int64_t tj, int64_t T) {
  const int64_t Ts = T / 16, noff = Ts * (Ts - 1) / 2 * 256;
  const int64_t SI = ti / 16, SJ = tj / 16, li = ti % 16, lj = tj % 16;
  if (SI > SJ) {
    const int64_t R = (SI - 1) * SI / 2 + SJ;  // region (a + 1, b) at a (a + 1) / 2 + b
    return 256 * R + 32 * ((li / 4) * 2 + lj / 8) + 8 * (li % 4) + lj % 8;
  }
  return noff + 136 * SI + order_of_tile(li, lj, 16);
}

// Work units of the interior kernel.  The first ntiles - T2 tiles (in the
// region order for T % 16 == 0, else the super-tile order) are split P ways over the tokens, the last T2 tiles 2P ways
// into half-length units, which run last: T2 is chosen so that the full
// units fill whole rounds of 256 workgroups and the half units the rest, so
// no CU idles through a last, partly filled round of full units.  Workgroup
// b runs on XCD b % 8.  Split plans (P > 1): each kind of unit is dealt so
// that XCD x takes a contiguous range of it: whole token splits per XCD when
// the split count is a multiple of 8, and so the ~32 workgroups in flight on
// one XCD read the same token rows of a few channel blocks and share them
// through its L2.  Unsplit (P == 1): round by round, XCD x takes the x-th run
// of 32 of the round's 256 consecutive units (the region order above).
// half: the unit is a half-length one; slot: its partial tile.
__device__ __forceinline__ void hess_unit(int64_t b, int64_t P, int64_t T, int64_t T2,
                                          int64_t& p, int64_t& ti, int64_t& tj, bool& half,
                                          int64_t& slot) {
  const int64_t ntiles = T * (T + 1) / 2;
  const int64_t n1 = ntiles - T2;
  const int64_t U1 = n1 * P;
  half = b >= U1;
  const int64_t bb = half ? b - U1 : b;
  const int64_t U = half ? T2 * 2 * P : U1;
  int64_t u;
  if (P == 1) {
    // unsplit: round g's 256 units (one a CU) are consecutive in the order,
    // XCD x takes the x-th run of 32 of them
    const int64_t U256 = (U / 256) * 256;
    u = bb < U256 ? (bb / 256) * 256 + (bb % 8) * 32 + (bb % 256) / 8 : bb;
  } else {
    const int64_t U8 = (U / 8) * 8;
    u = bb < U8 ? (bb % 8) * (U8 / 8) + bb / 8 : bb;
  }
  const int64_t nt = half ? T2 : n1;
  p = u / nt;
  const int64_t Lb = (half ? n1 : 0) + u % nt;
  if (T % 16 == 0) region_tile(Lb, T, ti, tj);
  else tile_of_order(Lb, T, ti, tj);
  slot = half ? P * ntiles + p * T2 + (Lb - n1) : p * ntiles + ti * (ti + 1) / 2 + tj;
}

// One lane's share of a stage for one operand: 8 tokens x 8 channels.
struct Block8 {
  uint4 r[8];  // r[e]: token 8o + e, channels c .. c + 7
};

__device__ __forceinline__ void load_block8(const uint16_t* __restrict__ X, int64_t ldx,
                                            int64_t t_end, int64_t n, int64_t t, int64_t c,
                                            bool vec_ok, Block8& b) {
  const bool full = vec_ok && c + 8 <= n && t + 8 <= t_end;
  if (full) {
    const uint16_t* p = X + t * ldx + c;
#pragma unroll
    for (int e = 0; e < 8; ++e) b.r[e] = *reinterpret_cast<const uint4*>(p + e * ldx);
    return;
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    uint32_t w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      uint32_t lo = 0, hi = 0;
      if (t + e < t_end) {
        if (c + 2 * q < n) lo = X[(t + e) * ldx + c + 2 * q];
        if (c + 2 * q + 1 < n) hi = X[(t + e) * ldx + c + 2 * q + 1];
      }
      w[q] = lo | (hi << 16);
    }
    b.r[e] = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

__device__ __forceinline__ uint32_t word_of(const uint4& v, int w) {
  return w == 0 ? v.x : (w == 1 ? v.y : (w == 2 ? v.z : v.w));
}

// Transpose the 8 x 8 bf16 block in registers (v_perm_b32) and store channel
// rows: T[(c0 + ch) * HROW + 8 * o .. + 8] = tokens 8o .. 8o + 7 of channel c0 + ch.
__device__ __forceinline__ void store_block8(uint16_t* __restrict__ T, int c0, int o,
                                             const Block8& b) {
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    uint32_t lo[4], hi[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const uint32_t even = word_of(b.r[2 * p], w);      // token 2p: channels 2w, 2w+1
      const uint32_t odd = word_of(b.r[2 * p + 1], w);   // token 2p+1
      lo[p] = __builtin_amdgcn_perm(odd, even, 0x05040100u);  // channel 2w, tokens 2p, 2p+1
      hi[p] = __builtin_amdgcn_perm(odd, even, 0x07060302u);  // channel 2w+1
    }
    *reinterpret_cast<uint4*>(T + (c0 + 2 * w) * HROW + 8 * o) = make_uint4(lo[0], lo[1], lo[2], lo[3]);
    *reinterpret_cast<uint4*>(T + (c0 + 2 * w + 1) * HROW + 8 * o) =
        make_uint4(hi[0], hi[1], hi[2], hi[3]);
  }
}

// grid.x = ntiles * P; block L = blockIdx.x / P, split p = blockIdx.x % P (with P a
// multiple of 8 the workgroups of one token split share an XCD and its L2).
__global__ __launch_bounds__(256) void syrk_bf16_kernel(const uint16_t* __restrict__ X,
                                                        int64_t ldx, int64_t tokens, int64_t n,
                                                        int64_t tok_per_split, int64_t P,
                                                        float* __restrict__ S, int64_t lds,
                                                        float* __restrict__ part,
                                                        int64_t ntiles) {
  __shared__ __align__(16) uint16_t smem[4 * HT * HROW];
  // buffer b: operand A at smem + 2b * HT * HROW, operand B right after it
  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const int wr = wv >> 1, wc = wv & 1;
  const int64_t L = blockIdx.x / P;
  const int64_t p = blockIdx.x % P;
  int64_t ti, tj;
  tile_coords(L, ti, tj);
  const int64_t i0 = ti * HT, j0 = tj * HT;
  const bool diag = ti == tj;
  const bool skip_wave = diag && wr < wc;  // strictly upper quarter of a diagonal tile
  const int64_t t_begin = p * tok_per_split;
  const int64_t t_end = min(tokens, t_begin + tok_per_split);
  const bool vec_ok = ((reinterpret_cast<uintptr_t>(X) & 15) == 0) && (ldx % 8 == 0);

  // loader mapping: token octet o (0..7), channel block cb (0..31)
  const int o = tid & 7, cb = tid >> 3;

  f32x16 acc[HSUB][HSUB];
#pragma unroll
  for (int a = 0; a < HSUB; ++a)
#pragma unroll
    for (int b = 0; b < HSUB; ++b)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[a][b][q] = 0.0f;

  // The next stage is fetched one operand at a time (32 registers in flight),
  // each behind half of the current stage's MFMAs, then transposed into the
  // other LDS buffer; one barrier per stage.
  Block8 rg;
  int buf = 0;
  if (t_begin < t_end) {
    load_block8(X, ldx, t_end, n, t_begin + 8 * o, i0 + 8 * cb, vec_ok, rg);
    store_block8(smem, 8 * cb, o, rg);
    if (!diag) {
      load_block8(X, ldx, t_end, n, t_begin + 8 * o, j0 + 8 * cb, vec_ok, rg);
      store_block8(smem + HT * HROW, 8 * cb, o, rg);
    }
  }
  __syncthreads();
  auto mfma_half = [&](const uint16_t* At, const uint16_t* Bt, int kk0) {
#pragma unroll
    for (int kk = kk0; kk < kk0 + HK / 32; ++kk) {
      bf16x8 af[HSUB], bfr[HSUB];
#pragma unroll
      for (int a = 0; a < HSUB; ++a) {
        const int row = HWT * wr + 32 * a + (lane & 31);
        af[a] = *reinterpret_cast<const bf16x8*>(At + row * HROW + 16 * kk + 8 * (lane >> 5));
      }
#pragma unroll
      for (int b = 0; b < HSUB; ++b) {
        const int col = HWT * wc + 32 * b + (lane & 31);
        bfr[b] = *reinterpret_cast<const bf16x8*>(Bt + col * HROW + 16 * kk + 8 * (lane >> 5));
      }
#pragma unroll
      for (int a = 0; a < HSUB; ++a)
#pragma unroll
        for (int b = 0; b < HSUB; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[a], bfr[b], acc[a][b], 0, 0, 0);
    }
  };
  for (int64_t t0 = t_begin; t0 < t_end; t0 += HK) {
    const bool more = t0 + HK < t_end;
    const uint16_t* At = smem + 2 * buf * HT * HROW;
    const uint16_t* Bt = diag ? At : At + HT * HROW;
    uint16_t* nxt = smem + 2 * (buf ^ 1) * HT * HROW;
    if (more) load_block8(X, ldx, t_end, n, t0 + HK + 8 * o, i0 + 8 * cb, vec_ok, rg);
    if (!skip_wave) mfma_half(At, Bt, 0);
    if (more) {
      store_block8(nxt, 8 * cb, o, rg);
      if (!diag) load_block8(X, ldx, t_end, n, t0 + HK + 8 * o, j0 + 8 * cb, vec_ok, rg);
    }
    if (!skip_wave) mfma_half(At, Bt, HK / 32);
    if (more && !diag) store_block8(nxt + HT * HROW, 8 * cb, o, rg);
    __syncthreads();
    buf ^= 1;
  }
  if (skip_wave) return;

  // D layout of the 32x32 MFMA: lane l, register q -> row 8*(q/4) + 4*(l/32) + q%4, col l%32
#pragma unroll
  for (int a = 0; a < HSUB; ++a)
#pragma unroll
    for (int b = 0; b < HSUB; ++b)
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int ii = HWT * wr + 32 * a + 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3);
        const int jj = HWT * wc + 32 * b + (lane & 31);
        if (part) {
          part[((p * ntiles + L) * HT + ii) * HT + jj] = acc[a][b][q];
        } else {
          const int64_t gi = i0 + ii, gj = j0 + jj;
          if (gi < n && gj <= gi) S[gi * lds + gj] += acc[a][b][q];
        }
      }
}

// Interior kernel: every tile full (n % 256 == 0), every split a whole number
// of 64-token stages, rows 16-byte aligned; no bounds checks.  256 x 256 lower
// tiles, 1024 threads = 16 waves (4 per SIMD), each a 64 x 64 block of 4 x 4
// v_mfma_f32_16x16x32_bf16 accumulators (k-step 32 tokens), so one wave's
// waits are covered by the MFMAs of the three others on its SIMD.  Each
// output element is accumulated by one wave in token order.  The kernel is
// power-bound (the shader clock, not the MFMA pipes' busy fraction, sets the
// rate): at 28672 channels, 16 x 16 x 32 MFMAs run 6-8 % faster than
// 32 x 32 x 16 ones over the same tile (half the accumulator traffic per
// flop), and 16 waves faster than 8 waves of 128 x 64, which read a third
// less from LDS but leave each SIMD one partner wave.
//
// Each 64-token stage of the two 256-channel operands goes from global memory
// straight into LDS with global_load_lds_dwordx4 (16 bytes per lane, lane l
// landing at base + 16 l), in X's own token-major layout: token row t takes
// 512 bytes and 16-byte chunk k of the row sits at position
// k ^ (4 (t % 4) + 2 ((t / 8) % 2)).  MFMA operands come back with
// ds_read_b64_tr_b16, which hands each 16-lane group a 4-token x 16-channel
// block transposed (lane i: channel i, 4 consecutive tokens), i.e. the bf16
// operand layout, so there is no register staging and no permute.  With the
// swizzle the two 16-lane groups of a half-wave (tokens t .. t + 3 and
// t + 8 .. t + 11, the same two chunks of each row) read 16 distinct chunk
// positions: all 64 banks.  Two LDS buffers: the DMA of stage s + 2 is issued
// as soon as stage s is in registers.  The one barrier per stage (publishing
// stage s + 1) sits before the MFMAs of the last 32 tokens of stage s, whose
// operands are already in registers; each operand register is refilled for
// the next k-step right after its last MFMA, so LDS reads run under the
// MFMAs.  Diagonal tiles do the same work as the others (both operands
// loaded, every wave busy): tiles that finish early would start their next
// unit early and pull the workgroups of an XCD out of step, so that they no
// longer share the same token rows in its L2 (measured: 8 % faster than
// skipping the waves above the diagonal).
constexpr int FT_I = 256, FT_J = 256;   // tile
constexpr int WI = 64, WJ = 64;         // per wave
constexpr int MA = WI / 16, MB = WJ / 16;  // 16 x 16 accumulators per wave
constexpr int HWAVES = (FT_I / WI) * (FT_J / WJ);
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
constexpr int DROW = FT_I * 2;    // bytes per token row of one operand stage
constexpr int DSTAGE = HK * DROW;  // 32 KB per operand per stage

__device__ __forceinline__ int64_t uniform64(int64_t v) {
  const uint64_t u = (uint64_t)v;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)u);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(u >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ bf16x8 tr_operand(const uint8_t* p0) {
  // two transposing reads: tokens +0..3 and +4..7 of this lane's channel
  const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4i16*)(p0));
  const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4i16*)(p0 + 4 * DROW));
  typedef short v8i16 __attribute__((ext_vector_type(8)));
  const v8i16 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}

__global__ __launch_bounds__(64 * HWAVES) void syrk_bf16_dma_kernel(const uint16_t* __restrict__ X,
                                                            int64_t ldx, int64_t tokens,
                                                            int64_t P, int64_t T2,
                                                            float* __restrict__ S, int64_t lds,
                                                            float* __restrict__ part,
                                                            int64_t ntiles_edge) {
  __shared__ __align__(16) uint8_t smem[4 * DSTAGE];  // [buffer][operand]
  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  constexpr int RPW = HK / HWAVES;  // token rows loaded per wave per operand
  static_assert(RPW % 4 == 0 && 8 % RPW == 0,
                "a wave's rows: whole groups of 4, inside one group of 8");
  const int wr = wv / (FT_J / WJ), wc = wv % (FT_J / WJ);
  int64_t p, ti, tj, slot;
  bool half;
  hess_unit(blockIdx.x, P, ntiles_edge, T2, p, ti, tj, half, slot);
  const int64_t tok_per_split = half ? tokens / (2 * P) : tokens / P;
  const int64_t i0 = ti * FT_I, j0 = tj * FT_J;
  const int nstage = (int)(tok_per_split / HK);

  // DMA: instruction q of wave wv fills token rows RPW wv + 2 q and + 1 (lane
  // / 32); the swizzle depends on the row only through (2 q + lane / 32) % 4
  // and bit 3 of RPW wv, so two per-lane offsets (q even / odd) serve all q,
  // with the rest of the address wave-uniform.
  const int b3 = ((RPW * wv) >> 3) & 1;
  uint32_t voff[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int t = 2 * q + (lane >> 5);
    const int k = (lane & 31) ^ (4 * (t & 3) + 2 * b3);
    voff[q] = (uint32_t)(2 * (t * ldx + 8 * k));
  }
  const int wvu = __builtin_amdgcn_readfirstlane(wv);
  // the tile offsets come out of the unit's float arithmetic, where the
  // compiler cannot see that they are wave-uniform; the DMA wants them in SGPRs
  const char* xa = reinterpret_cast<const char*>(
      X + uniform64((p * tok_per_split + RPW * wvu) * ldx + i0));
  const int64_t jmi2 = uniform64(2 * (j0 - i0));
  const int64_t step2 = 2 * HK * ldx;
  const uint32_t lbase = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(uintptr_t)(
      __attribute__((address_space(3))) void*)(smem + RPW * wv * DROW));
  auto issue = [&](int s) {
    const uint32_t la = lbase + (uint32_t)((s & 1) * 2 * DSTAGE);
    const char* base = xa + (int64_t)s * step2;
#pragma unroll
    for (int q = 0; q < RPW / 2; ++q)
      lds_dma16(base + (int64_t)(4 * (q & ~1)) * ldx, voff[q & 1], la + 1024 * q);
#pragma unroll
    for (int q = 0; q < RPW / 2; ++q)
      lds_dma16(base + (int64_t)(4 * (q & ~1)) * ldx + jmi2, voff[q & 1], la + DSTAGE + 1024 * q);
  };

  // transposing reads: lane (g = lane / 16, i = lane % 16) points at token
  // 8 g + i / 4 (+ 32 kk, + 4 for the second read), channels 4 (i % 4) .. + 3
  // of a 16-channel block; the swizzle term of those rows is 4 (i / 4) +
  // 2 (g % 2)
  const int g = lane >> 4, i = lane & 15, qq = i >> 2, pch = i & 3;
  const int lane_off = (8 * g + qq) * DROW + 8 * (pch & 1);
  const int swz = 4 * qq + 2 * (g & 1);
  int offA[MA], offB[MB];
#pragma unroll
  for (int a = 0; a < MA; ++a)
    offA[a] = lane_off + 16 * ((((WI * wr + 16 * a) >> 3) + (pch >> 1)) ^ swz);
#pragma unroll
  for (int b = 0; b < MB; ++b)
    offB[b] = DSTAGE + lane_off + 16 * ((((WJ * wc + 16 * b) >> 3) + (pch >> 1)) ^ swz);

  f32x4 acc[MA][MB];
#pragma unroll
  for (int a = 0; a < MA; ++a)
#pragma unroll
    for (int b = 0; b < MB; ++b) acc[a][b] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  struct Ops {
    bf16x8 a[MA], b[MB];
  };
  auto rd = [&](int s, int kk, int off) {
    return tr_operand(smem + (s & 1) * 2 * DSTAGE + off + 32 * kk * DROW);
  };
  // the MFMAs of one k-step; each operand register is refilled with k-step
  // kn of stage sn right after its last use
  auto step = [&](Ops& o, int sn, int kn) {
#pragma unroll
    for (int a = 0; a < MA; ++a)
#pragma unroll
      for (int b = 0; b < MB; ++b) {
        acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(o.a[a], o.b[b], acc[a][b], 0, 0, 0);
        if (b == MB - 1) o.a[a] = rd(sn, kn, offA[a]);
        if (a == MA - 1) o.b[b] = rd(sn, kn, offB[b]);
      }
  };

  // stages 0 and 1 in flight; wait for stage 0 (vmcnt counts this wave's
  // outstanding DMA instructions: RPW per stage)
  issue(0);
  if (nstage > 1) issue(1);
  if (nstage > 1) {
    __builtin_amdgcn_s_waitcnt(0x0F70 | RPW);
  } else {
    __builtin_amdgcn_s_waitcnt(0x0F70);
  }
  __syncthreads();
  static_assert(HK == 64, "the k-step schedule below covers 2 x 32 tokens");
  Ops o;
#pragma unroll
  for (int a = 0; a < MA; ++a) o.a[a] = rd(0, 0, offA[a]);
#pragma unroll
  for (int b = 0; b < MB; ++b) o.b[b] = rd(0, 0, offB[b]);
  for (int s = 0; s < nstage; ++s) {
    step(o, s, 1);
    // stage s is in registers once the refills above have landed (the
    // barrier waits for this wave's LDS reads); stage s + 1 is published once
    // every wave's DMA has
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
    if (s + 2 < nstage) issue(s + 2);
    // after the last stage these refills read the other buffer's stale (in
    // bounds) contents, which nothing uses
    step(o, s + 1, 0);
  }

  // accumulator (a, b): lane l holds rows 4 (l / 16) + q, column l % 16
#pragma unroll
  for (int a = 0; a < MA; ++a)
#pragma unroll
    for (int b = 0; b < MB; ++b)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int ii = WI * wr + 16 * a + 4 * (lane >> 4) + q;
        const int jj = WJ * wc + 16 * b + (lane & 15);
        if (part) {
          part[(slot * FT_I + ii) * FT_J + jj] = acc[a][b][q];
        } else if (jj + j0 <= ii + i0) {
          S[(i0 + ii) * lds + j0 + jj] += acc[a][b][q];
        }
      }
}

// S[lower] += sum over splits of the 256 x 256 partial tiles, splits in order.
// Each thread sums 4 consecutive entries of a tile row (16-byte loads, the
// loads of 8 splits in flight before their in-order adds).
__global__ __launch_bounds__(256) void reduce_full_partials_kernel(const float* __restrict__ part,
                                                                   int64_t P, int64_t T2,
                                                                   int64_t T,
                                                                   float* __restrict__ S,
                                                                   int64_t lds, int vec_s) {
  constexpr int CH = FT_I * FT_J / 1024;
  const int64_t ntiles = T * (T + 1) / 2;
  const int64_t L = blockIdx.x / CH;
  const int64_t chunk = blockIdx.x % CH;
  int64_t ti, tj;
  tile_coords(L, ti, tj);
  const int e = (int)chunk * 1024 + 4 * threadIdx.x;
  const int ii = e / FT_J, jj = e % FT_J;
  const int64_t gi = ti * FT_I + ii, gj = tj * FT_J + jj;
  if (gj > gi) return;  // the whole quad lies above the diagonal
  // this tile's partials: P full splits, or 2P half splits for the last T2 tiles
  const int64_t Lb = T % 16 == 0 ? order_of_region_tile(ti, tj, T) : order_of_tile(ti, tj, T);
  const int64_t n1 = ntiles - T2;
  const bool halves = Lb >= n1;
  const int64_t first = halves ? P * ntiles + (Lb - n1) : L;
  const int64_t nq = halves ? 2 * P : P;
  const float4* src = reinterpret_cast<const float4*>(part + first * FT_I * FT_J + e);
  // float4s from one split to the next
  const int64_t stride = (halves ? T2 : ntiles) * (FT_I * FT_J / 4);
  float4 s = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  for (int64_t q0 = 0; q0 < nq; q0 += 8) {
    float4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (q0 + u < nq) v[u] = src[(q0 + u) * stride];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (q0 + u < nq) {
        s.x += v[u].x;
        s.y += v[u].y;
        s.z += v[u].z;
        s.w += v[u].w;
      }
  }
  float* d = S + gi * lds + gj;
  if (vec_s && gj + 3 <= gi) {
    float4 o = *reinterpret_cast<float4*>(d);
    o.x += s.x;
    o.y += s.y;
    o.z += s.z;
    o.w += s.w;
    *reinterpret_cast<float4*>(d) = o;
  } else {
    const float sv[4] = {s.x, s.y, s.z, s.w};
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (gj + u <= gi) d[u] += sv[u];
  }
}

// S[lower] += sum over splits of the partial tiles, splits in order.
__global__ __launch_bounds__(256) void reduce_partials_kernel(const float* __restrict__ part,
                                                              int64_t P, int64_t ntiles,
                                                              int64_t n, float* __restrict__ S,
                                                              int64_t lds) {
  const int64_t L = blockIdx.x / (HT * HT / 1024);
  const int64_t chunk = blockIdx.x % (HT * HT / 1024);
  int64_t ti, tj;
  tile_coords(L, ti, tj);
  for (int r = 0; r < 4; ++r) {
    const int e = (int)chunk * 1024 + r * 256 + threadIdx.x;
    const int ii = e / HT, jj = e % HT;
    const int64_t gi = ti * HT + ii, gj = tj * HT + jj;
    if (gi >= n || gj > gi) continue;
    float s = 0.0f;
    for (int64_t q = 0; q < P; ++q) s += part[(q * ntiles + L) * HT * HT + e];
    S[gi * lds + gj] += s;
  }
}

// fp32 activations: SIMT SYRK, 64x64 lower tiles, 256 threads x 4x4 outputs.
// fp32 activations: S += X^T X on v_mfma_f32_16x16x4_f32.  64 x 64 lower
// tiles, one per workgroup of 4 waves (each 32 x 32: 2 x 2 MFMA tiles), 64
// tokens a stage staged in LDS in X's own token-major layout (row stride 80
// floats: the 4 k rows of an operand read fall on distinct banks), the next
// stage's loads in registers while this one is multiplied.  Any n, tokens,
// ldx (bounds-checked loads; zeros past the ends).  fp32 products and sums:
// each entry within (tokens + 8) 2^-24 sum_t |x_ti x_tj| of the exact sum.
constexpr int FT = 64, FK = 64, FLD = FT + 16;
typedef float f32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void syrk_f32_kernel(const float* __restrict__ X, int64_t ldx,
                                                       int64_t tokens, int64_t n,
                                                       float* __restrict__ S, int64_t lds) {
  __shared__ float As[FK][FLD];
  __shared__ float Bs[FK][FLD];
  int64_t ti, tj;
  tile_coords(blockIdx.x, ti, tj);
  const int64_t i0 = ti * FT, j0 = tj * FT;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int wi = wv >> 1, wj = wv & 1;
  constexpr int PER = FK * FT / 256;  // elements a thread stages per operand (16)
  float ra[PER], rb[PER];
  auto fetch = [&](int64_t t0) {
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const int idx = tid + 256 * e, kk = idx / FT, cc = idx % FT;
      const int64_t t = t0 + kk;
      ra[e] = (t < tokens && i0 + cc < n) ? X[t * ldx + i0 + cc] : 0.0f;
      rb[e] = (t < tokens && j0 + cc < n) ? X[t * ldx + j0 + cc] : 0.0f;
    }
  };
  f32x4 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  fetch(0);
  for (int64_t t0 = 0; t0 < tokens; t0 += FK) {
    __syncthreads();  // every wave has read the previous stage
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const int idx = tid + 256 * e, kk = idx / FT, cc = idx % FT;
      As[kk][cc] = ra[e];
      Bs[kk][cc] = rb[e];
    }
    __syncthreads();
    if (t0 + FK < tokens) fetch(t0 + FK);
#pragma unroll
    for (int ks = 0; ks < FK; ks += 4) {
      float af[2], bf[2];
#pragma unroll
      for (int a = 0; a < 2; ++a) af[a] = As[ks + (lane >> 4)][32 * wi + 16 * a + (lane & 15)];
#pragma unroll
      for (int b = 0; b < 2; ++b) bf[b] = Bs[ks + (lane >> 4)][32 * wj + 16 * b + (lane & 15)];
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x4f32(af[a], bf[b], acc[a][b], 0, 0, 0);
    }
  }
  // D layout: lane l, element q -> row 4 (l / 16) + q, column l % 16
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t gi = i0 + 32 * wi + 16 * a + 4 * (lane >> 4) + q;
        const int64_t gj = j0 + 32 * wj + 16 * b + (lane & 15);
        if (gi < n && gj <= gi) S[gi * lds + gj] += acc[a][b][q];
      }
}

struct HessPlan {
  int64_t ntiles, P, tok_per_split;
  size_t ws;
};

HessPlan plan_bf16(int64_t n, int64_t tokens) {
  HessPlan pl;
  const int64_t T = ceil_div(n, HT);
  pl.ntiles = T * (T + 1) / 2;
  // Few tiles: split the tokens 8 ways, one split per XCD, partials reduced after.
  int64_t P = (pl.ntiles < 256 && tokens >= 8 * 512) ? 8 : 1;
  pl.tok_per_split = ceil_div(ceil_div(tokens, P), HK) * HK;
  P = hmax(1, ceil_div(tokens, pl.tok_per_split));
  if (P > 1 && P < 8) P = 8;  // keep p -> XCD; trailing splits may be empty
  pl.P = P;
  pl.ws = P > 1 ? (size_t)P * pl.ntiles * HT * HT * sizeof(float) : 0;
  return pl;
}

// Interior tiling (256 x 256 tiles of the lower triangle).  P = 0: not usable
// for these sizes (n not a multiple of 256, or not whole 64-token stages).
//
// A unit streams its tile's tokens from its start to its end, and the ~32
// workgroups in flight on one XCD share their channel blocks through its L2
// only while they stay near the same token rows.  Over a long token axis they
// drift apart and the L2 stops serving them: with all 524,288 tokens of a
// 28672-wide layer in one launch (8192 stages a unit) the L2 serves about a
// third of the 3.4 TB the tiles request and the launch takes ~438 ms; as
// launches of 32K-96K tokens, each adding its tiles to S, it takes ~387 ms
// (the extra read and write of S, 3.3 GB a launch, is small beside that).
// Split plans (P > 1) already give a unit tokens / P tokens.
constexpr int64_t HCHUNK = 65536;  // tokens per launch of an unsplit plan
struct FullPlan {
  int64_t ntiles, P, T2;
  size_t ws;
};

FullPlan plan_full(int64_t n, int64_t tokens) {
  FullPlan fp{0, 0, 0, 0};
  if (n % FT_I != 0) return fp;
  const int64_t T = n / FT_I;
  fp.ntiles = T * (T + 1) / 2;
  // Token split, one split per XCD (P a multiple of 8).  With one workgroup
  // per CU the grid runs in rounds of 256 units of tokens / P tokens each;
  // more splits fill the rounds better but write and re-read more partial
  // tiles (256 KB each).  T2 tiles split 2P ways make the last round one of
  // half-length units.  Time model fitted to n = 4096 with 8 to 32 splits:
  // ~30 ns per token per round, ~0.055 us per partial tile (its reduction).
  int64_t P = 1, T2 = 0;
  if (fp.ntiles <= 2048 && tokens % (8 * HK) == 0 && tokens >= 8 * 512) {
    double best = 0.0;
    for (int64_t c = 8; c <= 32; c *= 2) {
      if (tokens % (c * HK) != 0) break;
      const double per_round = (double)(tokens / c) * 30e-9;
      for (int h = 0; h < 2; ++h) {
        int64_t t2 = 0;
        if (h == 1) {
          if (tokens % (2 * c * HK) != 0) continue;
          t2 = fp.ntiles % (256 / c);
          if (t2 == 0) continue;
        }
        const double rounds = (double)ceil_div((fp.ntiles - t2) * c, 256) +
                              0.5 * (double)ceil_div(t2 * 2 * c, 256);
        const double t = rounds * per_round + (double)(c * fp.ntiles + c * t2) * 0.055e-6;
        if (P == 1 || t < best) {
          P = c;
          T2 = t2;
          best = t;
        }
      }
    }
  }
  if (tokens % (P * HK) != 0) return fp;
  fp.P = P;
  fp.T2 = T2;
  fp.ws = P > 1 ? (size_t)(P * fp.ntiles + 2 * P * T2) * FT_I * FT_J * sizeof(float) : 0;
  return fp;
}

}  // namespace

size_t hessian_ws_bytes(int64_t n, int64_t tokens, int dt) {
  if (dt != GPTQ_BF16 || tokens <= 0 || n <= 0) return 0;
  const FullPlan fp = plan_full(n, tokens);
  const size_t g = plan_bf16(n, tokens).ws;
  return fp.P > 0 && fp.ws > g ? fp.ws : g;
}

hipError_t launch_hessian(float* S, int64_t n, int64_t lds, const void* X, int dt, int64_t tokens,
                          int64_t ldx, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (tokens <= 0 || n <= 0) return hipSuccess;
  if (dt == GPTQ_F32) {
    const int64_t T = ceil_div(n, FT);
    hipLaunchKernelGGL(syrk_f32_kernel, dim3((unsigned)(T * (T + 1) / 2)), dim3(256), 0, stream,
                       reinterpret_cast<const float*>(X), ldx, tokens, n, S, lds);
    return hipGetLastError();
  }
  const FullPlan fp = plan_full(n, tokens);
  const bool interior = fp.P > 0 && (reinterpret_cast<uintptr_t>(X) % 16 == 0) && ldx % 8 == 0;
  if (interior) {
    if (ws_bytes < fp.ws) return hipErrorInvalidValue;
    float* part = fp.P > 1 ? reinterpret_cast<float*>(ws) : nullptr;
    const int64_t units = (fp.ntiles - fp.T2) * fp.P + fp.T2 * 2 * fp.P;
    // Unsplit (many tiles): one launch per HCHUNK tokens, each adding to S.
    // The tokens are whole stages (P == 1 plans need tokens % HK == 0).
    const int64_t chunk = fp.P == 1 ? HCHUNK : tokens;
    for (int64_t t0 = 0; t0 < tokens; t0 += chunk) {
      hipLaunchKernelGGL(syrk_bf16_dma_kernel, dim3((unsigned)units), dim3(64 * HWAVES), 0, stream,
                         reinterpret_cast<const uint16_t*>(X) + t0 * ldx, ldx,
                         hmin(chunk, tokens - t0), fp.P, fp.T2, S, lds, part, n / FT_I);
    }
    if (fp.P > 1) {
      const int vec_s = (reinterpret_cast<uintptr_t>(S) % 16 == 0) && lds % 4 == 0;
      hipLaunchKernelGGL(reduce_full_partials_kernel,
                         dim3((unsigned)(fp.ntiles * (FT_I * FT_J / 1024))), dim3(256), 0, stream,
                         part, fp.P, fp.T2, n / FT_I, S, lds, vec_s);
    }
    return hipGetLastError();
  }
  const HessPlan pl = plan_bf16(n, tokens);
  if (ws_bytes < pl.ws) return hipErrorInvalidValue;
  float* part = pl.P > 1 ? reinterpret_cast<float*>(ws) : nullptr;
  hipLaunchKernelGGL(syrk_bf16_kernel, dim3((unsigned)(pl.ntiles * pl.P)), dim3(256), 0, stream,
                     reinterpret_cast<const uint16_t*>(X), ldx, tokens, n, pl.tok_per_split,
                     pl.P, S, lds, part, pl.ntiles);
  if (pl.P > 1) {
    hipLaunchKernelGGL(reduce_partials_kernel, dim3((unsigned)(pl.ntiles * (HT * HT / 1024))),
                       dim3(256), 0, stream, part, pl.P, pl.ntiles, n, S, lds);
  }
  return hipGetLastError();
}

}  // namespace gptq
