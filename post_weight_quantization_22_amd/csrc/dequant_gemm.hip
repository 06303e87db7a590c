// Dequantized-weight matrix product Y = X W_q^T (16-bit activations, b-bit weights).
//
// "Quantized deployment, 1.5 TB to 250 GB" (lmnt.cn news 123823), section 2.1:
// a stored code q becomes the real value (q - zero_point) * scale.  "LLM
// quantization principles: GPTQ, AWQ, GGUF" (0539edu.com news 6111416), section
// 5.2: low-bit weights are turned back into 16-bit values before the product,
// and doing both in one operator is what keeps the dequantization from eating
// the bandwidth the small weights save.  This is that fused operator:
//
//   Y[t, r] = sum_p Xp[t, p] * w[r, p],   w[r, p] = bf16(fma(q[r, p], s, -(z * s)))
//
// with p the processing position (the weights are packed in processing order,
// so the groups of a row are runs of G consecutive positions), s = scale[r, p/G],
// z = zero[r, p/G] and Xp[t, p] = X[t, perm[p]] (X itself when perm is null).
//
// Work split.  A workgroup owns a BM x BN tile of Y (BM tokens, BN weight rows)
// and walks the 64-position chunks of its K range:
//   - the X tile (BM x 64 bf16) is loaded with 16-byte vector loads;
//   - the weight tile (BN x 64) arrives as packed words (2b words per row and
//     chunk, so every chunk starts on a word) and each of 2 BN threads turns 32
//     codes into bf16 in registers: the dequantization runs once per weight and
//     workgroup and is shared by its BM tokens;
//   - both tiles go to LDS (double-buffered, one barrier per chunk) in rows of
//     128 B whose 16-byte segments are XOR-swizzled by the row, so the MFMA
//     operand reads (8 consecutive positions of 32 rows) are free of bank
//     conflicts;
//   - waves of WM x WN run v_mfma_f32_32x32x16_bf16 on the tiles: exact bf16
//     products, fp32 accumulation; the loads of chunk j + 1 are in flight while
//     chunk j is multiplied.
// Decode-sized batches (a handful of tokens) are bound by the packed weights'
// HBM traffic; there the K range is split so the grid covers every CU, and the
// splits' fp32 partial sums are added in split order by a second kernel
// (deterministic).  Tiles are dealt to XCDs in contiguous runs, so the
// workgroups of one XCD share a token block (prefill) in its L2.
#include <type_traits>

#include "kernels.hpp"

namespace gptq {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BK = 64;         // positions per chunk
constexpr int ROWB = BK * 2;   // bytes of one LDS tile row
constexpr int kXcds = 8;

// Segment s of row r lives at segment s ^ ((r >> 1) & 7).  A 16-byte read of 16
// lanes covers 16 consecutive rows at one logical segment; the LDS serves 256
// bytes (64 banks) per cycle, i.e. two 128-byte rows, so the 16 lanes must hit
// 16 different (row parity, segment) pairs, which this swizzle gives.
__device__ __forceinline__ int swz(int r) { return (r >> 1) & 7; }
__device__ __forceinline__ int seg_off(int r, int s) { return r * ROWB + ((s ^ swz(r)) << 4); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// two fp32 -> packed bf16 pair, round to nearest even (one v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t bf16x2_bits(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// byte K of x as fp32 (v_cvt_f32_ubyteK; written out because the compiler folds
// the byte extraction into a bit-field extract when it knows the masked bits)
template <int K>
__device__ __forceinline__ float ubyte_f32(uint32_t x) {
  float r;
  if constexpr (K == 0) {
    __asm__("v_cvt_f32_ubyte0 %0, %1" : "=v"(r) : "v"(x));
  } else if constexpr (K == 1) {
    __asm__("v_cvt_f32_ubyte1 %0, %1" : "=v"(r) : "v"(x));
  } else if constexpr (K == 2) {
    __asm__("v_cvt_f32_ubyte2 %0, %1" : "=v"(r) : "v"(x));
  } else {
    __asm__("v_cvt_f32_ubyte3 %0, %1" : "=v"(r) : "v"(x));
  }
  return r;
}

// Code i (0..31) of a 32-code run held in BITS words, as fp32.
template <int BITS>
__device__ __forceinline__ float code_f32(const uint32_t (&w)[BITS], int i) {
  constexpr uint32_t MASK = (1u << BITS) - 1u;
  if constexpr (BITS == 1 || BITS == 2 || BITS == 4 || BITS == 8) {
    // BITS divides 8: code i is field (i % PER) of byte (i / PER) of its word,
    // so masking a whole word leaves one code per byte (v_cvt_f32_ubyteN)
    constexpr int PER = 8 / BITS;
    constexpr int CPW = 32 / BITS;
    const uint32_t word = w[i / CPW];
    const int k = i % CPW;
    const uint32_t spread = (word >> ((k % PER) * BITS)) & (MASK * 0x01010101u);
    return (float)((spread >> (8 * (k / PER))) & 0xFFu);
  } else {
    const int bit = i * BITS, wi = bit >> 5, off = bit & 31;
    uint32_t q;
    if (off + BITS <= 32) {
      q = (w[wi] >> off) & MASK;
    } else {
      q = __builtin_amdgcn_alignbit(w[wi + 1], w[wi], off) & MASK;
    }
    return (float)q;
  }
}

// Codes 8 s .. 8 s + 7 of a 32-code run held in BITS words, as fp32.
template <int BITS>
__device__ __forceinline__ void decode8(const uint32_t (&w)[BITS], int s, float (&f)[8]) {
  if constexpr (BITS == 4) {
    const uint32_t lo = w[s] & 0x0F0F0F0Fu, hi = (w[s] >> 4) & 0x0F0F0F0Fu;
    f[0] = ubyte_f32<0>(lo); f[1] = ubyte_f32<0>(hi);
    f[2] = ubyte_f32<1>(lo); f[3] = ubyte_f32<1>(hi);
    f[4] = ubyte_f32<2>(lo); f[5] = ubyte_f32<2>(hi);
    f[6] = ubyte_f32<3>(lo); f[7] = ubyte_f32<3>(hi);
  } else if constexpr (BITS == 8) {
    f[0] = ubyte_f32<0>(w[2 * s]); f[1] = ubyte_f32<1>(w[2 * s]);
    f[2] = ubyte_f32<2>(w[2 * s]); f[3] = ubyte_f32<3>(w[2 * s]);
    f[4] = ubyte_f32<0>(w[2 * s + 1]); f[5] = ubyte_f32<1>(w[2 * s + 1]);
    f[6] = ubyte_f32<2>(w[2 * s + 1]); f[7] = ubyte_f32<3>(w[2 * s + 1]);
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = code_f32<BITS>(w, 8 * s + e);
  }
}

struct DqArgs {
  const uint16_t* X;  // [tokens, ldx] bf16, 16-byte aligned, ldx % 8 == 0
  int64_t ldx, tokens, n;
  const uint32_t* P;  // [m, ldp] packed codes in processing order
  int64_t ldp, nwr;   // nwr = ceil(n * bits / 32) words of a row
  const float* scales;
  const float* zeros;
  int64_t ngroups, G;  // G <= 0: one group per row
  int gshift;          // log2(G) when G is a power of two, else -1
  int gs_run;          // 1 when every 32-position run lies in one group
  int64_t m;
  void* Y;  // [tokens, ldy] fp32 or bf16
  int64_t ldy;
  int ybf16;
  float* part;  // [ks, tokens, m] fp32 partial sums when ks > 1
  int64_t ntb, nrb, ks, chunks_per_split, nchunks, ntiles;
};

template <int BITS, int BM, int BN, int WM, int WN>
__global__ __launch_bounds__((BM / WM) * (BN / WN) * 64) void dequant_gemm_kernel(DqArgs a) {
  constexpr int NWN = BN / WN;
  constexpr int NT = (BM / WM) * NWN * 64;
  constexpr int XSEG = BM * 8;               // 16-byte X segments per chunk
  constexpr int XPT = (XSEG + NT - 1) / NT;  // per thread
  constexpr int UNITS = 2 * BN;              // 32-code runs per chunk
  constexpr int UPT = (UNITS + NT - 1) / NT;
  constexpr int STAGE = (BM + BN) * ROWB;
  constexpr int FA = WM / 32, FB = WN / 32;
  __shared__ __align__(16) uint8_t smem[2 * STAGE];

  // contiguous runs of tiles per XCD (workgroup b runs on XCD b % 8)
  const int64_t b = blockIdx.x;
  const int64_t xcd = b % kXcds, idx = b / kXcds;
  const int64_t per = a.ntiles / kXcds, rem = a.ntiles % kXcds;
  if (idx >= per + (xcd < rem ? 1 : 0)) return;
  const int64_t L = xcd * per + (xcd < rem ? xcd : rem) + idx;
  const int64_t rb = L % a.nrb;
  const int64_t kspl = (L / a.nrb) % a.ks;
  const int64_t tb = L / (a.nrb * a.ks);
  const int64_t tok0 = tb * BM, row0 = rb * BN;
  const int64_t c_begin = kspl * a.chunks_per_split;
  const int64_t c_end = min(a.nchunks, c_begin + a.chunks_per_split);

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int wm = wv / NWN, wn = wv % NWN;

  // ---- per-thread source rows (64-bit pointers formed once) ----
  const uint16_t* xrow[XPT];
  bool xlive[XPT];
#pragma unroll
  for (int i = 0; i < XPT; ++i) {
    const int sid = tid + i * NT;
    const int64_t t = tok0 + (sid >> 3);
    xlive[i] = sid < XSEG && t < a.tokens;
    xrow[i] = a.X + (xlive[i] ? t : 0) * a.ldx + 8 * (sid & 7);
  }
  const uint32_t* crow[UPT];
  const float* srow[UPT];
  const float* zrow[UPT];
  bool clive[UPT];
#pragma unroll
  for (int u = 0; u < UPT; ++u) {
    const int uid = tid + u * NT;
    const int64_t r = row0 + (uid >> 1);
    clive[u] = uid < UNITS && r < a.m;
    const int64_t rr = clive[u] ? r : 0;
    crow[u] = a.P + rr * a.ldp + (uid & 1) * BITS;
    srow[u] = a.scales + rr * a.ngroups;
    zrow[u] = a.zeros + rr * a.ngroups;
  }
  const int n32 = (int)a.n, nwr = (int)a.nwr, ng1 = (int)a.ngroups - 1, G = (int)a.G;

  // ---- global -> registers ----
  uint4 xr[XPT];
  uint32_t cw[UPT][BITS];
  float us[UPT][4], unz[UPT][4];

  auto group_of = [&](int p) -> int {
    if (G <= 0) return 0;
    const int g = a.gshift >= 0 ? (p >> a.gshift) : p / G;
    return min(g, ng1);
  };

  auto load_chunk = [&](int c) {
    const int k0 = c * BK;
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
      const int sid = tid + i * NT;
      const int col = k0 + 8 * (sid & 7);
      uint4 v = make_uint4(0, 0, 0, 0);
      if (xlive[i] && col < n32) {
        v = *reinterpret_cast<const uint4*>(xrow[i] + k0);
        if (col + 8 > n32) {  // last, partial segment: zero the columns past n
          uint32_t* e = reinterpret_cast<uint32_t*>(&v);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            if (col + 2 * q >= n32) e[q] = 0u;
            else if (col + 2 * q + 1 >= n32) e[q] &= 0xFFFFu;
          }
        }
      }
      xr[i] = v;
    }
#pragma unroll
    for (int u = 0; u < UPT; ++u) {
      const int uid = tid + u * NT;
      const int h = uid & 1;
      const int wbase = c * (2 * BITS) + h * BITS;
      const uint32_t* src = crow[u] + c * (2 * BITS);
      if (clive[u] && wbase + BITS <= nwr) {
#pragma unroll
        for (int q = 0; q < BITS; ++q) cw[u][q] = src[q];
      } else {
#pragma unroll
        for (int q = 0; q < BITS; ++q) cw[u][q] = (clive[u] && wbase + q < nwr) ? src[q] : 0u;
      }
      const int p0 = k0 + 32 * h;
      if (a.gs_run) {
        const int g = group_of(p0);
        const float sc = clive[u] ? srow[u][g] : 0.0f;
        const float zz = clive[u] ? zrow[u][g] : 0.0f;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          us[u][s] = sc;
          unz[u][s] = zz;
        }
      } else {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const int g = group_of(p0 + 8 * s);
          us[u][s] = clive[u] ? srow[u][g] : 0.0f;
          unz[u][s] = clive[u] ? zrow[u][g] : 0.0f;
        }
      }
    }
  };

  // ---- registers -> LDS (dequantizing the weight runs) ----
  auto store_chunk = [&](int c, int buf) {
    uint8_t* xt = smem + buf * STAGE;
    uint8_t* wt = xt + BM * ROWB;
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
      const int sid = tid + i * NT;
      if (sid < XSEG) *reinterpret_cast<uint4*>(xt + seg_off(sid >> 3, sid & 7)) = xr[i];
    }
    const int k0 = c * BK;
#pragma unroll
    for (int u = 0; u < UPT; ++u) {
      const int uid = tid + u * NT;
      if (uid >= UNITS) continue;
      const int rr = uid >> 1, h = uid & 1;
      const int p0 = k0 + 32 * h;
      const bool tail = p0 + 32 > n32;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const float sc = us[u][s];
        const float nzs = -(unz[u][s] * sc);
        float f[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] = fmaf(code_f32<BITS>(cw[u], 8 * s + e), sc, nzs);
        if (tail) {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (p0 + 8 * s + e >= n32) f[e] = 0.0f;
        }
        uint4 o;
        o.x = bf16x2_bits(f[0], f[1]);
        o.y = bf16x2_bits(f[2], f[3]);
        o.z = bf16x2_bits(f[4], f[5]);
        o.w = bf16x2_bits(f[6], f[7]);
        *reinterpret_cast<uint4*>(wt + seg_off(rr, 4 * h + s)) = o;
      }
    }
  };

  f32x16 acc[FA][FB];
#pragma unroll
  for (int i = 0; i < FA; ++i)
#pragma unroll
    for (int j = 0; j < FB; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;

  // operand reads: lane -> row (lane & 31) of a 32-row block, logical segment
  // 2 kk + (lane >> 5), i.e. positions 16 kk + 8 (lane >> 5) .. + 8
  auto compute = [&](int buf) {
    const uint8_t* xt = smem + buf * STAGE;
    const uint8_t* wt = xt + BM * ROWB;
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      bf16x8 av[FA], bv[FB];
      const int sg = 2 * kk + (lane >> 5);
#pragma unroll
      for (int i = 0; i < FA; ++i)
        av[i] = *reinterpret_cast<const bf16x8*>(xt + seg_off(WM * wm + 32 * i + (lane & 31), sg));
#pragma unroll
      for (int j = 0; j < FB; ++j)
        bv[j] = *reinterpret_cast<const bf16x8*>(wt + seg_off(WN * wn + 32 * j + (lane & 31), sg));
#pragma unroll
      for (int i = 0; i < FA; ++i)
#pragma unroll
        for (int j = 0; j < FB; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[i], bv[j], acc[i][j], 0, 0, 0);
    }
  };

  if (c_begin < c_end) {
    load_chunk((int)c_begin);
    store_chunk((int)c_begin, 0);
    __syncthreads();
    for (int c = (int)c_begin; c < (int)c_end; ++c) {
      const int buf = (c - (int)c_begin) & 1;
      const bool more = c + 1 < c_end;
      if (more) load_chunk(c + 1);
      compute(buf);
      if (more) store_chunk(c + 1, buf ^ 1);
      __syncthreads();
    }
  }

  // ---- epilogue: lane holds weight row (lane & 31) of each 32-block and
  // tokens 8 (q / 4) + 4 (lane / 32) + q % 4 ----
  const int64_t tw = tok0 + WM * wm + 4 * (lane >> 5);
  const int64_t rw = row0 + WN * wn + (lane & 31);
  const bool full = tok0 + WM * (wm + 1) <= a.tokens && row0 + WN * (wn + 1) <= a.m;
  float* outf;
  int64_t ld;
  if (a.ks > 1) {
    outf = a.part + kspl * a.tokens * a.m;
    ld = a.m;
  } else {
    outf = reinterpret_cast<float*>(a.Y);
    ld = a.ldy;
  }
  __bf16* outh = reinterpret_cast<__bf16*>(a.Y);
  const bool half = a.ks == 1 && a.ybf16;
#pragma unroll
  for (int i = 0; i < FA; ++i)
#pragma unroll
    for (int j = 0; j < FB; ++j) {
      const int64_t base = (tw + 32 * i) * ld + rw + 32 * j;
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int dt = 8 * (q >> 2) + (q & 3);
        if (!full && (tw + 32 * i + dt >= a.tokens || rw + 32 * j >= a.m)) continue;
        const int64_t o = base + (int64_t)dt * ld;
        if (half) {
          outh[o] = (__bf16)acc[i][j][q];
        } else {
          outf[o] = acc[i][j][q];
        }
      }
    }
}

// ---------------------------------------------------------------------------
// Tiles of TM tokens x 128 weight rows (TM = 256, 128 or 32), 4 waves.
// Everything that comes from HBM arrives by LDS DMA (global_load_lds), so the
// only loads the compiler schedules are LDS reads, and each stage's arrival is
// awaited with one explicit vmcnt before the barrier that publishes it:
//   X tile    3 stages, issued 2 chunks ahead (TM x 128 bytes each);
//   codes     4 stages, issued 3 chunks ahead (128 rows x 2b words);
//   scale/zero 4 stages, with the codes (one group per row and chunk: G is a
//             multiple of 64 or a whole row);
//   W tile    2 buffers: chunk c + 1 is dequantized (codes -> bf16) by all
//             threads while chunk c is multiplied.
// Rows past the last token or weight row, and columns past n in the last chunk,
// are read from clamped (valid) addresses; their products are discarded (rows)
// or zeroed in LDS (columns).  Small batches (TM = 32) are bound by the codes'
// HBM traffic; the deep DMA pipeline keeps several chunks of every workgroup
// in flight.
constexpr int DN = 128;  // weight rows per tile
constexpr int DX_STAGES = 3, DC_STAGES = 4;
constexpr int DW_BYTES = DN * ROWB;  // 16 KB

template <int BITS, int TM>
struct DmaLayout {
  static constexpr int X_BYTES = TM * ROWB;
  static constexpr int C_BYTES = DN * 2 * BITS * 4;  // codes of one chunk
  static constexpr int Z_BYTES = DN * 2 * 4;         // scales then zeros
  static constexpr int X_OFF = 0;
  static constexpr int W_OFF = X_OFF + DX_STAGES * X_BYTES;
  static constexpr int C_OFF = W_OFF + 2 * DW_BYTES;
  static constexpr int Z_OFF = C_OFF + DC_STAGES * C_BYTES;
  static constexpr int TOTAL = Z_OFF + DC_STAGES * Z_BYTES;
  // 4 waves: TM >= 128 -> 2 x 2 waves of (TM / 2) x 64; TM = 32 -> 1 x 4 of 32 x 32
  static constexpr int NWM = TM >= 128 ? 2 : 1, NWN = 4 / NWM;
  static constexpr int WM = TM / NWM, WN = DN / NWN;
  static constexpr int X_PER_WAVE = X_BYTES / 1024 / 4;  // 1 KB X DMAs per wave and chunk
  static constexpr int ISSUE = X_PER_WAVE + BITS + 1;    // DMAs per wave and chunk
};

template <int BITS, int TM>
__global__ __launch_bounds__(256) void dequant_gemm_dma_kernel(DqArgs a) {
  using Lay = DmaLayout<BITS, TM>;
  static_assert(Lay::TOTAL <= 160 * 1024, "LDS");
  constexpr int DM = TM, DWM = Lay::WM, DWN = Lay::WN, NWN = Lay::NWN;
  constexpr int X_PER_WAVE = Lay::X_PER_WAVE;
  constexpr int DX_BYTES = Lay::X_BYTES;
  __shared__ __align__(16) uint8_t smem[Lay::TOTAL];

  const int64_t b = blockIdx.x;
  const int64_t xcd = b % kXcds, idx = b / kXcds;
  const int64_t per = a.ntiles / kXcds, rem = a.ntiles % kXcds;
  if (idx >= per + (xcd < rem ? 1 : 0)) return;
  const int64_t L = xcd * per + (xcd < rem ? xcd : rem) + idx;
  const int64_t rb = L % a.nrb;
  const int64_t kspl = (L / a.nrb) % a.ks;
  const int64_t tb = L / (a.nrb * a.ks);
  const int64_t tok0 = tb * DM, row0 = rb * DN;
  const int c_begin = (int)(kspl * a.chunks_per_split);
  const int c_end = (int)min(a.nchunks, (int64_t)c_begin + a.chunks_per_split);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wv / NWN, wn = wv % NWN;
  const int n32 = (int)a.n, nwr = (int)a.nwr;
  const int tmax = (int)(a.tokens - 1 - tok0);  // last valid row of the tile
  const int rmax = (int)(a.m - 1 - row0);

  // ---- DMA sources (per-lane 32-bit offsets fixed for the tile) ----
  // X: instruction j of wave wv fills rows 8 (wv X_PER_WAVE + j) .. + 8; lane l
  // lands on row + l / 8, physical segment l % 8, so it loads the logical
  // segment (l % 8) ^ swz(row)
  uint32_t xoff[X_PER_WAVE];
  int xseg[X_PER_WAVE];
#pragma unroll
  for (int j = 0; j < X_PER_WAVE; ++j) {
    const int row = 8 * (wv * X_PER_WAVE + j) + (lane >> 3);
    xseg[j] = (lane & 7) ^ swz(row);
    xoff[j] = (uint32_t)(2 * ((int64_t)min(row, tmax) * a.ldx + 8 * xseg[j]));
  }
  const char* xbase = reinterpret_cast<const char*>(a.X + tok0 * a.ldx);
  uint32_t crow_off[BITS];
  int cword[BITS];
#pragma unroll
  for (int q = 0; q < BITS; ++q) {
    const int d = q * 256 + tid;
    const int row = d / (2 * BITS);
    cword[q] = d % (2 * BITS);
    crow_off[q] = (uint32_t)(4 * ((int64_t)min(row, rmax) * a.ldp));
  }
  const char* cbase = reinterpret_cast<const char*>(a.P + row0 * a.ldp);
  const int zrow = min(tid & 127, rmax);  // waves 0, 1: scales; 2, 3: zeros
  const char* zbase = reinterpret_cast<const char*>((wv < 2 ? a.scales : a.zeros) +
                                                    row0 * a.ngroups);
  const uint32_t lds0 = lds_addr(smem);

  auto issue_x = [&](int c) {
    const int k0 = c * BK;
    const uint32_t dst = lds0 + Lay::X_OFF + (c % DX_STAGES) * DX_BYTES +
                         wv * X_PER_WAVE * 1024;
    const char* src = xbase + 2 * (int64_t)k0;
    if (k0 + BK <= n32) {
#pragma unroll
      for (int j = 0; j < X_PER_WAVE; ++j) lds_dma16(src, xoff[j], dst + 1024 * j);
    } else {  // last chunk: segments past n re-read the last valid one (zeroed later)
#pragma unroll
      for (int j = 0; j < X_PER_WAVE; ++j) {
        const int clamp = 2 * (min(8 * xseg[j], n32 - 8 - k0) - 8 * xseg[j]);
        lds_dma16(src, xoff[j] + (uint32_t)clamp, dst + 1024 * j);
      }
    }
  };
  auto issue_c = [&](int c) {
    const int st = c % DC_STAGES;
    const uint32_t dst = lds0 + Lay::C_OFF + st * Lay::C_BYTES + wv * 256;
    const int w0 = c * 2 * BITS;
#pragma unroll
    for (int q = 0; q < BITS; ++q) {
      const int word = min(w0 + cword[q], nwr - 1);
      lds_dma4(cbase, crow_off[q] + 4u * (uint32_t)word, dst + 1024 * q);
    }
    const int g = a.G > 0 ? min((c * BK) / (int)a.G, (int)a.ngroups - 1) : 0;
    lds_dma4(zbase, (uint32_t)(4 * ((int64_t)zrow * a.ngroups + g)),
             lds0 + Lay::Z_OFF + st * Lay::Z_BYTES + wv * 256);
  };

  // ---- dequantization: thread -> weight row tid / 2, codes 32 (tid & 1) ..
  // + 32 of the chunk, in 4 parts of 8 codes (one 16-byte LDS row segment each)
  // interleaved with the MFMAs of the chunk before ----
  const int drow = tid >> 1, dh = tid & 1;
  struct Dq {
    uint32_t w[BITS];
    float sc, nzs;
  };
  auto dq_load = [&](int c, Dq& d) {
    const int st = c % DC_STAGES;
    const uint32_t* cs = reinterpret_cast<const uint32_t*>(smem + Lay::C_OFF + st * Lay::C_BYTES);
    const float* zs = reinterpret_cast<const float*>(smem + Lay::Z_OFF + st * Lay::Z_BYTES);
#pragma unroll
    for (int q = 0; q < BITS; ++q) d.w[q] = cs[drow * 2 * BITS + dh * BITS + q];
    d.sc = zs[drow];
    d.nzs = -(zs[DN + drow] * d.sc);
  };
  auto dq_part = [&](int c, const Dq& d, int s) {
    float f[8];
    decode8<BITS>(d.w, s, f);
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = fmaf(f[e], d.sc, d.nzs);
    uint4 o;
    o.x = bf16x2_bits(f[0], f[1]);
    o.y = bf16x2_bits(f[2], f[3]);
    o.z = bf16x2_bits(f[4], f[5]);
    o.w = bf16x2_bits(f[6], f[7]);
    uint8_t* wt = smem + Lay::W_OFF + (c & 1) * DW_BYTES;
    *reinterpret_cast<uint4*>(wt + seg_off(drow, 4 * dh + s)) = o;
  };

  f32x16 acc[DWM / 32][DWN / 32];
#pragma unroll
  for (int i = 0; i < DWM / 32; ++i)
#pragma unroll
    for (int j = 0; j < DWN / 32; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;

  struct Ops {
    bf16x8 a[DWM / 32], b[DWN / 32];
  };
  auto read_ops = [&](const uint8_t* xt, const uint8_t* wt, int kk, Ops& o) {
    const int sg = 2 * kk + (lane >> 5);
#pragma unroll
    for (int i = 0; i < DWM / 32; ++i)
      o.a[i] = *reinterpret_cast<const bf16x8*>(xt + seg_off(DWM * wm + 32 * i + (lane & 31), sg));
#pragma unroll
    for (int j = 0; j < DWN / 32; ++j)
      o.b[j] = *reinterpret_cast<const bf16x8*>(wt + seg_off(DWN * wn + 32 * j + (lane & 31), sg));
  };
  // multiply chunk c (operands of step kk + 1 read while step kk multiplies);
  // with DQ, dequantize chunk c + 1 alongside, one part per step
  auto compute = [&](int c, auto dq_tag) {
    constexpr bool DQ = decltype(dq_tag)::value;
    const uint8_t* xt = smem + Lay::X_OFF + (c % DX_STAGES) * DX_BYTES;
    const uint8_t* wt = smem + Lay::W_OFF + (c & 1) * DW_BYTES;
    Dq d;
    if constexpr (DQ) dq_load(c + 1, d);
    Ops o[2];
    read_ops(xt, wt, 0, o[0]);
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      if (kk + 1 < BK / 16) read_ops(xt, wt, kk + 1, o[(kk + 1) & 1]);
#pragma unroll
      for (int i = 0; i < DWM / 32; ++i)
#pragma unroll
        for (int j = 0; j < DWN / 32; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(o[kk & 1].a[i], o[kk & 1].b[j],
                                                              acc[i][j], 0, 0, 0);
      if constexpr (DQ) dq_part(c + 1, d, kk);
    }
  };
  // columns past n of the last chunk (their X is a re-read of a valid segment)
  // are set to 0 in LDS, so whatever the weights there, the products are 0
  auto zero_x_tail = [&](int c) {
    uint8_t* xt = smem + Lay::X_OFF + (c % DX_STAGES) * DX_BYTES;
    const int k0 = c * BK;
    for (int i = tid; i < DM * 8; i += 256) {
      const int row = i >> 3, sg = i & 7;
      if (k0 + 8 * sg >= n32) *reinterpret_cast<uint4*>(xt + seg_off(row, sg)) = make_uint4(0, 0, 0, 0);
    }
  };
  const bool tail = c_end * BK > n32;  // this split ends with the partial last chunk

  if (c_begin < c_end) {
    // prologue: X of chunks 0, 1 and codes of chunks 0, 1, 2 in flight; chunk 0
    // dequantized once its codes have landed
    const int c0 = c_begin;
    issue_c(c0);
    issue_x(c0);
    if (c0 + 1 < c_end) { issue_c(c0 + 1); issue_x(c0 + 1); }
    if (c0 + 2 < c_end) issue_c(c0 + 2);
    __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
    __syncthreads();
    {
      Dq d;
      dq_load(c0, d);
#pragma unroll
      for (int s = 0; s < 4; ++s) dq_part(c0, d, s);
    }
    __builtin_amdgcn_s_waitcnt(0x0070);
    __syncthreads();
    int c = c0;
    for (; c + 1 < c_end; ++c) {
      // X of c + 2 and codes of c + 3; the wait at the end covers everything
      // issued one iteration ago (X of c + 1, codes of c + 2)
      if (c + 2 < c_end) issue_x(c + 2);
      if (c + 3 < c_end) issue_c(c + 3);
      compute(c, std::true_type{});
      if (c + 3 < c_end) {
        __builtin_amdgcn_s_waitcnt(0x0070 | (Lay::ISSUE & 15) | ((Lay::ISSUE >> 4) << 14));
      } else {
        __builtin_amdgcn_s_waitcnt(0x0070);
      }
      __syncthreads();
    }
    if (tail) {
      zero_x_tail(c);
      __builtin_amdgcn_s_waitcnt(0x0070);
      __syncthreads();
    }
    compute(c, std::false_type{});
  }

  // ---- epilogue ----
  const int64_t tw = tok0 + DWM * wm + 4 * (lane >> 5);
  const int64_t rw = row0 + DWN * wn + (lane & 31);
  const bool fulltile = tok0 + DWM * (wm + 1) <= a.tokens && row0 + DWN * (wn + 1) <= a.m;
  float* outf;
  int64_t ld;
  if (a.ks > 1) {
    outf = a.part + kspl * a.tokens * a.m;
    ld = a.m;
  } else {
    outf = reinterpret_cast<float*>(a.Y);
    ld = a.ldy;
  }
  __bf16* outh = reinterpret_cast<__bf16*>(a.Y);
  const bool half = a.ks == 1 && a.ybf16;
#pragma unroll
  for (int i = 0; i < DWM / 32; ++i)
#pragma unroll
    for (int j = 0; j < DWN / 32; ++j) {
      const int64_t base = (tw + 32 * i) * ld + rw + 32 * j;
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int dt = 8 * (q >> 2) + (q & 3);
        if (!fulltile && (tw + 32 * i + dt >= a.tokens || rw + 32 * j >= a.m)) continue;
        const int64_t o = base + (int64_t)dt * ld;
        if (half) {
          outh[o] = (__bf16)acc[i][j][q];
        } else {
          outf[o] = acc[i][j][q];
        }
      }
    }
}

// ---------------------------------------------------------------------------
// Dense bf16 product Y = X W^T (X [tokens, n], W [m, n], both bf16 with n
// contiguous).  256 x 256 tiles, 1024 threads = 16 waves (4 per SIMD), each a
// 64 x 64 block of 4 x 4 v_mfma_f32_16x16x32_bf16 accumulators.  Chunks of 64
// positions of both tiles arrive by LDS DMA (global_load_lds_dwordx4, each wave
// 16 rows of each) in 128-byte rows whose 16-byte segments are XOR-swizzled by
// the row (seg_off), two buffers, one explicit vmcnt and one barrier per chunk,
// the DMA of chunk c + 2 issued as soon as chunk c is in registers.  A lane
// (q = lane / 16, r = lane % 16) reads positions 8 q .. + 7 (k-step kk:
// segment 4 kk + q) of row r of a 16-row block, the operand layout of the
// 16 x 16 x 32 MFMA, conflict-free under the swizzle; each operand register is
// refilled for the next k-step right after its last MFMA, so the LDS reads run
// under the MFMAs.  The 16 x 16 x 32 instruction and 4 waves per SIMD against
// 4 waves of 128 x 128 on 32 x 32 x 16 (measured on the calibration-forward
// and prefill shapes: 0.95-1.06 -> 1.21-1.32 PFLOP/s, the same sums).  For the
// calibration forward of a quantized layer over many tokens the weights are
// dequantized once (gptq_dequantize) and multiplied here, so no tile
// re-dequantizes them.
struct DenseArgs {
  const uint16_t* X;
  int64_t ldx, tokens, n;
  const uint16_t* W;
  int64_t ldw, m;
  void* Y;
  int64_t ldy;
  int ybf16;
  int64_t nrb, ntiles, nchunks;
};

constexpr int DD_TM = 256, DD_TN = 256;
constexpr int64_t DD_GT = 4;  // token blocks per group of the tile order

__global__ __launch_bounds__(1024) void dense_gemm16_kernel(DenseArgs a) {
  constexpr int X_BYTES = DD_TM * ROWB, W_BYTES = DD_TN * ROWB;  // 32 KB each
  constexpr int STAGE = X_BYTES + W_BYTES;
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  __shared__ __align__(16) uint8_t smem[2 * STAGE];
  const int64_t b = blockIdx.x;
  const int64_t xcd = b % kXcds, idx = b / kXcds;
  const int64_t per = a.ntiles / kXcds, rem = a.ntiles % kXcds;
  if (idx >= per + (xcd < rem ? 1 : 0)) return;
  const int64_t L = xcd * per + (xcd < rem ? xcd : rem) + idx;
  // tiles in groups of DD_GT token blocks: consecutive L walk down a group's
  // token blocks, then its next row block, so the ~32 workgroups an XCD runs at
  // once cover ~4 token x 8 row blocks and share both operands in its L2
  // (rather than one token block and 32 row blocks: every weight tile fetched
  // again for each token block)
  const int64_t ntb = (a.tokens + DD_TM - 1) / DD_TM;
  const int64_t grp = L / (DD_GT * a.nrb), in = L - grp * DD_GT * a.nrb;
  const int64_t tb0 = grp * DD_GT, gsz = min((int64_t)DD_GT, ntb - tb0);
  const int64_t tb = tb0 + in % gsz, rb = in / gsz;
  const int64_t tok0 = tb * DD_TM, row0 = rb * DD_TN;
  const int nst = (int)a.nchunks;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wv >> 2, wn = wv & 3;
  const int n32 = (int)a.n;
  const int tmax = (int)(a.tokens - 1 - tok0);
  const int rmax = (int)(a.m - 1 - row0);

  // DMA: wave wv fills rows 16 wv .. 16 wv + 15 of both tiles, two
  // instructions each; lane l lands on row + l / 8, physical segment l % 8, so
  // it loads the logical segment (l % 8) ^ swz(row); rows past the end re-read
  // the last one, and in the last chunk segments past n re-read the last valid
  // one (finite values, multiplied by X's zeroed columns there)
  const char* xbase = reinterpret_cast<const char*>(a.X + tok0 * a.ldx);
  const char* wbase = reinterpret_cast<const char*>(a.W + row0 * a.ldw);
  const uint32_t lds0 = lds_addr(smem);
  auto src_off = [&](int row, int rmaxv, int64_t ld, int k0) -> uint32_t {
    const int seg = (lane & 7) ^ swz(row);
    int s8 = 8 * seg;
    if (k0 + BK > n32) s8 = min(s8, n32 - 8 - k0);
    return (uint32_t)(2 * ((int64_t)min(row, rmaxv) * ld + s8));
  };
  auto issue = [&](int c) {
    const int k0 = c * BK;
    const uint32_t xdst = lds0 + (c & 1) * STAGE + wv * 2048;
    const uint32_t wdst = xdst + X_BYTES;
    const char* xs = xbase + 2 * (int64_t)k0;
    const char* ws = wbase + 2 * (int64_t)k0;
#pragma unroll
    for (int j = 0; j < 2; ++j)
      lds_dma16(xs, src_off(16 * wv + 8 * j + (lane >> 3), tmax, a.ldx, k0), xdst + 1024 * j);
#pragma unroll
    for (int j = 0; j < 2; ++j)
      lds_dma16(ws, src_off(16 * wv + 8 * j + (lane >> 3), rmax, a.ldw, k0), wdst + 1024 * j);
  };
  // columns past n of the last chunk are set to 0 in X's tile
  auto zero_x_tail = [&](int c) {
    uint8_t* xt = smem + (c & 1) * STAGE;
    const int k0 = c * BK;
    for (int i = tid; i < DD_TM * 8; i += 1024) {
      const int row = i >> 3, sg = i & 7;
      if (k0 + 8 * sg >= n32) *reinterpret_cast<uint4*>(xt + seg_off(row, sg)) = make_uint4(0, 0, 0, 0);
    }
  };

  // a lane reads rows r + 16 i (+ 64 wm or 64 wn), whose swizzle is swz(r)
  const int q = lane >> 4, r16 = lane & 15;
  const int segoff0 = (q ^ swz(r16)) << 4, segoff1 = ((4 + q) ^ swz(r16)) << 4;
  int offA[4], offB[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    offA[i] = (64 * wm + 16 * i + r16) * ROWB;
    offB[i] = X_BYTES + (64 * wn + 16 * i + r16) * ROWB;
  }
  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  struct Ops {
    bf16x8 a[4], b[4];
  };
  auto rd = [&](int c, int kk, int off) {
    return *reinterpret_cast<const bf16x8*>(smem + (c & 1) * STAGE + off + (kk ? segoff1 : segoff0));
  };
  // the MFMAs of one k-step; each operand register is refilled with k-step kn
  // of chunk cn right after its last use
  auto step = [&](Ops& o, int cn, int kn) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(o.a[i], o.b[j], acc[i][j], 0, 0, 0);
        if (j == 3) o.a[i] = rd(cn, kn, offA[i]);
        if (i == 3) o.b[j] = rd(cn, kn, offB[j]);
      }
  };

  // chunks 0 and 1 in flight; wait for chunk 0 (vmcnt counts this wave's
  // outstanding DMA instructions: 4 per chunk)
  issue(0);
  if (nst > 1) issue(1);
  if (nst > 1) {
    __builtin_amdgcn_s_waitcnt(0x0F70 | 4);
  } else {
    __builtin_amdgcn_s_waitcnt(0x0F70);
  }
  __syncthreads();
  if (nst == 1 && BK > n32) {
    zero_x_tail(0);
    __syncthreads();
  }
  Ops o;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    o.a[i] = rd(0, 0, offA[i]);
    o.b[i] = rd(0, 0, offB[i]);
  }
  // steady chunks (the tail chunk, if any, is not among the next ones); the
  // barrier publishes chunk c + 1 after chunk c is in registers
  int c = 0;
  for (; c + 2 < nst; ++c) {
    step(o, c, 1);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
    issue(c + 2);
    step(o, c + 1, 0);
  }
  if (c + 1 < nst) {  // the last chunk arrives: its X past n to 0 before its reads
    step(o, c, 1);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
    if (nst * BK > n32) {
      zero_x_tail(c + 1);
      __syncthreads();
    }
    step(o, c + 1, 0);
    ++c;
  }
  // the last chunk's two k-steps; the refills past it read the other
  // buffer's stale (in bounds) contents, which nothing uses
  step(o, c, 1);
  step(o, c + 1, 0);

  // accumulator (i, j): lane l holds tokens 4 (l / 16) + e, weight row l % 16
  const bool fulltile = tok0 + 64 * (wm + 1) <= a.tokens && row0 + 64 * (wn + 1) <= a.m;
  float* outf = reinterpret_cast<float*>(a.Y);
  __bf16* outh = reinterpret_cast<__bf16*>(a.Y);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t t = tok0 + 64 * wm + 16 * i + 4 * q + e;
        const int64_t r = row0 + 64 * wn + 16 * j + r16;
        if (!fulltile && (t >= a.tokens || r >= a.m)) continue;
        const int64_t o2 = t * a.ldy + r;
        if (a.ybf16) {
          outh[o2] = (__bf16)acc[i][j][e];
        } else {
          outf[o2] = acc[i][j][e];
        }
      }
}

// W[r, p] = bf16(fma(q[r, p], s, -(z s))) from codes packed in processing order:
// the weights the products above form, written once.  A wave covers 256
// 8-position segments of a row: lane j, store s writes segment 256 x + 64 s + j
// (16 bytes), so every store instruction writes 1 KB of whole lines; the lane
// reads the BITS words of that segment's 32-code run (four lanes share a run:
// one coalesced load) and its group's scale and zero (a group holds whole
// segments; n a multiple of 8).  The row is blockIdx.y (strided past the
// grid), so no 64-bit division is needed.
template <int BITS>
__global__ __launch_bounds__(64) void dequantize_kernel(const uint32_t* __restrict__ P,
                                                        int64_t ldp, int64_t m, int64_t n,
                                                        const float* __restrict__ scales,
                                                        const float* __restrict__ zeros,
                                                        int64_t G, int64_t ngroups,
                                                        uint16_t* __restrict__ W, int64_t ldw) {
  const int nseg = (int)(n / 8);
  const int nwr = (int)((n * BITS + 31) / 32);
  const int g32 = (int)G;
  const int k0 = (int)blockIdx.x * 256 + (int)threadIdx.x;
  for (int64_t r = blockIdx.y; r < m; r += gridDim.y) {
    const uint32_t* prow = P + r * ldp;
    const float* srow = scales + r * ngroups;
    const float* zrow = zeros + r * ngroups;
    uint16_t* wrow = W + r * ldw;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int k = k0 + 64 * s;  // segment: positions 8 k .. 8 k + 7
      if (k < nseg) {
        const int run = k >> 2;
        uint32_t w[BITS];
#pragma unroll
        for (int q = 0; q < BITS; ++q) {
          const int wi = run * BITS + q;
          w[q] = wi < nwr ? prow[wi] : 0u;  // the last run's words past the row are not read
        }
        const int g = g32 > 0 ? (8 * k) / g32 : 0;
        const float sc = srow[g];
        const float nzs = -(zrow[g] * sc);
        float f[8];
        decode8<BITS>(w, k & 3, f);
        uint4 o;
        o.x = bf16x2_bits(fmaf(f[0], sc, nzs), fmaf(f[1], sc, nzs));
        o.y = bf16x2_bits(fmaf(f[2], sc, nzs), fmaf(f[3], sc, nzs));
        o.z = bf16x2_bits(fmaf(f[4], sc, nzs), fmaf(f[5], sc, nzs));
        o.w = bf16x2_bits(fmaf(f[6], sc, nzs), fmaf(f[7], sc, nzs));
        *reinterpret_cast<uint4*>(wrow + 8 * k) = o;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Decode batches of at most 16 tokens, n a multiple of 128, every 32-position
// run in one group: one workgroup per 16 weight rows over the whole K range, so
// no second kernel adds split partial sums and no partials go through HBM.
// The eight waves take an eighth of the 128-position chunks each (at n = 4096
// four chunks, whose loads are all in flight at once).  Per chunk a
// lane (weight row l % 16 and token l % 16, run g = l / 16) loads the 32 codes
// of run g of its row (BITS words) and the 32 activations of run g of its
// token (four 16-byte loads), both straight into registers, and feeds four
// v_mfma_f32_16x16x32_bf16 whose k slots of
// lane group g hold positions 8 j .. 8 j + 7 of run g on both sides.  The
// waves' 16 x 16 sums are added through LDS in wave order.
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int GV16_WAVES = 8;

template <int BITS>
__global__ __launch_bounds__(GV16_WAVES * 64) void dequant_gemv16_kernel(DqArgs a) {
  constexpr int CB = 4;  // chunks whose loads are in flight together
  __shared__ f32x4_t red[GV16_WAVES - 1][64];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int rl = lane & 15, g = lane >> 4;
  const int64_t row0 = (int64_t)blockIdx.x * 16;
  const int64_t r = min(row0 + rl, a.m - 1);
  const int64_t t = min((int64_t)rl, a.tokens - 1);
  const int nch = (int)(a.n / 128);
  const int cw = (nch + GV16_WAVES - 1) / GV16_WAVES;
  const int c0 = wv * cw, c1 = min(nch, c0 + cw);
  const uint32_t* prow = a.P + r * a.ldp;
  const uint16_t* xrow = a.X + t * a.ldx;
  f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int cb = c0; cb < c1; cb += CB) {
    uint32_t w[CB][BITS];
    uint4 xv[CB][4];
    float sc[CB], nz[CB];
#pragma unroll
    for (int u = 0; u < CB; ++u) {
      const int c = min(cb + u, c1 - 1);  // a valid chunk; unused past c1
      const int64_t pos = 128 * (int64_t)c + 32 * g;
#pragma unroll
      for (int i = 0; i < BITS; ++i) w[u][i] = prow[(pos >> 5) * BITS + i];
#pragma unroll
      for (int i = 0; i < 4; ++i) xv[u][i] = *reinterpret_cast<const uint4*>(xrow + pos + 8 * i);
      const int64_t grp = a.G > 0 ? pos / a.G : 0;
      const float s = a.scales[r * a.ngroups + grp];
      sc[u] = s;
      nz[u] = -(a.zeros[r * a.ngroups + grp] * s);
    }
#pragma unroll
    for (int u = 0; u < CB; ++u) {
      if (cb + u < c1) {  // uniform in the workgroup
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float f[8];
          decode8<BITS>(w[u], j, f);
          uint4 bw;
          bw.x = bf16x2_bits(fmaf(f[0], sc[u], nz[u]), fmaf(f[1], sc[u], nz[u]));
          bw.y = bf16x2_bits(fmaf(f[2], sc[u], nz[u]), fmaf(f[3], sc[u], nz[u]));
          bw.z = bf16x2_bits(fmaf(f[4], sc[u], nz[u]), fmaf(f[5], sc[u], nz[u]));
          bw.w = bf16x2_bits(fmaf(f[6], sc[u], nz[u]), fmaf(f[7], sc[u], nz[u]));
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, xv[u][j]),
                                                        __builtin_bit_cast(bf16x8, bw), acc, 0, 0,
                                                        0);
        }
      }
    }
  }
  if (wv > 0) red[wv - 1][lane] = acc;
  __syncthreads();
  if (wv != 0) return;
#pragma unroll
  for (int w = 0; w < GV16_WAVES - 1; ++w) acc += red[w][lane];
  // element q of lane l: token 4 (l / 16) + q, weight row row0 + l % 16
  const int64_t row = row0 + rl;
  if (row >= a.m) return;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int64_t tok = 4 * g + q;
    if (tok < a.tokens) {
      if (a.ybf16)
        reinterpret_cast<uint16_t*>(a.Y)[tok * a.ldy + row] =
            (uint16_t)(bf16x2_bits(acc[q], 0.0f) & 0xFFFFu);
      else
        reinterpret_cast<float*>(a.Y)[tok * a.ldy + row] = acc[q];
    }
  }
}

// ---------------------------------------------------------------------------
// Decode batches (<= 32 tokens), n a multiple of 128: bound by the codes' HBM
// traffic and by how many cache lines the loads touch, so the codes never go
// through LDS.  A workgroup of 4 waves owns 128 weight rows (32 per wave) and a
// K range walked in 128-position steps.  Per step each lane loads the 64
// codes of its row that its MFMA operands need (lane group g = lane / 32 takes
// positions 64 g .. 64 g + 63: 2 adjacent 16-byte loads for 4-bit codes, one
// cache line per row) and dequantizes them in registers straight into bf16 B
// operands; the 32 x 128 X tile of the step is loaded once per workgroup
// into LDS and read back as A operands with the same position order (step j,
// lane group g: positions 64 g + 8 j .. + 8).  Loads run one step (two chunks)
// ahead; K splits across workgroups are added by dequant_reduce_kernel.
constexpr int GV_STEP = 128;          // positions per pipeline step
constexpr int GV_ROWB = GV_STEP * 2;  // bytes of one X row of a step
constexpr int GV_MAXG = 32;           // quantization groups per workgroup K range

// X tile of a step: 32 rows of 16 segments; segment s of row r at s ^ (r & 15)
__device__ __forceinline__ int gv_off(int r, int s) { return r * GV_ROWB + ((s ^ (r & 15)) << 4); }

template <int BITS>
__global__ __launch_bounds__(256) void dequant_gemv_kernel(DqArgs a) {
  __shared__ __align__(16) uint8_t xs[2][32 * GV_ROWB];
  __shared__ float zsc[GV_MAXG][128], zzp[GV_MAXG][128];  // scale, zero: [group][row]
  const int64_t b = blockIdx.x;
  const int64_t xcd = b % kXcds, idx = b / kXcds;
  const int64_t per = a.ntiles / kXcds, rem = a.ntiles % kXcds;
  if (idx >= per + (xcd < rem ? 1 : 0)) return;
  const int64_t L = xcd * per + (xcd < rem ? xcd : rem) + idx;
  const int64_t rb = L % a.nrb;
  const int64_t kspl = L / a.nrb;
  const int64_t row0 = rb * 128;
  // chunks_per_split counts 128-position steps here
  const int s_begin = (int)(kspl * a.chunks_per_split);
  const int s_end = (int)min(a.nchunks, (int64_t)s_begin + a.chunks_per_split);

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int g = lane >> 5, l32 = lane & 31;
  const int64_t rw0 = row0 + 32 * wv;  // this wave's first weight row
  const int64_t r = min(rw0 + l32, a.m - 1);
  const uint32_t* crow = a.P + r * a.ldp + g * (2 * BITS);
  // X staging: thread -> token tid / 8 (rows past the last token re-read row 0;
  // their sums are never written), segments 2 (tid % 8), + 1
  const int xt_row = tid >> 3, xt_seg = 2 * (tid & 7);
  const uint16_t* xsrc = a.X + (xt_row < a.tokens ? xt_row : 0) * a.ldx + 8 * xt_seg;
  // the group parameters of the workgroup's K range, staged once (after the
  // first steps' code loads are in flight, so the two latencies overlap)
  const int G = (int)a.G;
  const int g_first = G > 0 ? (s_begin * GV_STEP) / G : 0;
  const int g_cnt = G > 0 ? min((int)a.ngroups, (s_end * GV_STEP + G - 1) / G) - g_first : 1;
  const int wrow = 32 * wv + l32;  // this lane's row within the workgroup

  struct Ld {
    uint32_t w[2 * BITS];  // codes 64 g .. 64 g + 63 of the step
    uint4 x[2];            // this thread's share of the X tile
    int st;                // the step
  };
  auto load = [&](int st, Ld& d) {
    const uint32_t* src = crow + st * (4 * BITS);
#pragma unroll
    for (int q = 0; q < 2 * BITS; ++q) d.w[q] = src[q];
    const int k0 = st * GV_STEP;
    d.x[0] = *reinterpret_cast<const uint4*>(xsrc + k0);
    d.x[1] = *reinterpret_cast<const uint4*>(xsrc + k0 + 8);
    d.st = st;
  };
  auto stage_x = [&](const Ld& d, int buf) {
    *reinterpret_cast<uint4*>(&xs[buf][gv_off(xt_row, xt_seg)]) = d.x[0];
    *reinterpret_cast<uint4*>(&xs[buf][gv_off(xt_row, xt_seg + 1)]) = d.x[1];
  };

  f32x16 acc;
#pragma unroll
  for (int q = 0; q < 16; ++q) acc[q] = 0.0f;
  // lane group g's 64 codes are the half g of the step: half g's parameters
  auto step = [&](const Ld& d, int buf) {
    const int gi = G > 0 ? (d.st * GV_STEP + 64 * g) / G - g_first : 0;
    const float sc = zsc[gi][wrow];
    const float nzs = -(zzp[gi][wrow] * sc);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float f[8];
      uint32_t w4[BITS];
#pragma unroll
      for (int q = 0; q < BITS; ++q) w4[q] = d.w[(j >> 2) * BITS + q];
      decode8<BITS>(w4, j & 3, f);
#pragma unroll
      for (int e = 0; e < 8; ++e) f[e] = fmaf(f[e], sc, nzs);
      uint4 o;
      o.x = bf16x2_bits(f[0], f[1]);
      o.y = bf16x2_bits(f[2], f[3]);
      o.z = bf16x2_bits(f[4], f[5]);
      o.w = bf16x2_bits(f[6], f[7]);
      const bf16x8 av = *reinterpret_cast<const bf16x8*>(&xs[buf][gv_off(l32, 8 * g + j)]);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, __builtin_bit_cast(bf16x8, o), acc, 0, 0,
                                                    0);
    }
  };

  // Pipeline: step i multiplies from X buffer i % 2; then step i + 2 is loaded
  // into the registers step i has just consumed and the X of step i + 1 (loaded
  // one step ago) is staged into the other buffer, so two steps of loads are in
  // flight while a wave waits.  Loads are issued
  // unconditionally inside the loop and the last steps are peeled, so every
  // path issues a fixed sequence and the waits only cover the step in use.
  auto stage_groups = [&]() {
    for (int i = tid; i < g_cnt * 128; i += 256) {
      const int j = i >> 7, rr = i & 127;
      const int64_t rsrc = min(row0 + rr, a.m - 1);
      zsc[j][rr] = a.scales[rsrc * a.ngroups + g_first + j];
      zzp[j][rr] = a.zeros[rsrc * a.ngroups + g_first + j];
    }
  };
  const int nst = s_end - s_begin;
  Ld d0, d1;
  // (scheduling barriers keep the compiler from hoisting the next step's
  // work, and with it a wait on loads just issued, above the barrier)
  auto half = [&](Ld& cur, Ld& nxt, int buf, bool stage_next, int load_step) {
    step(cur, buf);
    __builtin_amdgcn_sched_barrier(0);
    if (load_step >= 0) load(load_step, cur);
    __builtin_amdgcn_sched_barrier(0);
    if (stage_next) stage_x(nxt, buf ^ 1);
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
  };
  if (nst == 1) {
    load(s_begin, d0);
    stage_groups();
    stage_x(d0, 0);
    __syncthreads();
    step(d0, 0);
  } else if (nst > 1) {
    load(s_begin, d0);
    load(s_begin + 1, d1);
    stage_groups();
    stage_x(d0, 0);
    __syncthreads();
    int i = 0;
    for (; i + 3 < nst; i += 2) {
      half(d0, d1, 0, true, s_begin + i + 2);
      half(d1, d0, 1, true, s_begin + i + 3);
    }
    if (nst - i == 3) {
      half(d0, d1, 0, true, s_begin + i + 2);
      half(d1, d0, 1, true, -1);
      step(d0, 0);
    } else {
      half(d0, d1, 0, true, -1);
      step(d1, 1);
    }
  }

  // lane holds weight row rw0 + (lane & 31), tokens 8 (q / 4) + 4 (lane / 32) + q % 4
  float* outf;
  int64_t ld;
  if (a.ks > 1) {
    outf = a.part + kspl * a.tokens * a.m;
    ld = a.m;
  } else {
    outf = reinterpret_cast<float*>(a.Y);
    ld = a.ldy;
  }
  const int64_t rr = rw0 + l32;
  if (rr < a.m) {
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int tt = 8 * (q >> 2) + 4 * g + (q & 3);
      if (tt >= a.tokens) continue;
      const int64_t o = tt * ld + rr;
      if (a.ks == 1 && a.ybf16) {
        reinterpret_cast<__bf16*>(a.Y)[o] = (__bf16)acc[q];
      } else {
        outf[o] = acc[q];
      }
    }
  }
}

// Decode batches of at most 16 tokens over a long K (n a multiple of 256,
// groups a multiple of 64 positions): a workgroup of 8 waves owns 128 weight
// rows (16 per wave) and a K range walked in steps of 256 positions.  The
// v_mfma_f32_16x16x32_bf16 k index is permuted inside a step so that lane
// (q = lane / 16, r = lane % 16) owns positions 64 q .. 64 q + 63 of row r:
// k-block j of the step takes positions 64 q + 8 j .. + 7 on both sides, so a
// lane's codes are 2 BITS contiguous words (16-byte loads at even widths) and
// its 64 positions lie in one group (one scale and zero a step).  Codes,
// group parameters and the lane's share of the step's X tile are loaded two
// steps ahead into registers; the 16 x 256 X tile goes through LDS with its
// 16-byte segments XOR-swizzled by token.  The codes take 16 of the 64 lanes'
// worth of each MFMA's k slots per row block, so the dequantization (decode,
// fma, round to bf16: ~21 VALU instructions per 8 codes) is the other bound
// beside the HBM stream; K splits go through dequant_reduce_kernel.
constexpr int GW_STEP = 256;  // positions per step
constexpr int GW_WAVES = 8;

template <int BITS, bool VEC16>
__global__ __launch_bounds__(GW_WAVES * 64) void dequant_gemv16w_kernel(DqArgs a) {
  constexpr int QP = GW_STEP / 4;          // positions a lane owns in a step
  constexpr int NKB = QP / 8;              // k-blocks of a step
  constexpr int WPR = QP * BITS / 32;      // code words a lane loads a step
  constexpr int ROWB = GW_STEP * 2;        // bytes of one X row of a step
  constexpr int NSEG = ROWB / 16;          // 16-byte segments of such a row
  constexpr int XU = NSEG * 16 / (64 * GW_WAVES);  // segments a thread stages
  static_assert(XU == 1 && NSEG == 32, "one X segment per thread");
  __shared__ __align__(16) uint8_t xs[2][16 * ROWB];
  const int64_t b = blockIdx.x;
  const int64_t xcd = b % kXcds, idx = b / kXcds;
  const int64_t per = a.ntiles / kXcds, rem = a.ntiles % kXcds;
  if (idx >= per + (xcd < rem ? 1 : 0)) return;
  const int64_t L = xcd * per + (xcd < rem ? xcd : rem) + idx;
  const int64_t rb = L % a.nrb;
  const int64_t kspl = L / a.nrb;
  const int s_begin = (int)(kspl * a.chunks_per_split);
  const int s_end = (int)min(a.nchunks, (int64_t)s_begin + a.chunks_per_split);
  const int nst = s_end - s_begin;  // >= 1: the host leaves no split empty
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int q = lane >> 4, r16 = lane & 15;
  const int64_t row = rb * (16 * GW_WAVES) + 16 * wv + r16;
  const int64_t rc = min(row, a.m - 1);
  const uint32_t* crow = a.P + rc * a.ldp + q * WPR;
  const float* srow = a.scales + rc * a.ngroups;
  const float* zrow = a.zeros + rc * a.ngroups;
  // X staging: thread -> token row tid / 32 (rows past the last token repeat
  // it; their sums are never written), segment tid % 32
  const int xt_row = tid >> 5, xt_seg = tid & 31;
  const uint16_t* xsrc = a.X + (xt_row < a.tokens ? xt_row : a.tokens - 1) * a.ldx + 8 * xt_seg;
  auto xoff = [](int t, int sg) { return t * ROWB + ((sg ^ t) << 4); };
  struct Ld {
    uint32_t w[WPR];
    uint4 x;
    float sc, z;
  };
  auto load = [&](int i, Ld& d) {
    const int st = s_begin + min(i, nst - 1);  // past the end: a valid step again
    const uint32_t* src = crow + (int64_t)st * (GW_STEP * BITS / 32);
    if constexpr (VEC16) {
#pragma unroll
      for (int u = 0; u < WPR / 4; ++u) {
        const uint4 v = *reinterpret_cast<const uint4*>(src + 4 * u);
        d.w[4 * u] = v.x; d.w[4 * u + 1] = v.y; d.w[4 * u + 2] = v.z; d.w[4 * u + 3] = v.w;
      }
    } else {
#pragma unroll
      for (int u = 0; u < WPR / 2; ++u) {
        const uint2 v = *reinterpret_cast<const uint2*>(src + 2 * u);
        d.w[2 * u] = v.x; d.w[2 * u + 1] = v.y;
      }
    }
    const int64_t k0 = (int64_t)st * GW_STEP;
    d.x = *reinterpret_cast<const uint4*>(xsrc + k0);
    const int64_t gi = a.G > 0 ? (k0 + QP * q) / a.G : 0;
    d.sc = srow[gi];
    d.z = zrow[gi];
  };
  auto stage_x = [&](const Ld& d, int buf) {
    *reinterpret_cast<uint4*>(&xs[buf][xoff(xt_row, xt_seg)]) = d.x;
  };
  f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
  auto step = [&](const Ld& d, int buf) {
    const float sc = d.sc, nzs = -(d.z * d.sc);
#pragma unroll
    for (int j = 0; j < NKB; ++j) {
      const bf16x8 av = *reinterpret_cast<const bf16x8*>(&xs[buf][xoff(r16, (QP * q + 8 * j) / 8)]);
      float f[8];
      uint32_t w4[BITS];
#pragma unroll
      for (int u = 0; u < BITS; ++u) w4[u] = d.w[(j >> 2) * BITS + u];
      decode8<BITS>(w4, j & 3, f);
#pragma unroll
      for (int e = 0; e < 8; ++e) f[e] = fmaf(f[e], sc, nzs);
      uint4 o;
      o.x = bf16x2_bits(f[0], f[1]);
      o.y = bf16x2_bits(f[2], f[3]);
      o.z = bf16x2_bits(f[4], f[5]);
      o.w = bf16x2_bits(f[6], f[7]);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, __builtin_bit_cast(bf16x8, o), acc, 0, 0,
                                                    0);
    }
  };
  // step i multiplies from X buffer i % 2; then step i + 2 is loaded into the
  // registers step i has consumed and the X of step i + 1 is staged into the
  // other buffer (scheduling barriers keep the next step's work, and a wait
  // on the loads just issued, below the barrier)
  Ld d0, d1;
  load(0, d0);
  load(1, d1);
  stage_x(d0, 0);
  __syncthreads();
  auto body = [&](Ld& cur, Ld& nxt, int i, int buf) {
    if (i < nst) step(cur, buf);
    __builtin_amdgcn_sched_barrier(0);
    load(i + 2, cur);
    __builtin_amdgcn_sched_barrier(0);
    if (i + 1 < nst) stage_x(nxt, buf ^ 1);
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
  };
  for (int i = 0; i < nst; i += 2) {
    body(d0, d1, i, 0);
    body(d1, d0, i + 1, 1);
  }
  // element e of lane l: token 4 (l / 16) + e, weight row r
  if (row < a.m) {
    float* outf = a.ks > 1 ? a.part + kspl * a.tokens * a.m : reinterpret_cast<float*>(a.Y);
    const int64_t ld = a.ks > 1 ? a.m : a.ldy;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int tt = 4 * q + e;
      if (tt >= a.tokens) continue;
      if (a.ks == 1 && a.ybf16) {
        reinterpret_cast<__bf16*>(a.Y)[tt * ld + row] = (__bf16)acc[e];
      } else {
        outf[tt * ld + row] = acc[e];
      }
    }
  }
}

// Y[t, r] = sum over splits s = 0, 1, ... of part[s, t, r], in that order.
// One thread per 4 consecutive outputs of a row; the loads of 8 splits are in
// flight before their in-order adds.
__global__ __launch_bounds__(256) void dequant_reduce_kernel(const float* __restrict__ part,
                                                             int64_t ks, int64_t tokens,
                                                             int64_t m, void* Y, int64_t ldy,
                                                             int ybf16) {
  const int64_t per_row = (m + 3) / 4;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= tokens * per_row) return;
  const int64_t t = i / per_row, r0 = 4 * (i - t * per_row);
  const int64_t plane = tokens * m;
  const float* src = part + t * m + r0;
  float s[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  if (r0 + 4 <= m && (m & 3) == 0) {
    int64_t k = 0;
    for (; k + 8 <= ks; k += 8) {
      float4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = *reinterpret_cast<const float4*>(src + (k + u) * plane);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        s[0] += v[u].x;
        s[1] += v[u].y;
        s[2] += v[u].z;
        s[3] += v[u].w;
      }
    }
    if (k < ks) {  // the last < 8 splits: every load issued before the in-order adds
      float4 v[7];
#pragma unroll
      for (int u = 0; u < 7; ++u)
        if (k + u < ks) v[u] = *reinterpret_cast<const float4*>(src + (k + u) * plane);
#pragma unroll
      for (int u = 0; u < 7; ++u) {
        if (k + u < ks) {
          s[0] += v[u].x;
          s[1] += v[u].y;
          s[2] += v[u].z;
          s[3] += v[u].w;
        }
      }
    }
  } else {
    for (int64_t k = 0; k < ks; ++k)
      for (int e = 0; e < 4 && r0 + e < m; ++e) s[e] += src[k * plane + e];
  }
  for (int e = 0; e < 4 && r0 + e < m; ++e) {
    if (ybf16) {
      reinterpret_cast<__bf16*>(Y)[t * ldy + r0 + e] = (__bf16)s[e];
    } else {
      reinterpret_cast<float*>(Y)[t * ldy + r0 + e] = s[e];
    }
  }
}

// Xp[t, p] = X[t, perm[p]] for p < n, 0 for n <= p < ldxp (ldxp = n rounded up
// to 8); one thread per 8-column segment, one 16-byte store.
__global__ __launch_bounds__(256) void gather_columns_kernel(const uint16_t* __restrict__ X,
                                                             int64_t ldx,
                                                             const int32_t* __restrict__ perm,
                                                             int64_t tokens, int64_t n,
                                                             int64_t ldxp,
                                                             uint16_t* __restrict__ Xp) {
  const int64_t segs = ldxp / 8;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= tokens * segs) return;
  const int64_t t = i / segs, p0 = 8 * (i - t * segs);
  const uint16_t* row = X + t * ldx;
  uint32_t w[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int64_t p = p0 + 2 * q;
    const uint32_t lo = p < n ? row[perm[p]] : 0u;
    const uint32_t hi = p + 1 < n ? row[perm[p + 1]] : 0u;
    w[q] = lo | (hi << 16);
  }
  *reinterpret_cast<uint4*>(Xp + t * ldxp + p0) = make_uint4(w[0], w[1], w[2], w[3]);
}

// The same gather with every row staged in LDS: a workgroup walks a run of
// rows; a row arrives with 16-byte loads (coalesced) straight into LDS and
// leaves permuted, 8 positions per thread and 16-byte store, the permuted
// reads served by the LDS.  One row buffer (two barriers a row), so several
// workgroups share a CU and one's loads overlap another's permute; a row is
// not prefetched into a register array (at 8 or more 16-byte entries a
// thread the compiler keeps such an array in scratch memory).  The
// permutation is read once per workgroup into registers (16-bit entries, two
// to a word), not once per row.  n and ldx multiples of 8, X 16-byte aligned,
// n <= NCAP.  Out-of-range perm entries read as zero.
template <int NCAP>
__global__ __launch_bounds__(512) void gather_rows_kernel(const uint16_t* __restrict__ X,
                                                          int64_t ldx,
                                                          const int32_t* __restrict__ perm,
                                                          int64_t tokens, int64_t n, int64_t ldxp,
                                                          int64_t rows_per_wg,
                                                          uint16_t* __restrict__ Xp) {
  constexpr int CH = NCAP / 8 / 512;  // 16-byte chunks of a row per thread
  constexpr int SEG = NCAP / 8 / 512; // output segments per thread (ldxp <= NCAP)
  static_assert(NCAP <= 65535 + 1, "16-bit permutation entries");
  __shared__ __align__(16) uint16_t buf[NCAP];
  const int tid = threadIdx.x;
  const int64_t t0 = (int64_t)blockIdx.x * rows_per_wg;
  const int64_t t1 = min(tokens, t0 + rows_per_wg);
  if (t0 >= t1) return;
  const int nch = (int)(n / 8);
  const int nseg = (int)(ldxp / 8);
  // this thread's segments tid + 512 i: source positions, 0xFFFF = zero
  uint32_t pk[SEG][4];
#pragma unroll
  for (int i = 0; i < SEG; ++i) {
    const int sg = tid + 512 * i;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      uint32_t h[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int64_t p = 8 * (int64_t)sg + 2 * q + e;
        const int32_t src = (sg < nseg && p < n) ? perm[p] : -1;
        h[e] = (src >= 0 && src < n) ? (uint32_t)src : 0xFFFFu;
      }
      pk[i][q] = h[0] | (h[1] << 16);
    }
  }
  for (int64_t t = t0; t < t1; ++t) {
    __syncthreads();  // every thread has permuted the previous row
    {
      const uint4* src = reinterpret_cast<const uint4*>(X + t * ldx);
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        const int idx = tid + 512 * c;
        if (idx < nch) reinterpret_cast<uint4*>(buf)[idx] = src[idx];
      }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < SEG; ++i) {
      const int sg = tid + 512 * i;
      if (sg < nseg) {
        uint32_t w[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t s0 = pk[i][q] & 0xFFFFu, s1 = pk[i][q] >> 16;
          const uint32_t lo = s0 != 0xFFFFu ? (uint32_t)buf[s0] : 0u;
          const uint32_t hi = s1 != 0xFFFFu ? (uint32_t)buf[s1] : 0u;
          w[q] = lo | (hi << 16);
        }
        *reinterpret_cast<uint4*>(Xp + t * ldxp + 8 * (int64_t)sg) =
            make_uint4(w[0], w[1], w[2], w[3]);
      }
    }
  }
}

struct Shape {
  int bm, bn;
  int64_t ks;
};

// Tile shape and K split for a problem.  Large batches take 256-token tiles
// (the dequantization of a weight is shared by 256 tokens); small ones shrink
// the token side and split K until the grid holds ~4 workgroups per CU.
Shape choose_shape(int64_t tokens, int64_t m, int64_t n) {
  Shape s;
  s.bm = tokens > 128 ? 256 : (tokens > 32 ? 128 : 32);
  s.bn = 128;
  const int64_t nchunks = ceil_div(n, BK);
  s.ks = 1;
  if (tokens <= 32) {
    // decode batches (the split path, 17..32 tokens or shapes the 16-token
    // kernel does not take): 128-row workgroups, K split until ~1 workgroup per
    // CU (measured at 4096 x 4096: 11.9 us at 32 tokens against 14.4 us with
    // ~2 per CU), >= 2 steps of 128 positions per split
    const int64_t tiles = ceil_div(m, 128);
    const int64_t steps = ceil_div(n, 128);
    while (tiles * s.ks * 2 <= 256 && steps / (s.ks * 2) >= 2) s.ks *= 2;
    // the group parameters of a split are staged in LDS: at most 16 steps
    // (2048 positions, 32 groups of 64) per split
    while (ceil_div(steps, s.ks) > 16) s.ks *= 2;
    return s;
  }
  const int64_t tiles = ceil_div(tokens, s.bm) * ceil_div(m, s.bn);
  // split K until the grid holds ~2 workgroups per CU (128-token tiles) or one
  // per CU (256-token tiles, one resident per CU), keeping >= 4 (8) chunks per split
  const int64_t want = tokens <= 128 ? 512 : 256;
  const int64_t min_chunks = tokens <= 128 ? 4 : 8;
  while (tiles * s.ks * 2 <= want && nchunks / (s.ks * 2) >= min_chunks) s.ks *= 2;
  return s;
}

template <int BITS, int BM, int BN, int WM, int WN>
hipError_t launch_tile(const DqArgs& a, hipStream_t stream) {
  const int64_t grid = ceil_div(a.ntiles, kXcds) * kXcds;
  constexpr int NT = (BM / WM) * (BN / WN) * 64;
  hipLaunchKernelGGL((dequant_gemm_kernel<BITS, BM, BN, WM, WN>), dim3((unsigned)grid),
                     dim3(NT), 0, stream, a);
  return hipGetLastError();
}

template <int BITS>
hipError_t launch_dma(const DqArgs& a, int tm, hipStream_t stream) {
  const int64_t grid = ceil_div(a.ntiles, kXcds) * kXcds;
  switch (tm) {
    case 256:
      hipLaunchKernelGGL((dequant_gemm_dma_kernel<BITS, 256>), dim3((unsigned)grid), dim3(256), 0,
                         stream, a);
      break;
    case 128:
      hipLaunchKernelGGL((dequant_gemm_dma_kernel<BITS, 128>), dim3((unsigned)grid), dim3(256), 0,
                         stream, a);
      break;
    default:
      hipLaunchKernelGGL((dequant_gemm_dma_kernel<BITS, 32>), dim3((unsigned)grid), dim3(256), 0,
                         stream, a);
  }
  return hipGetLastError();
}

template <int BITS>
hipError_t launch_bits(const DqArgs& a, int bm, hipStream_t stream) {
  switch (bm) {
    case 256: return launch_tile<BITS, 256, 128, 64, 64>(a, stream);
    case 128: return launch_tile<BITS, 128, 128, 64, 64>(a, stream);
    default: return launch_tile<BITS, 32, 128, 32, 32>(a, stream);
  }
}

}  // namespace

void launch_gather(const uint16_t* X, int64_t ldx, const int32_t* perm, int64_t tokens,
                   int64_t n, int64_t ldxp, uint16_t* Xp, hipStream_t stream) {
  if (tokens <= 0) return;
  // (ldxp bounds the output segments a thread holds positions for).  Rows
  // staged in LDS pay for reading the permutation once per workgroup over its
  // rows; below 64 tokens (decode batches) the per-element gather spreads the
  // few rows over many workgroups instead (16 x 28672: 35 us staged in 4
  // workgroups)
  const bool rows = tokens >= 64 && n % 8 == 0 && ldx % 8 == 0 &&
                    (reinterpret_cast<uintptr_t>(X) & 15) == 0 && ldxp <= 32768;
  if (rows) {
    // about 1024 workgroups, at least 4 rows each
    const int64_t rpw = hmax((int64_t)4, ceil_div(tokens, (int64_t)1024));
    const dim3 grid((unsigned)ceil_div(tokens, rpw));
    if (ldxp <= 16384)
      hipLaunchKernelGGL(gather_rows_kernel<16384>, grid, dim3(512), 0, stream, X, ldx, perm,
                         tokens, n, ldxp, rpw, Xp);
    else
      hipLaunchKernelGGL(gather_rows_kernel<32768>, grid, dim3(512), 0, stream, X, ldx, perm,
                         tokens, n, ldxp, rpw, Xp);
  } else {
    const int64_t total = tokens * (ldxp / 8);
    hipLaunchKernelGGL(gather_columns_kernel, dim3((unsigned)ceil_div(total, 256)), dim3(256), 0,
                       stream, X, ldx, perm, tokens, n, ldxp, Xp);
  }
}

// Batches of at least this many tokens, whose 256 x 256 output tiles fill the
// GPU, dequantize the weights once into the workspace (bf16, the same weights
// the fused kernels form) and multiply them with the dense kernel: at 2048
// tokens on 8192 x 28672 the dense product runs at ~1.25 PFLOP/s against ~0.75
// for the fused one, which pays back the weights' extra 2 bytes written and
// read.  Fewer tiles leave CUs idle (the fused kernel splits K instead).
constexpr int64_t DENSE_PATH_TOKENS = 1024;

static bool dense_path(int64_t tokens, int64_t m, int64_t n) {
  return tokens >= DENSE_PATH_TOKENS && n % 8 == 0 &&
         ceil_div(tokens, (int64_t)256) * ceil_div(m, (int64_t)256) >= 256;
}

size_t dequant_gemm_ws_bytes(int64_t tokens, int64_t m, int64_t n, int has_perm) {
  const Shape s = choose_shape(tokens, m, n);
  size_t bytes = 0;
  if (has_perm) bytes += align_up((size_t)tokens * (size_t)align_up((size_t)n, 8) * 2, 256);
  if (dense_path(tokens, m, n)) return bytes + align_up((size_t)m * (size_t)n * 2, 256);
  if (s.ks > 1) bytes += (size_t)s.ks * (size_t)tokens * (size_t)m * 4;
  return bytes;
}

hipError_t launch_dequant_gemm(const DequantArgs& d, hipStream_t stream) {
  const Shape s = choose_shape(d.tokens, d.m, d.n);
  DqArgs a;
  uint8_t* ws = static_cast<uint8_t*>(d.ws);
  a.X = static_cast<const uint16_t*>(d.X);
  a.ldx = d.ldx;
  if (d.perm) {
    const int64_t ldxp = (int64_t)align_up((size_t)d.n, 8);
    uint16_t* Xp = reinterpret_cast<uint16_t*>(ws);
    ws += align_up((size_t)d.tokens * (size_t)ldxp * 2, 256);
    launch_gather(a.X, d.ldx, d.perm, d.tokens, d.n, ldxp, Xp, stream);
    a.X = Xp;
    a.ldx = ldxp;
  }
  if (dense_path(d.tokens, d.m, d.n) && a.ldx < (int64_t(1) << 23) && d.n < (int64_t(1) << 23)) {
    uint16_t* Wd = reinterpret_cast<uint16_t*>(ws);  // [m, n] bf16, row stride n
    hipError_t e = launch_dequantize(d.packed, d.ldp, d.bits, d.m, d.n, d.scales, d.zeros,
                                     d.group_size, Wd, d.n, stream);
    if (e != hipSuccess) return e;
    return launch_dense_gemm(a.X, a.ldx, d.tokens, d.n, Wd, d.n, d.m, d.Y, d.ldy,
                             d.ydt == GPTQ_BF16 ? 1 : 0, stream);
  }
  a.tokens = d.tokens;
  a.n = d.n;
  a.P = d.packed;
  a.ldp = d.ldp;
  a.nwr = ceil_div(d.n * d.bits, 32);
  a.scales = d.scales;
  a.zeros = d.zeros;
  a.G = d.group_size > 0 ? d.group_size : 0;
  a.ngroups = d.group_size > 0 ? ceil_div(d.n, d.group_size) : 1;
  a.gs_run = (d.group_size <= 0 || d.group_size % 32 == 0) ? 1 : 0;
  a.gshift = -1;
  if (d.group_size > 0 && (d.group_size & (d.group_size - 1)) == 0) {
    a.gshift = 0;
    while ((1 << a.gshift) < d.group_size) ++a.gshift;
  }
  a.m = d.m;
  a.Y = d.Y;
  a.ldy = d.ldy;
  a.ybf16 = d.ydt == GPTQ_BF16 ? 1 : 0;
  a.part = s.ks > 1 ? reinterpret_cast<float*>(ws) : nullptr;
  a.ntb = ceil_div(d.tokens, s.bm);
  a.nrb = ceil_div(d.m, s.bn);
  a.ks = s.ks;
  a.nchunks = ceil_div(d.n, BK);
  a.chunks_per_split = ceil_div(a.nchunks, s.ks);
  a.ntiles = a.ntb * a.nrb * a.ks;
  // the DMA kernel: 16-byte X rows (n % 8 == 0, aligned), one group per row and
  // chunk, codes of <= 6 bits (LDS budget), 32-bit offsets
  const bool dma = d.n % 8 == 0 && d.bits <= 6 &&
                   (d.group_size <= 0 || d.group_size % 64 == 0) && a.ldx % 8 == 0 &&
                   (reinterpret_cast<uintptr_t>(a.X) & 15) == 0 && a.ldx < (int64_t(1) << 23) &&
                   d.ldp < (int64_t(1) << 23);
  hipError_t e;
  // up to 16 tokens and n <= 8192: the single-kernel path (whole K per
  // workgroup).  Each workgroup of 16 rows reads all of X from the L2, which
  // at large n costs more than the split path's partial sums (at 8192 x
  // 28672, 16 tokens: the split path reads X once per 128-row block)
  const bool gv16 = dma && d.tokens <= 16 && d.n % 128 == 0 && d.n <= 8192 &&
                    (d.group_size <= 0 || d.group_size % 32 == 0);
  // up to 16 tokens over a longer K: 128-row workgroups, K split over ~256
  // workgroups (at 8192 x 28672, 16 tokens, 4 bits: 38 us against 66 us for
  // the 32 x 32 split kernel below; more splits, more waves per SIMD, were not
  // faster, the dequantization's VALU work being the other bound)
  const bool even = d.bits % 2 == 0;
  const bool w16 = dma && d.tokens <= 16 && d.n > 8192 && d.n % GW_STEP == 0 &&
                   (d.group_size <= 0 || d.group_size % 64 == 0) &&
                   (reinterpret_cast<uintptr_t>(d.packed) & (even ? 15 : 7)) == 0 &&
                   d.ldp % (even ? 4 : 2) == 0;
  if (w16) {
    const int64_t steps = d.n / GW_STEP;
    a.nrb = ceil_div(d.m, (int64_t)(16 * GW_WAVES));
    int64_t ks = hmin(hmax((int64_t)1, ceil_div((int64_t)256, a.nrb)), hmin(s.ks, steps));
    a.chunks_per_split = ceil_div(steps, ks);
    ks = ceil_div(steps, a.chunks_per_split);  // no empty split
    a.ks = ks;
    a.nchunks = steps;
    a.ntiles = a.nrb * ks;
    a.part = ks > 1 ? reinterpret_cast<float*>(ws) : nullptr;
    const int64_t grid = ceil_div(a.ntiles, kXcds) * kXcds;
    const dim3 g3((unsigned)grid), b3(GW_WAVES * 64);
    switch (d.bits) {
      case 2: hipLaunchKernelGGL((dequant_gemv16w_kernel<2, true>), g3, b3, 0, stream, a); break;
      case 3: hipLaunchKernelGGL((dequant_gemv16w_kernel<3, false>), g3, b3, 0, stream, a); break;
      case 4: hipLaunchKernelGGL((dequant_gemv16w_kernel<4, true>), g3, b3, 0, stream, a); break;
      case 5: hipLaunchKernelGGL((dequant_gemv16w_kernel<5, false>), g3, b3, 0, stream, a); break;
      default: hipLaunchKernelGGL((dequant_gemv16w_kernel<6, true>), g3, b3, 0, stream, a);
    }
    e = hipGetLastError();
    if (e != hipSuccess || ks == 1) return e;
    const int64_t total = d.tokens * ceil_div(d.m, 4);
    hipLaunchKernelGGL(dequant_reduce_kernel, dim3((unsigned)ceil_div(total, 256)), dim3(256), 0,
                       stream, a.part, ks, d.tokens, d.m, d.Y, d.ldy, a.ybf16);
    return hipGetLastError();
  }
  if (gv16) {
    const dim3 grid((unsigned)ceil_div(d.m, 16));
    switch (d.bits) {
      case 2: hipLaunchKernelGGL(dequant_gemv16_kernel<2>, grid, dim3(GV16_WAVES * 64), 0, stream, a); break;
      case 3: hipLaunchKernelGGL(dequant_gemv16_kernel<3>, grid, dim3(GV16_WAVES * 64), 0, stream, a); break;
      case 4: hipLaunchKernelGGL(dequant_gemv16_kernel<4>, grid, dim3(GV16_WAVES * 64), 0, stream, a); break;
      case 5: hipLaunchKernelGGL(dequant_gemv16_kernel<5>, grid, dim3(GV16_WAVES * 64), 0, stream, a); break;
      default: hipLaunchKernelGGL(dequant_gemv16_kernel<6>, grid, dim3(GV16_WAVES * 64), 0, stream, a);
    }
    return hipGetLastError();
  }
  const int64_t gv_steps = d.n / GV_STEP;
  const int64_t gv_per_split = ceil_div(gv_steps, s.ks);
  const bool gv = dma && s.bm == 32 && d.n % GV_STEP == 0 &&
                  (d.group_size <= 0 || ceil_div(gv_per_split * GV_STEP, d.group_size) + 1 <= GV_MAXG);
  if (gv) {
    a.nrb = ceil_div(d.m, 128);
    a.nchunks = gv_steps;
    a.chunks_per_split = gv_per_split;
    a.ntiles = a.nrb * a.ks;
    const int64_t grid = ceil_div(a.ntiles, kXcds) * kXcds;
    switch (d.bits) {
      case 2:
        hipLaunchKernelGGL(dequant_gemv_kernel<2>, dim3((unsigned)grid), dim3(256), 0, stream, a);
        break;
      case 3:
        hipLaunchKernelGGL(dequant_gemv_kernel<3>, dim3((unsigned)grid), dim3(256), 0, stream, a);
        break;
      case 4:
        hipLaunchKernelGGL(dequant_gemv_kernel<4>, dim3((unsigned)grid), dim3(256), 0, stream, a);
        break;
      case 5:
        hipLaunchKernelGGL(dequant_gemv_kernel<5>, dim3((unsigned)grid), dim3(256), 0, stream, a);
        break;
      default:
        hipLaunchKernelGGL(dequant_gemv_kernel<6>, dim3((unsigned)grid), dim3(256), 0, stream, a);
    }
    e = hipGetLastError();
  } else if (dma) {
    switch (d.bits) {
      case 2: e = launch_dma<2>(a, s.bm, stream); break;
      case 3: e = launch_dma<3>(a, s.bm, stream); break;
      case 4: e = launch_dma<4>(a, s.bm, stream); break;
      case 5: e = launch_dma<5>(a, s.bm, stream); break;
      default: e = launch_dma<6>(a, s.bm, stream); break;
    }
  } else {
    switch (d.bits) {
      case 2: e = launch_bits<2>(a, s.bm, stream); break;
      case 3: e = launch_bits<3>(a, s.bm, stream); break;
      case 4: e = launch_bits<4>(a, s.bm, stream); break;
      case 5: e = launch_bits<5>(a, s.bm, stream); break;
      case 6: e = launch_bits<6>(a, s.bm, stream); break;
      case 7: e = launch_bits<7>(a, s.bm, stream); break;
      default: e = launch_bits<8>(a, s.bm, stream); break;
    }
  }
  if (e != hipSuccess || s.ks == 1) return e;
  const int64_t total = d.tokens * ceil_div(d.m, 4);
  hipLaunchKernelGGL(dequant_reduce_kernel, dim3((unsigned)ceil_div(total, 256)), dim3(256), 0,
                     stream, a.part, s.ks, d.tokens, d.m, d.Y, d.ldy, a.ybf16);
  return hipGetLastError();
}

hipError_t launch_dense_gemm(const uint16_t* X, int64_t ldx, int64_t tokens, int64_t n,
                             const uint16_t* W, int64_t ldw, int64_t m, void* Y, int64_t ldy,
                             int ybf16, hipStream_t stream) {
  DenseArgs a;
  a.X = X; a.ldx = ldx; a.tokens = tokens; a.n = n;
  a.W = W; a.ldw = ldw; a.m = m;
  a.Y = Y; a.ldy = ldy; a.ybf16 = ybf16;
  a.nrb = ceil_div(m, DD_TN);
  a.ntiles = ceil_div(tokens, DD_TM) * a.nrb;
  a.nchunks = ceil_div(n, BK);
  const int64_t grid = ceil_div(a.ntiles, kXcds) * kXcds;
  hipLaunchKernelGGL(dense_gemm16_kernel, dim3((unsigned)grid), dim3(1024), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_dequantize(const uint32_t* P, int64_t ldp, int bits, int64_t m, int64_t n,
                             const float* scales, const float* zeros, int64_t group_size,
                             uint16_t* W, int64_t ldw, hipStream_t stream) {
  const int64_t G = group_size > 0 ? group_size : 0;
  const int64_t ngroups = G > 0 ? ceil_div(n, G) : 1;
  const dim3 grid((unsigned)ceil_div(n / 8, (int64_t)256), (unsigned)hmin(m, (int64_t)65535));
#define GPTQ_DQ(B)                                                                            \
  hipLaunchKernelGGL(dequantize_kernel<B>, grid, dim3(64), 0, stream, P, ldp, m, n, scales,  \
                     zeros, G, ngroups, W, ldw)
  switch (bits) {
    case 2: GPTQ_DQ(2); break;
    case 3: GPTQ_DQ(3); break;
    case 4: GPTQ_DQ(4); break;
    case 5: GPTQ_DQ(5); break;
    case 6: GPTQ_DQ(6); break;
    case 7: GPTQ_DQ(7); break;
    default: GPTQ_DQ(8); break;
  }
#undef GPTQ_DQ
  return hipGetLastError();
}

}  // namespace gptq
